// fwd_f16.hip -- tree-attention forward for fp16 K/V on the matrix cores.
//
// "tree_attention.metal" (mlx-native 0.9.1), tree_attention_impl computes,
// per (query, head), an online softmax over KV chunks with an explicit mask
// and GQA, and writes split-KV partials.  Every query row that shares a kv
// head -- q_l nodes x (n_heads / n_kv_heads) heads -- reads the same K/V, so
// here one workgroup takes 64 such rows and turns Q.K^T and P.V into dense
// tiles for v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation):
//
//   S^T[key][row] = K[key][:] . Q'[row][:]     A = K (LDS), B = Q'^T (VGPRs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  A = V^T (LDS), B = P^T (VGPRs)
//
// With this orientation every lane owns one query row in both the score and
// the output accumulators, so the softmax state (M, S) and the rescale factor
// stay in the lane.  Q' = Q * scale * log2(e) is rounded to fp16 once; logits
// are kept in base-2 units and exponentiated with exp2.
//
// Workgroup = 4 wavefronts x 16 rows.  K/V tiles of BN keys are prefetched
// into registers one tile ahead and written to a double-buffered LDS: K as
// rows, V transposed so that the PV A-operand is one 16-byte LDS read.  One
// barrier per tile.  A tile whose mask cells are all <= -65504 for every row
// of the workgroup is skipped ("tree_attention.metal" skips fully masked
// chunks).
#include "common.h"

namespace ta {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 16;

template <int D> struct F16Shape {
  static constexpr int BN = (D == 128) ? 64 : 32;  // keys per tile
  static constexpr int KSTR = D + 8;                // K row stride (halfs)
  static constexpr int VSTR = BN + 8;               // V^T row stride (halfs)
  static constexpr int KB = BN / 16;                // 16-key score blocks
  static constexpr int KS = BN / 32;                // 32-key PV steps
  static constexpr int DS = D / 32;                 // QK steps over d
  static constexpr int DB = D / 16;                 // PV output blocks over d
  static constexpr int KCH = BN * D / 8 / kThreads; // K 16-byte chunks/thread
  static constexpr int VBLK = BN * D / 32 / kThreads; // V 4x8 blocks/thread
  static constexpr size_t LDS = 2 * (size_t)(BN * KSTR + D * VSTR) * sizeof(half_t);
  static constexpr int MIN_WAVES = (D >= 512) ? 1 : 2;
  static_assert(KCH >= 1 && VBLK >= 1, "tile too small for the workgroup");
};

// Position of key (4*b4 .. 4*b4+3) of a tile in the transposed V^T row.  The
// score accumulator of a lane in group gp holds keys 4gp..4gp+3 of each
// 16-key block; the PV B-operand of that lane takes, per 32-key step, those
// keys of both blocks, so the V^T row stores them side by side:
// [0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31] per 32 keys.
__device__ inline uint32_t vt_pos(uint32_t b4) {
  uint32_t step = b4 >> 3, bb = b4 & 7u;
  return 32u * step + (bb < 4u ? 8u * bb : 8u * (bb - 4u) + 4u);
}

template <bool IMPLICIT, bool VEC_MASK, int KB>
struct MaskTile {
  float m[KB][4];
};

template <int D, bool IMPLICIT, bool VEC_MASK>
__global__ __launch_bounds__(kThreads, F16Shape<D>::MIN_WAVES)
void fwd_f16_kernel(FwdArgs a) {
  using S = F16Shape<D>;
  constexpr int BN = S::BN, KB = S::KB, KS = S::KS, DS = S::DS, DB = S::DB;
  extern __shared__ __attribute__((aligned(16))) half_t lds_h[];
  half_t *Ks0 = lds_h;                       // [2][BN][KSTR]
  half_t *Vt0 = lds_h + 2 * BN * S::KSTR;    // [2][D][VSTR]

  uint32_t unit, rt;
  decode_block(blockIdx.x, a.row_tiles, unit, rt);
  if (unit >= a.units) return;
  const uint32_t hk = unit / a.nwg;
  const uint32_t split = unit % a.nwg;
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid / kWave;
  const uint32_t lane = tid % kWave;
  const uint32_t n = lane & 15u;   // the lane's query row within the wave
  const uint32_t gp = lane >> 4;   // lane group (k / key sub-block)

  const uint32_t gr = rt * (kThreads / kWave) * kRowsPerWave + wave * kRowsPerWave + n;
  const bool valid = gr < a.rows;
  const uint32_t node = valid ? gr / a.group : 0u;
  const uint32_t head = hk * a.group + (valid ? gr % a.group : 0u);

  // ---- Q'^T fragments: row n, d = 32*ds + 8*gp + 0..7 ----
  half8_t qf[DS];
  {
    const float *qrow = a.q + ((size_t)head * a.q_l + node) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      floatx4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (valid) {
        x0 = *reinterpret_cast<const floatx4 *>(qrow + 32 * ds + 8 * gp);
        x1 = *reinterpret_cast<const floatx4 *>(qrow + 32 * ds + 8 * gp + 4);
      }
      x0 *= a.qscale;
      x1 *= a.qscale;
      qf[ds] = half8_t{(half_t)x0[0], (half_t)x0[1], (half_t)x0[2], (half_t)x0[3],
                       (half_t)x1[0], (half_t)x1[1], (half_t)x1[2], (half_t)x1[3]};
    }
  }

  const size_t kvbase = (size_t)hk * a.kv_capacity * D;
  const half_t *K = static_cast<const half_t *>(a.k) + kvbase;
  const half_t *V = static_cast<const half_t *>(a.v) + kvbase;
  const float *mrow = IMPLICIT ? nullptr : a.mask + (size_t)node * a.mask_stride;
  const int64_t causal_last = (int64_t)a.kv_seq_len - (int64_t)a.q_l + (int64_t)node;

  // Mask cells of the lane's row for keys 16kb + 4gp + j of tile t.
  auto fetch_mask = [&](uint32_t t, float (&m)[KB][4]) {
    const uint32_t key0 = t * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t kk = key0 + 16u * kb + 4u * gp;
      if (IMPLICIT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t key = kk + j;
          bool in = valid && key < a.kv_seq_len && (int64_t)key <= causal_last;
          m[kb][j] = in ? 0.0f : kMasked;
        }
      } else if (VEC_MASK && valid && kk + 3u < a.kv_seq_len) {
        floatx4 x = *reinterpret_cast<const floatx4 *>(mrow + kk);
        m[kb][0] = x[0]; m[kb][1] = x[1]; m[kb][2] = x[2]; m[kb][3] = x[3];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t key = kk + j;
          m[kb][j] = (valid && key < a.kv_seq_len) ? mrow[key] : kMasked;
        }
      }
    }
  };
  auto lane_live = [&](const float (&m)[KB][4]) {
    int live = 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) live |= (m[kb][j] > kMasked);
    return live;
  };

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[S::KCH];
  u32x4 vreg[S::VBLK][4];
  auto load_kv = [&](uint32_t t) {
    const uint32_t key0 = t * BN;
#pragma unroll
    for (int u = 0; u < S::KCH; ++u) {
      uint32_t c = tid + kThreads * u;
      uint32_t key = c / (D / 8), col8 = c % (D / 8);
      uint32_t gk = key0 + key;
      kreg[u] = (gk < a.kv_seq_len)
                    ? *reinterpret_cast<const u32x4 *>(K + (size_t)gk * D + 8 * col8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < S::VBLK; ++u) {
      uint32_t b = tid + kThreads * u;
      uint32_t col8 = b % (D / 8), b4 = b / (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t gk = key0 + 4 * b4 + j;
        vreg[u][j] = (gk < a.kv_seq_len)
                         ? *reinterpret_cast<const u32x4 *>(V + (size_t)gk * D + 8 * col8)
                         : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_kv = [&](uint32_t buf) {
    half_t *Ks = Ks0 + buf * BN * S::KSTR;
    half_t *Vt = Vt0 + buf * D * S::VSTR;
#pragma unroll
    for (int u = 0; u < S::KCH; ++u) {
      uint32_t c = tid + kThreads * u;
      uint32_t key = c / (D / 8), col8 = c % (D / 8);
      *reinterpret_cast<u32x4 *>(Ks + key * S::KSTR + 8 * col8) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < S::VBLK; ++u) {
      uint32_t b = tid + kThreads * u;
      uint32_t col8 = b % (D / 8), b4 = b / (D / 8);
      uint32_t pos = vt_pos(b4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // 32-bit word e of each key row holds dims 2e (low) and 2e+1 (high).
        uint32_t w0 = vreg[u][0][e], w1 = vreg[u][1][e];
        uint32_t w2 = vreg[u][2][e], w3 = vreg[u][3][e];
        u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(Vt + (8 * col8 + 2 * e) * S::VSTR + pos) = lo;
        *reinterpret_cast<u32x2 *>(Vt + (8 * col8 + 2 * e + 1) * S::VSTR + pos) = hi;
      }
    }
  };

  // ---- online-softmax state of the lane's row ----
  float Mrow = -INFINITY;  // running max, base-2 units
  float Srow = 0.0f;       // running sum of this lane's keys
  floatx4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](uint32_t buf, const float (&m)[KB][4]) {
    const half_t *Ks = Ks0 + buf * BN * S::KSTR;
    const half_t *Vt = Vt0 + buf * D * S::VSTR;
    floatx4 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        half8_t kf = *reinterpret_cast<const half8_t *>(
            Ks + (16 * kb + n) * S::KSTR + 32 * ds + 8 * gp);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ds], sacc[kb], 0, 0, 0);
      }
    }
    // logits in base 2; masked cells drop out
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s = (m[kb][j] > kMasked) ? fmaf(m[kb][j], kLog2e, sacc[kb][j]) : -INFINITY;
        sacc[kb][j] = s;
        tmax = fmaxf(tmax, s);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(Mrow, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(Mrow - m_use);
    float psum = 0.0f;
    half8_t pf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sacc[2 * ks][j] - m_use);
        p[4 + j] = __builtin_amdgcn_exp2f(sacc[2 * ks + 1][j] - m_use);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) psum += p[j];
      pf[ks] = half8_t{(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3],
                       (half_t)p[4], (half_t)p[5], (half_t)p[6], (half_t)p[7]};
    }
    Srow = Srow * alpha + psum;
    Mrow = m_new;
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        half8_t vf = *reinterpret_cast<const half8_t *>(
            Vt + (16 * db + n) * S::VSTR + 32 * ks + 8 * gp);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[ks], oacc[db], 0, 0, 0);
      }
    }
  };

  // ---- main loop: prefetch tile t+1 while tile t is on the matrix cores ----
  uint32_t t0, t1;
  split_range(a.n_tiles, a.nwg, split, t0, t1);
  float m_cur[KB][4], m_nxt[KB][4];
  int live_cur = 0;
  if (t0 < t1) {
    load_kv(t0);
    fetch_mask(t0, m_cur);
    store_kv(0);
    live_cur = __syncthreads_or(lane_live(m_cur));
  }
  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t buf = (t - t0) & 1u;
    const bool has_next = t + 1 < t1;
    if (has_next) {
      load_kv(t + 1);
      fetch_mask(t + 1, m_nxt);
    }
    if (live_cur) compute(buf, m_cur);
    if (has_next) store_kv(buf ^ 1u);
    int live_nxt = __syncthreads_or(has_next ? lane_live(m_nxt) : 0);
    if (has_next) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) m_cur[kb][j] = m_nxt[kb][j];
    }
    live_cur = live_nxt;
  }

  // ---- results ----
  float stot = Srow + __shfl_xor(Srow, 16);
  stot += __shfl_xor(stot, 32);
  if (!valid) return;
  const size_t rid = (size_t)node * a.n_heads + head;
  if (a.nwg == 1) {
    const float inv = (stot > 0.0f) ? 1.0f / stot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<floatx4 *>(a.out + rid * D + 16 * db + 4 * gp) = oacc[db] * inv;
  } else {
    const size_t nrows = (size_t)a.n_heads * a.q_l;
    const size_t prow = (size_t)split * nrows + rid;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<floatx4 *>(a.part_o + prow * D + 16 * db + 4 * gp) = oacc[db];
    if (gp == 0) {
      a.part_sm[prow * 2 + 0] = stot;
      a.part_sm[prow * 2 + 1] = Mrow;
    }
  }
}

template <int D, bool IMPLICIT, bool VEC>
hipError_t launch_f16_v(const FwdArgs &a, hipStream_t s) {
  constexpr size_t lds = F16Shape<D>::LDS;
  static const bool attr_set = [] {
    (void)hipFuncSetAttribute((const void *)fwd_f16_kernel<D, IMPLICIT, VEC>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)attr_set;
  dim3 grid(grid_size(a.units, a.row_tiles));
  hipLaunchKernelGGL((fwd_f16_kernel<D, IMPLICIT, VEC>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f16_d(const FwdArgs &a, hipStream_t s) {
  if (a.mask == nullptr) return launch_f16_v<D, true, false>(a, s);
  bool vec = ((uintptr_t)a.mask % 16u == 0) && (a.mask_stride % 4u == 0);
  if (vec) return launch_f16_v<D, false, true>(a, s);
  return launch_f16_v<D, false, false>(a, s);
}

}  // namespace

uint32_t f16_tile_keys(uint32_t head_dim) { return head_dim == 128 ? 64u : 32u; }

hipError_t launch_forward_f16(const FwdArgs &a, uint32_t head_dim,
                              hipStream_t s) {
  switch (head_dim) {
    case 128: return launch_f16_d<128>(a, s);
    case 256: return launch_f16_d<256>(a, s);
    case 512: return launch_f16_d<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
