// fwd_f16.hip -- tree-attention forward for fp16 K/V on the matrix cores.
//
// "tree_attention.metal" (mlx-native 0.9.1), tree_attention_impl computes,
// per (query, head), an online softmax over KV chunks with an explicit mask
// and GQA, and writes split-KV partials.  Every query row that shares a kv
// head -- q_l nodes x (n_heads / n_kv_heads) heads -- reads the same K/V, so
// here one workgroup takes up to 192 such rows and turns Q.K^T and P.V into
// dense tiles for v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation):
//
//   S^T[key][row] = K[key][:] . Q'[row][:]       A = K   (LDS), B = Q'^T (VGPRs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  A = V^T (LDS), B = P^T (VGPRs)
//
// With this orientation every lane owns one query row in both the score and
// the output accumulators, so the softmax state (M, S) and the rescale factor
// stay in the lane.  Q' = Q * scale * log2(e) is rounded to fp16 once; logits
// are kept in base-2 units and exponentiated with exp2.
//
// Workgroup = 4 wavefronts; each wavefront owns RB blocks of 16 rows and
// feeds every K/V operand it reads from LDS to RB matrix instructions, which
// keeps LDS traffic below the matrix-core rate (LDS delivers ~128 B/clk/CU;
// one 16x16x32 instruction consumes 1 KB of A operand for 16 kflop).
//
// K/V tiles of 32 keys move global -> registers during the previous tile's
// arithmetic and registers -> LDS after it (double-buffered LDS, one barrier
// per tile).  K and V are both stored row-major with a 16-byte-chunk XOR swizzle
// (chunk c of row r lives at c ^ (r & 15)), which makes every operand read
// bank-conflict free; V^T operands come from ds_read_b64_tr_b16, which
// transposes 4x16 blocks of 16-bit values on the way out of LDS.
//
// The explicit mask tile of the workgroup's tree nodes is staged in LDS with
// the K/V tile.  A wavefront whose rows have every cell of a tile at or below
// -65504 skips that tile's arithmetic ("tree_attention.metal" skips fully
// masked chunks); the tile's K/V is still fetched for the other wavefronts.
#include "common.h"

namespace ta {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BN = 32;   // keys per tile
constexpr int MST = BN + 4;  // mask tile row stride (floats)
// Lazy-rescale threshold of the running max, in base-2 logit units.
constexpr float kLazy = 8.0f;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

template <int D, int RB, int MROWS = 64 * RB> struct F16Shape {
  static constexpr int RPW = kWaves * 16 * RB;           // rows per workgroup
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int KB = BN / 16;                     // 16-key score blocks
  static constexpr int DS = D / 32;                      // QK steps over d
  static constexpr int DB = D / 16;                      // PV output blocks over d
  static constexpr int KVCH = BN * CH / kThreads;        // K (and V) chunks per thread
  static constexpr int MCH = (MROWS * (BN / 4) + kThreads - 1) / kThreads;  // mask float4/thread
  static constexpr size_t KV_LDS = 2 * 2 * (size_t)BN * D * sizeof(half_t);
  static_assert(KVCH >= 1, "tile too small for the workgroup");
};

__device__ inline uint32_t swz(uint32_t row, uint32_t chunk) { return chunk ^ (row & 15u); }

// MROWS: tree nodes the workgroup's mask tile can hold (64, or every row).
template <int D, int RB, int MROWS, bool IMPLICIT, bool VEC_MASK>
__global__ __launch_bounds__(kThreads, 1) void fwd_f16_kernel(FwdArgs a) {
  using S = F16Shape<D, RB, MROWS>;
  constexpr int KB = S::KB, DS = S::DS, DB = S::DB, KVCH = S::KVCH, MCH = S::MCH;
  extern __shared__ __attribute__((aligned(16))) half_t lds_h[];
  half_t *Ks0 = lds_h;                        // [2][BN][D] swizzled
  half_t *Vs0 = lds_h + 2 * BN * D;           // [2][BN][D] swizzled
  float *Ms0 = reinterpret_cast<float *>(lds_h + 4 * BN * D);  // [2][nodes][MST]

  uint32_t unit, rt;
  decode_block(blockIdx.x, a.row_tiles, unit, rt);
  if (unit >= a.units) return;
  const uint32_t hk = unit / a.nwg;
  const uint32_t split = unit % a.nwg;
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid / kWave;
  const uint32_t lane = tid % kWave;
  const uint32_t n = lane & 15u;   // the lane's query row within a 16-row block
  const uint32_t gp = lane >> 4;   // lane group

  const uint32_t row0 = rt * S::RPW;
  const uint32_t node0 = row0 / a.group;
  const uint32_t last_row = min(row0 + S::RPW, a.rows) - 1u;
  const uint32_t nnodes = last_row / a.group - node0 + 1u;   // nodes of this workgroup

  // ---- the lane's rows and their Q'^T fragments: row n, d = 32ds + 8gp + 0..7 ----
  uint32_t node[RB];
  bool valid[RB];
  half8_t qf[RB][DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t gr = row0 + wave * 16u * RB + 16u * rb + n;
    valid[rb] = gr < a.rows;
    node[rb] = valid[rb] ? gr / a.group : node0;
    const uint32_t head = hk * a.group + (valid[rb] ? gr % a.group : 0u);
    const float *qrow = a.q + ((size_t)head * a.q_l + node[rb]) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      floatx4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (valid[rb]) {
        x0 = *reinterpret_cast<const floatx4 *>(qrow + 32 * ds + 8 * gp);
        x1 = *reinterpret_cast<const floatx4 *>(qrow + 32 * ds + 8 * gp + 4);
      }
      x0 *= a.qscale;
      x1 *= a.qscale;
      qf[rb][ds] = half8_t{(half_t)x0[0], (half_t)x0[1], (half_t)x0[2], (half_t)x0[3],
                           (half_t)x1[0], (half_t)x1[1], (half_t)x1[2], (half_t)x1[3]};
    }
  }

  const size_t kvbase = (size_t)hk * a.kv_capacity * D;
  const half_t *K = static_cast<const half_t *>(a.k) + kvbase;
  const half_t *V = static_cast<const half_t *>(a.v) + kvbase;
  const uint32_t L = a.kv_seq_len;

  // ---- global -> register staging of one tile (K, V and the mask tile) ----
  struct Stage {
    u32x4 k[KVCH], v[KVCH];
    floatx4 m[IMPLICIT ? 1 : MCH];
  };
  auto load = [&](uint32_t t, Stage &st) {
    const uint32_t key0 = t * BN;
    if (key0 + BN <= L) {  // whole tile in range: no per-lane checks
#pragma unroll
      for (int u = 0; u < KVCH; ++u) {
        const uint32_t c = tid + kThreads * u;
        const size_t off = (size_t)key0 * D + (size_t)(c / S::CH) * D + 8 * (c % S::CH);
        st.k[u] = *reinterpret_cast<const u32x4 *>(K + off);
        st.v[u] = *reinterpret_cast<const u32x4 *>(V + off);
      }
    } else {
#pragma unroll
      for (int u = 0; u < KVCH; ++u) {
        const uint32_t c = tid + kThreads * u;
        const uint32_t key = c / S::CH, ch = c % S::CH;
        const bool in = key0 + key < L;
        const size_t off = (size_t)(key0 + key) * D + 8 * ch;
        st.k[u] = in ? *reinterpret_cast<const u32x4 *>(K + off) : u32x4{0u, 0u, 0u, 0u};
        st.v[u] = in ? *reinterpret_cast<const u32x4 *>(V + off) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (!IMPLICIT) {
#pragma unroll
      for (int u = 0; u < MCH; ++u) {
        const uint32_t e = tid + kThreads * u;        // float4 index in the tile
        const uint32_t nd = e / (BN / 4), k4 = 4u * (e % (BN / 4));
        floatx4 x = {kMasked, kMasked, kMasked, kMasked};
        if (nd < nnodes) {
          const float *mr = a.mask + (size_t)(node0 + nd) * a.mask_stride + key0 + k4;
          if (VEC_MASK && key0 + k4 + 3u < L) {
            x = *reinterpret_cast<const floatx4 *>(mr);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (key0 + k4 + j < L) x[j] = mr[j];
          }
        }
        st.m[u] = x;
      }
    }
  };
  auto store = [&](const Stage &st, uint32_t buf) {
    half_t *Ks = Ks0 + buf * BN * D;
    half_t *Vs = Vs0 + buf * BN * D;
#pragma unroll
    for (int u = 0; u < KVCH; ++u) {
      const uint32_t c = tid + kThreads * u;
      const uint32_t key = c / S::CH, ch = c % S::CH;
      const uint32_t pos = key * D + 8 * swz(key, ch);
      *reinterpret_cast<u32x4 *>(Ks + pos) = st.k[u];
      *reinterpret_cast<u32x4 *>(Vs + pos) = st.v[u];
    }
    if (!IMPLICIT) {
      float *Ms = Ms0 + buf * (size_t)MROWS * MST;
#pragma unroll
      for (int u = 0; u < MCH; ++u) {
        const uint32_t e = tid + kThreads * u;
        const uint32_t nd = e / (BN / 4), k4 = 4u * (e % (BN / 4));
        // stored as the base-2 logit offset: log2(e) * m, or -inf when the
        // cell excludes the key (m <= -65504)
        floatx4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = st.m[u][j] > kMasked ? st.m[u][j] * kLog2e : -INFINITY;
        if (nd < nnodes) *reinterpret_cast<floatx4 *>(Ms + nd * MST + k4) = x;
      }
    }
  };

  // ---- online-softmax state of the lane's rows ----
  float Mrow[RB], Srow[RB];
  floatx4 oacc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    Mrow[rb] = -INFINITY;
    Srow[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  int64_t causal_last[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    causal_last[rb] = (int64_t)L - (int64_t)a.q_l + (int64_t)node[rb];

  // Scores and online softmax of tile t (buffer buf) for the lane's rows.
  // Sets pf (the P^T operands) and alpha (the rescale of O each row needs,
  // 1 almost always); returns 0 if none of the wavefront's cells is live.
  auto qk_softmax = [&](uint32_t t, uint32_t buf, float (&alpha_out)[RB],
                        half8_t (&pf)[RB]) -> int {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) alpha_out[rb] = 1.0f;
    const half_t *Ks = Ks0 + buf * BN * D;
    const half_t *Vs = Vs0 + buf * BN * D;
    const float *Ms = Ms0 + buf * (size_t)MROWS * MST;
    const uint32_t key0 = t * BN;
    // base-2 logit offsets of the lane's rows, keys 16kb + 4gp + j: log2(e)
    // times the mask cell, -inf for an excluded key.  Rows past the end use
    // node0's cells; their Q is zero and their results are never written.
    float m[RB][KB][4];
    float mmax = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (IMPLICIT) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = key0 + 16u * kb + 4u * gp + j;
            const bool in = key < L && (int64_t)key <= causal_last[rb];
            m[rb][kb][j] = in ? 0.0f : -INFINITY;
          }
        } else {
          const floatx4 x = *reinterpret_cast<const floatx4 *>(
              Ms + (node[rb] - node0) * MST + 16 * kb + 4 * gp);
#pragma unroll
          for (int j = 0; j < 4; ++j) m[rb][kb][j] = x[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) mmax = fmaxf(mmax, m[rb][kb][j]);
      }
    if (!__any(mmax > -INFINITY)) return 0;

    // S^T: each K operand feeds RB instructions
    floatx4 sacc[RB][KB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc[rb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t row = 16u * kb + n;
        const half8_t kf = *reinterpret_cast<const half8_t *>(
            Ks + row * D + 8 * swz(row, 4u * ds + gp));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[rb][ds], sacc[rb][kb], 0, 0, 0);
      }
    }
    // online softmax per row block; P^T operands
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s = sacc[rb][kb][j] + m[rb][kb][j];
          sacc[rb][kb][j] = s;
          tmax = fmaxf(tmax, s);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      // Lazy rescale: the reference max moves (and O, S are rescaled) only
      // when the tile's max exceeds it by more than kLazy (base 2); until
      // then p = 2^(s - M) <= 2^kLazy, exact in fp16 and fp32.  O, S and M
      // stay consistent, so the result is the same softmax.
      float alpha = 1.0f;
      if (tmax > Mrow[rb] + kLazy) {
        // (O and S are still zero when M is -inf: nothing to rescale)
        alpha = (Mrow[rb] == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(Mrow[rb] - tmax);
        Mrow[rb] = tmax;
      }
      const float m_use = (Mrow[rb] == -INFINITY) ? 0.0f : Mrow[rb];
      float p[8], psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sacc[rb][0][j] - m_use);
        p[4 + j] = __builtin_amdgcn_exp2f(sacc[rb][1][j] - m_use);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) psum += p[j];
      Srow[rb] = Srow[rb] * alpha + psum;
      pf[rb] = half8_t{(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3],
                       (half_t)p[4], (half_t)p[5], (half_t)p[6], (half_t)p[7]};
      alpha_out[rb] = alpha;
    }
    return 1;
  };
  // O^T += V^T P^T for tile buffer buf.
  auto pv = [&](uint32_t buf, const half8_t (&pf)[RB]) {
    const half_t *Vs = Vs0 + buf * BN * D;
    // O^T += V^T P^T: V^T operand of d-block db for keys F(gp, 0..7) read as
    // two transposed 4x16 blocks (keys 4gp..4gp+3 and 16+4gp..16+4gp+3)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      short4_t lo, hi;
      {
        const uint32_t r0 = 4u * gp + (n >> 2), r1 = r0 + 16u;
        const uint32_t ch = 2u * db + ((n & 3u) >> 1), half_off = 4u * (n & 1u);
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4 *)(Vs + r0 * D + 8 * swz(r0, ch) + half_off));
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4 *)(Vs + r1 * D + 8 * swz(r1, ch) + half_off));
      }
      const half8_t vf = __builtin_bit_cast(half8_t,
          (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                      hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rb], oacc[rb][db], 0, 0, 0);
    }
  };
  // The rare rescale of O: kept out of the tile loop below so that the
  // output accumulators stay in the matrix-core registers inside it.
  auto rescale = [&](const float (&alpha)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha[rb];
  };

  // ---- main loop: tile t on the matrix cores while t+1 is in flight ----
  uint32_t t0, t1;
  split_range(a.n_tiles, a.nwg, split, t0, t1);
  Stage st;
  if (t0 < t1) {
    load(t0, st);
    store(st, 0);
    __syncthreads();
  }
  uint32_t t = t0;
  float alpha[RB];
  half8_t pf[RB];
  while (t < t1) {
    // Inner loop: nothing but matrix instructions touches O.  A wavefront
    // that must rescale leaves it; every wavefront still passes exactly one
    // barrier per tile, here or in the rescale path below.
    bool need = false;
    for (; t < t1; ++t) {
      const uint32_t buf = (t - t0) & 1u;
      if (t + 1 < t1) load(t + 1, st);
      const int live = qk_softmax(t, buf, alpha, pf);
      bool r = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) r |= alpha[rb] != 1.0f;
      if (__builtin_expect(__any(r), 0)) {
        need = true;
        break;
      }
      if (live) pv(buf, pf);
      if (t + 1 < t1) store(st, buf ^ 1u);
      __syncthreads();
    }
    if (!need) break;
    const uint32_t buf = (t - t0) & 1u;
    rescale(alpha);
    pv(buf, pf);
    if (t + 1 < t1) store(st, buf ^ 1u);
    __syncthreads();
    ++t;
  }

  // ---- results ----
  const size_t nrows = (size_t)a.n_heads * a.q_l;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float stot = Srow[rb] + __shfl_xor(Srow[rb], 16);
    stot += __shfl_xor(stot, 32);
    if (!valid[rb]) continue;
    const uint32_t gr = row0 + wave * 16u * RB + 16u * rb + n;
    const uint32_t head = hk * a.group + gr % a.group;
    const size_t rid = (size_t)node[rb] * a.n_heads + head;
    if (a.nwg == 1) {
      const float inv = (stot > 0.0f) ? 1.0f / stot : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<floatx4 *>(a.out + rid * D + 16 * db + 4 * gp) = oacc[rb][db] * inv;
    } else {
      const size_t prow = (size_t)split * nrows + rid;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<floatx4 *>(a.part_o + prow * D + 16 * db + 4 * gp) = oacc[rb][db];
      if (gp == 0) {
        a.part_sm[prow * 2 + 0] = stot;
        a.part_sm[prow * 2 + 1] = Mrow[rb];
      }
    }
  }
}

template <int D, int RB, int MROWS, bool IMPLICIT, bool VEC>
hipError_t launch_v(const FwdArgs &a, hipStream_t s) {
  using Sh = F16Shape<D, RB, MROWS>;
  const size_t lds = Sh::KV_LDS + (IMPLICIT ? 0 : 2 * (size_t)MROWS * MST * sizeof(float));
  static const bool attr_set = [] {
    (void)hipFuncSetAttribute((const void *)fwd_f16_kernel<D, RB, MROWS, IMPLICIT, VEC>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_set;
  dim3 grid(grid_size(a.units, a.row_tiles));
  hipLaunchKernelGGL((fwd_f16_kernel<D, RB, MROWS, IMPLICIT, VEC>), grid, dim3(kThreads), lds,
                     s, a);
  return hipGetLastError();
}

template <int D, int RB>
hipError_t launch_rb(const FwdArgs &a, hipStream_t s) {
  constexpr int RPW = 64 * RB;
  if (a.mask == nullptr) return launch_v<D, RB, 64, true, false>(a, s);
  // a row tile spans at most floor((RPW - 1) / group) + 2 tree nodes
  const bool narrow = (RPW - 1) / a.group + 2 <= 64u;
  const bool vec = ((uintptr_t)a.mask % 16u == 0) && (a.mask_stride % 4u == 0);
  if (narrow)
    return vec ? launch_v<D, RB, 64, false, true>(a, s) : launch_v<D, RB, 64, false, false>(a, s);
  return vec ? launch_v<D, RB, RPW, false, true>(a, s) : launch_v<D, RB, RPW, false, false>(a, s);
}

}  // namespace

uint32_t f16_tile_keys(uint32_t) { return (uint32_t)BN; }

// Row blocks per wavefront: as many as registers allow without spilling (3
// for head_dim 128, 2 for 256, 1 for 512), fewer when that wastes fewer
// padded rows.
uint32_t f16_row_blocks(uint32_t head_dim, uint32_t rows) {
  const uint32_t max_rb = head_dim >= 512 ? 1u : head_dim >= 256 ? 2u : 3u;
  uint32_t best = 1, best_waste = 0xffffffffu;
  for (uint32_t rb = max_rb; rb >= 1; --rb) {
    const uint32_t rpw = 64u * rb;
    const uint32_t waste = ((rows + rpw - 1) / rpw) * rpw - rows;
    if (waste < best_waste) {
      best = rb;
      best_waste = waste;
    }
  }
  return best;
}

hipError_t launch_forward_f16(const FwdArgs &a, uint32_t head_dim, hipStream_t s) {
  const uint32_t rb = f16_row_blocks(head_dim, a.rows);
  switch (head_dim) {
    case 128:
      return rb == 3 ? launch_rb<128, 3>(a, s) : rb == 2 ? launch_rb<128, 2>(a, s)
                                                         : launch_rb<128, 1>(a, s);
    case 256:
      return rb == 2 ? launch_rb<256, 2>(a, s) : launch_rb<256, 1>(a, s);
    case 512: return launch_rb<512, 1>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
