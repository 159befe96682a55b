// fwd_f32.hip -- tree-attention forward for fp32 K/V on the vector ALUs.
//
// "tree_attention.metal" (mlx-native 0.9.1), tree_attention_impl: per
// (query, head) an online softmax over KV chunks with an explicit mask, GQA
// head mapping, split-KV partials.  Here one workgroup serves every query row
// that shares a kv head (up to 16 rows: (node, head-in-group) pairs), so each
// K/V tile is read from memory once for all of them; K/V, Q and the
// probabilities are staged in LDS.  All arithmetic is fp32 (no fp16 rounding
// of Q, K or P), which keeps the result within 1e-4 of the exact softmax.
#include "common.h"

namespace ta {

namespace {

constexpr int kThreads = 256;
constexpr int kRT = (int)kF32RowsPerWG;  // rows per workgroup

template <int D> struct F32Shape {
  static constexpr int BN = (D >= 512) ? 16 : 32;  // keys per tile
  static constexpr int KST = D + 1;                // K row stride (floats)
  static constexpr int QST = D + 4;                // Q row stride
  static constexpr int PST = BN + 1;               // P row stride
  static constexpr int EPT = kRT * D / kThreads;   // outputs per thread
};

template <int D>
constexpr size_t f32_lds_bytes() {
  using S = F32Shape<D>;
  return sizeof(float) * (S::BN * S::KST + S::BN * D + kRT * S::QST +
                          kRT * S::PST + 3 * kRT);
}

// Mask cell of (node i, key j), or "excluded".  IMPLICIT computes the
// causal / sliding-window rule of the "tree_attention.metal" header
// (key_lo <= j <= L - q_l + i); the explicit form reads the caller's
// [q_l, mask_stride] buffer.  Both feed the same arithmetic below, so an
// explicit mask of the same rule reproduces the implicit result bit for bit
// whenever both cover the same tiles.
template <bool IMPLICIT>
__device__ inline float mask_cell(const FwdArgs &a, uint32_t i, uint32_t j) {
  if (IMPLICIT) {
    int64_t last = (int64_t)a.kv_seq_len - (int64_t)a.q_l + (int64_t)i;
    return (j >= a.key_lo && (int64_t)j <= last) ? 0.0f : kMasked;
  }
  return a.mask[(size_t)i * a.mask_stride + j];
}

template <int D, bool IMPLICIT>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  using S = F32Shape<D>;
  constexpr int BN = S::BN;
  extern __shared__ float lds[];
  float *Ks = lds;                       // [BN][KST]
  float *Vs = Ks + BN * S::KST;          // [BN][D]
  float *Qs = Vs + BN * D;               // [RT][QST]
  float *Ps = Qs + kRT * S::QST;         // [RT][PST]
  float *Mrow = Ps + kRT * S::PST;       // running max (base 2)
  float *Srow = Mrow + kRT;              // running sum
  float *Arow = Srow + kRT;              // rescale of the current tile

  uint32_t unit, rt;
  decode_block(blockIdx.x, a.row_tiles, unit, rt);
  if (unit >= a.units) return;
  const uint32_t hk = unit / a.nwg;
  const uint32_t split = unit % a.nwg;
  const uint32_t tid = threadIdx.x;
  const uint32_t row0 = rt * kRT;

  if (tid < (uint32_t)kRT) {
    Mrow[tid] = -INFINITY;
    Srow[tid] = 0.0f;
  }
  float acc[S::EPT];
#pragma unroll
  for (int k = 0; k < S::EPT; ++k) acc[k] = 0.0f;

  // the splits cover the tiles from the one that holds key_lo
  const uint32_t tile_lo = a.key_lo / S::BN;
  uint32_t t0, t1;
  uint32_t span_lo, span_hi;
  split_tiles(a, S::BN, tile_lo, span_lo, span_hi);
  split_range(span_hi - span_lo, a.nwg, split, t0, t1);
  t0 += span_lo;
  t1 += span_lo;
  const size_t kvbase = (size_t)hk * a.kv_capacity * D;
  const float *K = static_cast<const float *>(a.k) + kvbase;
  const float *V = static_cast<const float *>(a.v) + kvbase;

  // Score-phase mapping: key column j, rows r0 + 8*u.
  const uint32_t sj = tid % BN;
  const uint32_t sr = tid / BN;
  constexpr int kRowsPerThread = kRT * BN / kThreads;
  constexpr int kRowStep = kThreads / BN;

  // K/V tile loads go into registers one tile ahead, so that their latency
  // overlaps the arithmetic of the tile before.  They are unconditional, from
  // an in-bounds address (a key past kv_seq_len reads row kv_seq_len - 1),
  // and such rows are zeroed where they are staged, so no load waits at a
  // branch.  (Loading the mask cells one tile ahead as well measured slower
  // on the short calls this kernel serves; they are read at the top of
  // their tile.)
  constexpr int kLoadsPerThread = BN * D / 4 / kThreads;
  static_assert(kLoadsPerThread * kThreads * 4 == BN * D, "tile / thread shape");
  floatx4 kreg[kLoadsPerThread], vreg[kLoadsPerThread];
  auto load_kv = [&](uint32_t t) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const uint32_t e = tid + (uint32_t)i * kThreads;
      const uint32_t key = min(t * BN + e / (D / 4), a.kv_seq_len - 1u), c4 = e % (D / 4);
      kreg[i] = *reinterpret_cast<const floatx4 *>(K + (size_t)key * D + 4 * c4);
      vreg[i] = *reinterpret_cast<const floatx4 *>(V + (size_t)key * D + 4 * c4);
    }
  };
  if (t0 < t1) load_kv(t0);

  // Q rows of this workgroup (rows past the end read as zero), loaded after
  // the first tile's so that the two latencies overlap
  {
    constexpr int kQPerThread = kRT * D / 4 / kThreads;
    static_assert(kQPerThread * kThreads * 4 == kRT * D, "Q / thread shape");
#pragma unroll
    for (int v = 0; v < kQPerThread; ++v) {
      const uint32_t e = tid + (uint32_t)v * kThreads;
      const uint32_t r = e / (D / 4), c4 = e % (D / 4), gr = row0 + r;
      const uint32_t grc = gr < a.rows ? gr : row0;
      const uint32_t i = grc / a.group, h = hk * a.group + grc % a.group;
      const floatx4 x = *reinterpret_cast<const floatx4 *>(a.q + ((size_t)h * a.q_l + i) * D + 4 * c4);
      *reinterpret_cast<floatx4 *>(Qs + r * S::QST + 4 * c4) =
          gr < a.rows ? x : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t key0 = t * BN;
    // --- mask cells of this thread's (row, key) pairs; tile liveness ---
    float mval[kRowsPerThread];
    int live = 0;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      uint32_t r = sr + u * kRowStep, gr = row0 + r, j = key0 + sj;
      float m = kMasked;
      if (gr < a.rows && j < a.kv_seq_len) m = mask_cell<IMPLICIT>(a, gr / a.group, j);
      mval[u] = m;
      live |= (m > kMasked);
    }
    // Every cell of the tile masked: skip it ("tree_attention.metal" skips a
    // chunk whose cells are all at or below -65504).
    if (!__syncthreads_or(live)) {
      if (t + 1 < t1) load_kv(t + 1);   // (the registers held this tile)
      continue;
    }

    // --- stage the K/V tile from registers (keys past kv_seq_len as zero),
    // then fetch the next one ---
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const uint32_t e = tid + (uint32_t)i * kThreads;
      const uint32_t key = e / (D / 4), c4 = e % (D / 4);
      const bool in = key0 + key < a.kv_seq_len;
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      const floatx4 kx = in ? kreg[i] : zero;
#pragma unroll
      for (int x = 0; x < 4; ++x) Ks[key * S::KST + 4 * c4 + x] = kx[x];
      *reinterpret_cast<floatx4 *>(Vs + key * D + 4 * c4) = in ? vreg[i] : zero;
    }
    __syncthreads();
    if (t + 1 < t1) load_kv(t + 1);

    // --- scores s = scale*log2e * q.k + log2e * mask (base-2 logits) ---
    // (four partial sums over d, so that the FMA chains overlap)
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      uint32_t r = sr + u * kRowStep;
      const float *qr = Qs + r * S::QST;
      const float *kr = Ks + sj * S::KST;
      float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
      for (int d = 0; d < D; d += 4) {
        const floatx4 q4 = *reinterpret_cast<const floatx4 *>(qr + d);
#pragma unroll
        for (int x = 0; x < 4; ++x) d4[x] = fmaf(q4[x], kr[d + x], d4[x]);
      }
      const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      float s = fmaf(dot, a.qscale, mval[u] * kLog2e);
      Ps[r * S::PST + sj] = (mval[u] > kMasked) ? s : -INFINITY;
    }
    __syncthreads();

    // --- online softmax, one wavefront per 4 rows, 32 lanes per row ---
    {
      const uint32_t wave = tid / kWave, lane = tid % kWave;
      const uint32_t half = lane / 32, col = lane % 32;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        uint32_t r = wave * 4 + pr * 2 + half;
        float s = (col < (uint32_t)BN) ? Ps[r * S::PST + col] : -INFINITY;
        float mx = s;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float m_old = Mrow[r];
        float m_new = fmaxf(m_old, mx);
        float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        float p = exp2f(s - m_use);
        float ps = p;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
        if (col < (uint32_t)BN) Ps[r * S::PST + col] = p;
        if (col == 0) {
          float alpha = exp2f(m_old - m_use);
          Arow[r] = alpha;
          Srow[r] = Srow[r] * alpha + ps;
          Mrow[r] = m_new;
        }
      }
    }
    __syncthreads();

    // --- O = alpha * O + P V ---
#pragma unroll
    for (int k = 0; k < S::EPT; ++k) {
      uint32_t e = tid + k * kThreads;
      uint32_t r = e / D, d = e % D;
      const float *pr = Ps + r * S::PST;
      float o4[4] = {acc[k] * Arow[r], 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < BN; j += 4)
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = fmaf(pr[j + x], Vs[(j + x) * D + d], o4[x]);
      acc[k] = (o4[0] + o4[1]) + (o4[2] + o4[3]);
    }
    __syncthreads();
  }

  // --- results: partials (nwg > 1) or the normalised output (nwg == 1) ---
  const size_t nrows = (size_t)a.n_heads * a.q_l;
#pragma unroll
  for (int k = 0; k < S::EPT; ++k) {
    uint32_t e = tid + k * kThreads;
    uint32_t r = e / D, d = e % D, gr = row0 + r;
    if (gr >= a.rows) continue;
    uint32_t i = gr / a.group, h = hk * a.group + gr % a.group;
    size_t rid = (size_t)i * a.n_heads + h;
    if (a.nwg == 1) {
      float s = Srow[r];
      a.out[rid * D + d] = (s > 0.0f) ? acc[k] / s : 0.0f;
    } else {
      a.part_o[((size_t)split * nrows + rid) * D + d] = acc[k];
      if (d == 0) {
        a.part_sm[((size_t)split * nrows + rid) * 2 + 0] = Srow[r];
        a.part_sm[((size_t)split * nrows + rid) * 2 + 1] = Mrow[r];
      }
    }
  }
}

template <int D>
hipError_t launch_f32_d(const FwdArgs &a, hipStream_t s) {
  constexpr size_t lds = f32_lds_bytes<D>();
  dim3 grid(grid_size(a.units, a.row_tiles));
  if (a.mask == nullptr) {
    (void)hipFuncSetAttribute((const void *)fwd_f32_kernel<D, true>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), grid, dim3(kThreads), lds, s, a);
  } else {
    (void)hipFuncSetAttribute((const void *)fwd_f32_kernel<D, false>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), grid, dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

uint32_t f32_tile_keys(uint32_t head_dim) { return head_dim >= 512 ? 16u : 32u; }

hipError_t launch_forward_f32(const FwdArgs &a, uint32_t head_dim,
                              hipStream_t s) {
  switch (head_dim) {
    case 128: return launch_f32_d<128>(a, s);
    case 256: return launch_f32_d<256>(a, s);
    case 512: return launch_f32_d<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
