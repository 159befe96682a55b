// kern_misc.hip -- the two small kernels of the path: explicit tree-mask
// construction and the log-sum-exp merge of split partials.
#include "common.h"

namespace ta {

// ---------------------------------------------------------------------------
// Tree mask ("tree_attention.metal" header: every tree topology becomes a
// [q_l, kv_seq_len] mask of 0 / -65504; node i sits at kv_seq_len - q_l + i).
// Grid (column blocks, q_l); each block first marks node i's root path in an
// LDS bitmap, then writes its slice of row i.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tree_mask_kernel(MaskArgs a) {
  __shared__ uint32_t path[kMaxTreeNodes / 32];
  const uint32_t i = blockIdx.y;
  for (uint32_t w = threadIdx.x; w < kMaxTreeNodes / 32; w += blockDim.x)
    path[w] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    // parents[n] < n for n > 0 and parents[0] == -1 (checked on the host),
    // so the walk ends after at most i steps.
    int n = (int)i;
    while (n >= 0) {
      path[n >> 5] |= 1u << (n & 31);
      n = a.parents[n];
    }
  }
  __syncthreads();
  const uint32_t base = a.kv_seq_len - a.q_l;
  float *row = a.mask + (size_t)i * a.mask_stride;
  const uint32_t step = gridDim.x * blockDim.x;
  for (uint32_t j = blockIdx.x * blockDim.x + threadIdx.x; j < a.mask_stride;
       j += step) {
    float val = kMasked;
    if (j < base) {
      val = 0.0f;
    } else if (j < a.kv_seq_len) {
      uint32_t n = j - base;
      val = ((path[n >> 5] >> (n & 31)) & 1u) ? 0.0f : kMasked;
    }
    row[j] = val;
  }
}

hipError_t launch_tree_mask(const MaskArgs &a, hipStream_t s) {
  uint32_t per_block = 256u * 8u;
  uint32_t bx = (a.mask_stride + per_block - 1) / per_block;
  if (bx == 0) bx = 1;
  hipLaunchKernelGGL(tree_mask_kernel, dim3(bx, a.q_l), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of split partials (log-sum-exp combine).  M is in base-2 units, so
// split w's rescale factor is 2^(M_w - M*), M* the largest M of a non-empty
// split; the row is sum_w O_w 2^(M_w - M*) / sum_w S_w 2^(M_w - M*), and an
// empty row (no non-empty split) is 0.
//
// A block of 256 threads owns RPB rows.  Phase 1: wavefront v finds M* and
// 1/S* of rows v, v+4, ... (lanes over splits) and leaves them in LDS.
// Phase 2: TPR threads per row each own float4 columns of the row and walk the
// splits in index order, eight independent loads at a time, so the sum does
// not depend on timing and enough loads are in flight to cover latency.
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

typedef float float2_t __attribute__((ext_vector_type(2)));

template <bool OUT_F16, uint32_t TPR>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  constexpr uint32_t RPB = 256u / TPR;
  constexpr uint32_t U = 8;
  __shared__ float s_mstar[RPB], s_inv[RPB];
  const uint32_t wv = threadIdx.x >> 6, lane = threadIdx.x & 63u;
  const size_t nrows = a.nrows;
  const float2_t *sm = reinterpret_cast<const float2_t *>(a.part_sm);  // (S, M)
  const uint32_t row0 = blockIdx.x * RPB;

  for (uint32_t rr = wv; rr < RPB; rr += 4u) {
    const size_t r = row0 + rr;
    float mstar = -INFINITY, ssum = 0.0f;
    if (r < nrows) {
      for (uint32_t w = lane; w < a.nwg; w += 64u) {
        const float2_t v = sm[(size_t)w * nrows + r];
        if (v.x > 0.0f) mstar = fmaxf(mstar, v.y);
      }
      mstar = wave_max(mstar);
      if (mstar != -INFINITY) {
        for (uint32_t w = lane; w < a.nwg; w += 64u) {
          const float2_t v = sm[(size_t)w * nrows + r];
          if (v.x > 0.0f) ssum += v.x * exp2f(v.y - mstar);
        }
      }
      ssum = wave_sum(ssum);
    }
    if (lane == 0) {
      s_mstar[rr] = mstar;
      s_inv[rr] = ssum > 0.0f ? 1.0f / ssum : 0.0f;
    }
  }
  __syncthreads();

  const uint32_t rr = threadIdx.x / TPR, t = threadIdx.x % TPR;
  const size_t r = row0 + rr;
  if (r >= nrows) return;
  const float mstar = s_mstar[rr], inv = s_inv[rr];
  const uint32_t d4n = a.dim / 4u;
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (uint32_t d4 = t; d4 < d4n; d4 += TPR) {
    floatx4 acc = zero;
    if (inv > 0.0f) {
      const floatx4 *po = reinterpret_cast<const floatx4 *>(a.part_o) + r * d4n + d4;
      const size_t wstride = nrows * d4n;
      uint32_t w = 0;
      for (; w + U <= a.nwg; w += U) {
        floatx4 o[U];
        float2_t v[U];
#pragma unroll
        for (uint32_t j = 0; j < U; ++j) {
          v[j] = sm[(size_t)(w + j) * nrows + r];
          o[j] = po[(size_t)(w + j) * wstride];
        }
#pragma unroll
        for (uint32_t j = 0; j < U; ++j) {
          // an empty split (S = 0) contributes nothing, whatever its O holds
          const bool use = v[j].x > 0.0f;
          const float f = use ? exp2f(v[j].y - mstar) : 0.0f;
          acc += (use ? o[j] : zero) * f;
        }
      }
      for (; w < a.nwg; ++w) {
        const float2_t v = sm[(size_t)w * nrows + r];
        const floatx4 o = po[(size_t)w * wstride];
        const bool use = v.x > 0.0f;
        const float f = use ? exp2f(v.y - mstar) : 0.0f;
        acc += (use ? o : zero) * f;
      }
    }
    acc *= inv;
    if (OUT_F16) {
      half4_t h = {(half_t)acc[0], (half_t)acc[1], (half_t)acc[2], (half_t)acc[3]};
      reinterpret_cast<half4_t *>(a.out)[r * d4n + d4] = h;
    } else {
      reinterpret_cast<floatx4 *>(a.out)[r * d4n + d4] = acc;
    }
  }
}

template <uint32_t TPR>
hipError_t launch_reduce_t(const ReduceArgs &a, hipStream_t s) {
  constexpr uint32_t RPB = 256u / TPR;
  dim3 grid((a.nrows + RPB - 1u) / RPB);
  if (a.out_f16)
    hipLaunchKernelGGL((reduce_kernel<true, TPR>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((reduce_kernel<false, TPR>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s) {
  const uint32_t d4n = a.dim / 4u;
  if (d4n >= 64u) return launch_reduce_t<64>(a, s);
  if (d4n >= 32u) return launch_reduce_t<32>(a, s);
  return launch_reduce_t<16>(a, s);
}

}  // namespace ta
