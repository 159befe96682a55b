// kern_misc.hip -- the small kernels of the path: explicit tree-mask
// construction, the live-key scan of an explicit mask, and the log-sum-exp
// merge of split partials.
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
// One block of 256 threads per output row.  Phase 1: wavefront 0 finds M*
// and 1/S* (lanes over splits).  Phase 2: thread (g, t) owns float4 columns
// t, t + T, ... of the row and sums splits g, g + G, g + 2G, ... in index
// order (G = 256 / T split groups, so every thread has few splits and all of
// its loads are in flight together); the G group sums are then added in
// group order through LDS.  The result does not depend on timing.
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

template <int OUT, uint32_t T, uint32_t C>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  // T threads per column set, C float4 columns per thread (dim = 4 T C at
  // most), G split groups
  constexpr uint32_t G = 256u / T;
  __shared__ float s_mstar, s_inv;
  __shared__ floatx4 s_part[G][T * C];
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const size_t nrows = a.nrows;
  const size_t r = blockIdx.x;
  const float2_t *sm = reinterpret_cast<const float2_t *>(a.part_sm);  // (S, M)

  if (tid < 64) {
    float mstar = -INFINITY, ssum = 0.0f;
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
    if (lane == 0) {
      s_mstar = mstar;
      s_inv = ssum > 0.0f ? 1.0f / ssum : 0.0f;
    }
  }
  __syncthreads();
  const float mstar = s_mstar, inv = s_inv;
  const uint32_t g = tid / T, t = tid % T;
  const uint32_t d4n = a.dim / 4u;
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const floatx4 *po = reinterpret_cast<const floatx4 *>(a.part_o) + r * d4n;
  const size_t wstride = nrows * d4n;
  floatx4 acc[C];
#pragma unroll
  for (uint32_t c = 0; c < C; ++c) acc[c] = zero;
  if (inv > 0.0f) {
    constexpr uint32_t U = 4;
    uint32_t w = g;
    for (; w + (U - 1) * G < a.nwg; w += U * G) {
      float2_t v[U];
      floatx4 o[U][C];
#pragma unroll
      for (uint32_t j = 0; j < U; ++j) {
        v[j] = sm[(size_t)(w + j * G) * nrows + r];
#pragma unroll
        for (uint32_t c = 0; c < C; ++c) {
          const uint32_t d4 = t + c * T;
          o[j][c] = d4 < d4n ? po[(size_t)(w + j * G) * wstride + d4] : zero;
        }
      }
#pragma unroll
      for (uint32_t j = 0; j < U; ++j) {
        // an empty split (S = 0) contributes nothing, whatever its O holds
        const bool use = v[j].x > 0.0f;
        const float f = use ? exp2f(v[j].y - mstar) : 0.0f;
#pragma unroll
        for (uint32_t c = 0; c < C; ++c) acc[c] += (use ? o[j][c] : zero) * f;
      }
    }
    for (; w < a.nwg; w += G) {
      const float2_t v = sm[(size_t)w * nrows + r];
      const bool use = v.x > 0.0f;
      const float f = use ? exp2f(v.y - mstar) : 0.0f;
#pragma unroll
      for (uint32_t c = 0; c < C; ++c) {
        const uint32_t d4 = t + c * T;
        const floatx4 o = d4 < d4n ? po[(size_t)w * wstride + d4] : zero;
        acc[c] += (use ? o : zero) * f;
      }
    }
  }
#pragma unroll
  for (uint32_t c = 0; c < C; ++c) s_part[g][t + c * T] = acc[c];
  __syncthreads();
  // group sums in group order; thread tid < T * C finishes column tid
  for (uint32_t d4 = tid; d4 < d4n && d4 < T * C; d4 += 256u) {
    floatx4 sum = s_part[0][d4];
#pragma unroll
    for (uint32_t gg = 1; gg < G; ++gg) sum += s_part[gg][d4];
    sum *= inv;
    if (OUT == 1) {
      half4_t h = {(half_t)sum[0], (half_t)sum[1], (half_t)sum[2], (half_t)sum[3]};
      reinterpret_cast<half4_t *>(a.out)[r * d4n + d4] = h;
    } else if (OUT == 2) {
      const uint32_t lo = f32_to_bf16(sum[0]) | ((uint32_t)f32_to_bf16(sum[1]) << 16);
      const uint32_t hi = f32_to_bf16(sum[2]) | ((uint32_t)f32_to_bf16(sum[3]) << 16);
      reinterpret_cast<u32x2 *>(a.out)[r * d4n + d4] = u32x2{lo, hi};
    } else {
      reinterpret_cast<floatx4 *>(a.out)[r * d4n + d4] = sum;
    }
  }
}

template <uint32_t T, uint32_t C>
hipError_t launch_reduce_t(const ReduceArgs &a, hipStream_t s) {
  dim3 grid(a.nrows);
  if (a.out_type == 1)
    hipLaunchKernelGGL((reduce_kernel<1, T, C>), grid, dim3(256), 0, s, a);
  else if (a.out_type == 2)
    hipLaunchKernelGGL((reduce_kernel<2, T, C>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((reduce_kernel<0, T, C>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// dim <= 512 (checked by the caller): T C >= dim / 4
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s) {
  const uint32_t d4n = a.dim / 4u;
  if (d4n > 64u) return launch_reduce_t<64, 2>(a, s);
  if (d4n > 32u) return launch_reduce_t<64, 1>(a, s);
  if (d4n > 16u) return launch_reduce_t<32, 1>(a, s);
  return launch_reduce_t<16, 1>(a, s);
}

// ---------------------------------------------------------------------------
// Live-key scan of an explicit mask ("tree_attention.metal",
// tree_attention_impl: a key chunk whose mask cells are all at or below
// -65504 contributes nothing and is skipped).  Block c takes keys
// [c L / chunks, (c + 1) L / chunks) of every row and writes the first and
// last key with a live cell (a NaN cell counts as live, as the forward would
// add it), or (0xffffffff, 0).  The forward then splits only the tiles
// between the overall first and last live key, so a dead prefix or suffix
// (a sliding window written as a mask) is neither fetched nor given splits.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_range_kernel(MaskRangeArgs a) {
  __shared__ uint32_t s_first[4], s_last[4];
  const uint32_t c = blockIdx.x;
  const uint32_t k0 = (uint32_t)(((uint64_t)a.kv_seq_len * c) / a.chunks);
  const uint32_t k1 = (uint32_t)(((uint64_t)a.kv_seq_len * (c + 1)) / a.chunks);
  uint32_t first = 0xffffffffu, last = 0u;
  for (uint32_t j = k0 + threadIdx.x; j < k1; j += 256u) {
    bool live = false;
    for (uint32_t i = 0; i < a.q_l && !live; ++i)
      live = !(a.mask[(size_t)i * a.mask_stride + j] <= kMasked);
    if (live) {
      first = min(first, j);
      last = max(last, j);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    first = min(first, (uint32_t)__shfl_xor((int)first, o));
    last = max(last, (uint32_t)__shfl_xor((int)last, o));
  }
  const uint32_t wave = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    s_first[wave] = first;
    s_last[wave] = last;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      first = min(first, s_first[w]);
      last = max(last, s_last[w]);
    }
    if (first == 0xffffffffu) last = 0u;
    reinterpret_cast<u32x2 *>(a.out)[c] = u32x2{first, last};
  }
}

hipError_t launch_mask_range(const MaskRangeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(mask_range_kernel, dim3(a.chunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ta
