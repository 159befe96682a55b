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
// Merge of split partials.  One wavefront per output row; splits are visited
// in index order so the result does not depend on timing.  M is in base-2
// units, so the rescale factor of split w is 2^(M_w - M*).
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

template <bool OUT_F16>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t r = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (r >= a.nrows) return;
  const float *sm = a.part_sm;
  const size_t nrows = a.nrows;

  float mstar = -INFINITY;
  for (uint32_t w = lane; w < a.nwg; w += 64u) {
    float s = sm[((size_t)w * nrows + r) * 2 + 0];
    float m = sm[((size_t)w * nrows + r) * 2 + 1];
    if (s > 0.0f) mstar = fmaxf(mstar, m);
  }
  mstar = wave_max(mstar);
  float sstar = 0.0f;
  if (mstar != -INFINITY) {
    for (uint32_t w = lane; w < a.nwg; w += 64u) {
      float s = sm[((size_t)w * nrows + r) * 2 + 0];
      float m = sm[((size_t)w * nrows + r) * 2 + 1];
      if (s > 0.0f) sstar += s * exp2f(m - mstar);
    }
  }
  sstar = wave_sum(sstar);
  const float inv = (sstar > 0.0f) ? 1.0f / sstar : 0.0f;

  for (uint32_t d4 = lane; d4 < a.dim / 4u; d4 += 64u) {
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (sstar > 0.0f) {
      for (uint32_t w = 0; w < a.nwg; ++w) {
        float s = sm[((size_t)w * nrows + r) * 2 + 0];
        if (!(s > 0.0f)) continue;
        float f = exp2f(sm[((size_t)w * nrows + r) * 2 + 1] - mstar);
        const floatx4 o = *reinterpret_cast<const floatx4 *>(
            a.part_o + ((size_t)w * nrows + r) * a.dim + 4u * d4);
        acc += o * f;
      }
    }
    acc *= inv;
    if (OUT_F16) {
      half4_t h = {(half_t)acc[0], (half_t)acc[1], (half_t)acc[2],
                   (half_t)acc[3]};
      *reinterpret_cast<half4_t *>(static_cast<half_t *>(a.out) +
                                   (size_t)r * a.dim + 4u * d4) = h;
    } else {
      *reinterpret_cast<floatx4 *>(static_cast<float *>(a.out) +
                                   (size_t)r * a.dim + 4u * d4) = acc;
    }
  }
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s) {
  dim3 grid((a.nrows + 3u) / 4u);
  if (a.out_f16)
    hipLaunchKernelGGL(reduce_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(reduce_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ta
