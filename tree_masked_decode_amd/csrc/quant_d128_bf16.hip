// quant_d128_bf16.hip -- the head-dim-128 variants of the quantized kernel with
// bfloat16 queries, scales, biases, mask and output.
#include "quant_impl.h"

namespace ta {

hipError_t launch_quant_d128_bf16(const QuantArgs &a, uint32_t bits, uint32_t group,
                               hipStream_t s) {
  return launch_qb<128, 1>(a, bits, group, s);
}

uint32_t quant_wgs_d128_bf16(uint32_t bits, uint32_t group, int mask_kind) {
  return wgs_per_cu_b<128, 1>(bits, group, mask_kind);
}

}  // namespace ta
