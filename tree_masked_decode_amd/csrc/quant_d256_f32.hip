// quant_d256_f32.hip -- the head-dim-256 variants of the quantized kernel with
// fp32 queries, scales, biases, mask and output.
#include "quant_impl.h"

namespace ta {

hipError_t launch_quant_d256_f32(const QuantArgs &a, uint32_t bits, uint32_t group,
                               hipStream_t s) {
  return launch_qb<256, 2>(a, bits, group, s);
}

uint32_t quant_wgs_d256_f32(uint32_t bits, uint32_t group, int mask_kind) {
  return wgs_per_cu_b<256, 2>(bits, group, mask_kind);
}

}  // namespace ta
