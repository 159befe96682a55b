// quant_d512_f16.hip -- the head-dim-512 variants of the quantized kernel with
// fp16 queries, scales, biases, mask and output.
#include "quant_impl.h"

namespace ta {

hipError_t launch_quant_d512_f16(const QuantArgs &a, uint32_t bits, uint32_t group,
                               hipStream_t s) {
  return launch_qb<512, 0>(a, bits, group, s);
}

uint32_t quant_wgs_d512_f16(uint32_t bits, uint32_t group, int mask_kind) {
  return wgs_per_cu_b<512, 0>(bits, group, mask_kind);
}

}  // namespace ta
