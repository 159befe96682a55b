// quant.hip -- dispatch of the quantized forward over head dims (the
// kernel itself is in quant_impl.h, one translation unit per head dim).
#include "common.h"

namespace ta {

#define TA_QUANT_DIM(d)                                                                  \
  hipError_t launch_quant_d##d(const QuantArgs &a, uint32_t bits, uint32_t group,       \
                               hipStream_t s);                                           \
  uint32_t quant_wgs_d##d(uint32_t bits, uint32_t group, int mask_kind);
TA_QUANT_DIM(64)
TA_QUANT_DIM(96)
TA_QUANT_DIM(128)
TA_QUANT_DIM(256)
TA_QUANT_DIM(512)
#undef TA_QUANT_DIM

uint32_t quant_tile_keys(uint32_t) { return 32u; }

uint32_t quant_wgs_per_cu(uint32_t dim, uint32_t bits, uint32_t group, int mask_kind) {
  switch (dim) {
    case 64: return quant_wgs_d64(bits, group, mask_kind);
    case 96: return quant_wgs_d96(bits, group, mask_kind);
    case 128: return quant_wgs_d128(bits, group, mask_kind);
    case 256: return quant_wgs_d256(bits, group, mask_kind);
    case 512: return quant_wgs_d512(bits, group, mask_kind);
    default: return 0;
  }
}

hipError_t launch_quant_forward(const QuantArgs &a, uint32_t dim, uint32_t bits,
                                uint32_t group, hipStream_t s) {
  switch (dim) {
    case 64: return launch_quant_d64(a, bits, group, s);
    case 96: return launch_quant_d96(a, bits, group, s);
    case 128: return launch_quant_d128(a, bits, group, s);
    case 256: return launch_quant_d256(a, bits, group, s);
    case 512: return launch_quant_d512(a, bits, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
