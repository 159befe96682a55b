// quant.hip -- dispatch of the quantized forward over head dims and element
// types (the kernel itself is in quant_impl.h, one translation unit per head
// dim and element type).
#include "common.h"

namespace ta {

#define TA_QUANT_VARIANT(d, t)                                                           \
  hipError_t launch_quant_d##d##_##t(const QuantArgs &a, uint32_t bits, uint32_t group, \
                                     hipStream_t s);                                     \
  uint32_t quant_wgs_d##d##_##t(uint32_t bits, uint32_t group, int mask_kind);
#define TA_QUANT_DIM(d) TA_QUANT_VARIANT(d, f16) TA_QUANT_VARIANT(d, bf16) TA_QUANT_VARIANT(d, f32)
TA_QUANT_DIM(64)
TA_QUANT_DIM(96)
TA_QUANT_DIM(128)
TA_QUANT_DIM(256)
TA_QUANT_DIM(512)
#undef TA_QUANT_DIM
#undef TA_QUANT_VARIANT

uint32_t quant_tile_keys(uint32_t) { return 32u; }

// elem: 0 fp16, 1 bf16, 2 fp32
#define TA_BY_ELEM(d, call, ...)                                   \
  (elem == 1 ? call##_d##d##_bf16(__VA_ARGS__)                     \
             : elem == 2 ? call##_d##d##_f32(__VA_ARGS__) : call##_d##d##_f16(__VA_ARGS__))

uint32_t quant_wgs_per_cu(uint32_t dim, uint32_t bits, uint32_t group, int mask_kind,
                          int elem) {
  switch (dim) {
    case 64: return TA_BY_ELEM(64, quant_wgs, bits, group, mask_kind);
    case 96: return TA_BY_ELEM(96, quant_wgs, bits, group, mask_kind);
    case 128: return TA_BY_ELEM(128, quant_wgs, bits, group, mask_kind);
    case 256: return TA_BY_ELEM(256, quant_wgs, bits, group, mask_kind);
    case 512: return TA_BY_ELEM(512, quant_wgs, bits, group, mask_kind);
    default: return 0;
  }
}

hipError_t launch_quant_forward(const QuantArgs &a, uint32_t dim, uint32_t bits,
                                uint32_t group, hipStream_t s) {
  const int elem = a.elem;
  switch (dim) {
    case 64: return TA_BY_ELEM(64, launch_quant, a, bits, group, s);
    case 96: return TA_BY_ELEM(96, launch_quant, a, bits, group, s);
    case 128: return TA_BY_ELEM(128, launch_quant, a, bits, group, s);
    case 256: return TA_BY_ELEM(256, launch_quant, a, bits, group, s);
    case 512: return TA_BY_ELEM(512, launch_quant, a, bits, group, s);
    default: return hipErrorInvalidValue;
  }
}
#undef TA_BY_ELEM

}  // namespace ta
