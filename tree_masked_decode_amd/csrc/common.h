// common.h -- types, parameter blocks and launcher declarations shared by the
// HIP kernels of libtreeattn.so.  Internal: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ta {

// Mask sentinel of the explicit tree mask: cells at or below it exclude the
// key ("ops/tree_attention.rs", mask constants).
constexpr float kMasked = -65504.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// fp-path forward (f32 or f16 K/V).  Row r of a kv head is (node i, head in
// group hh) with r = i * group + hh; the output row is i * n_heads + h.
// ---------------------------------------------------------------------------
struct FwdArgs {
  const float *q;      // [n_heads, q_l, D] f32
  const void *k;       // [n_kv_heads, kv_capacity, D]
  const void *v;
  const float *mask;   // [q_l, mask_stride] f32, or nullptr (implicit causal)
  float *part_o;       // [nwg][nrows][D]     (nwg > 1)
  float *part_sm;      // [nwg][nrows][2]     (nwg > 1)
  float *out;          // [q_l, n_heads, D]   (nwg == 1)
  uint32_t n_heads, n_kv_heads, group, kv_seq_len, kv_capacity, q_l;
  uint32_t mask_stride;
  uint32_t nwg;        // KV splits
  uint32_t rows;       // rows per kv head = q_l * group
  uint32_t row_tiles;  // ceil(rows / rows per workgroup)
  uint32_t n_tiles;    // ceil(kv_seq_len / BN)
  uint32_t units;      // n_kv_heads * nwg
  uint32_t key_lo;     // implicit rule only: first key any row sees (window start)
  float qscale;        // scale * log2(e): logits in base-2 units (fp32 kernel)
  float scale;         // softmax scale: logits in natural units (fp16 kernel)
  // explicit mask only, or nullptr: (first, last) live key of each of
  // range_chunks key ranges (mask_range_kernel); the splits then divide the
  // tiles from the first live key's to the last live key's
  const uint32_t *range;
  uint32_t range_chunks;
  // fp16 kernel: K/V copies with the non-temporal policy (set for long K/V
  // streams, where it measured faster; short, latency-bound calls lose by it)
  uint32_t stream_nt;
};

// Live-key scan of an explicit mask: chunk c of `chunks` equal key ranges
// gets (first, last) key whose cell is live (not <= -65504) in any row, or
// (0xffffffff, 0) if none.
struct MaskRangeArgs {
  const float *mask;
  uint32_t *out;        // [chunks][2]
  uint32_t q_l, kv_seq_len, mask_stride, chunks;
};

// ---------------------------------------------------------------------------
// Quantized forward.
// ---------------------------------------------------------------------------
struct QuantArgs {
  const void *q;              // [BnQ, q_l, dim] T
  const uint32_t *kp, *vp;    // [BnKV, cap, dim/pf]
  const void *ks, *kb, *vs, *vb;  // [BnKV, cap, dim/G] T
  const float *sinks;         // [nQ] or nullptr
  const void *mask;           // T additive or nullptr
  const uint32_t *mbool;      // u32 visibility words or nullptr (never both)
  float *part_o, *part_sm;
  void *out;                  // [BnQ, q_l, dim] T
  uint64_t mask_head_stride;
  uint32_t mask_stride;
  uint32_t batch, nq, nkv, repeat, kv_seq_len, kv_capacity, q_l;
  uint32_t nwg, rows, row_tiles, n_tiles, units;
  uint32_t key_lo;            // first token the sliding window keeps (0: all)
  int elem;                   // T: 0 fp16, 1 bf16, 2 fp32
  float qscale;               // scale * log2(e)
};

// ---------------------------------------------------------------------------
// Reduce and mask construction.
// ---------------------------------------------------------------------------
struct ReduceArgs {
  const float *part_o, *part_sm;
  void *out;
  uint32_t nrows, dim, nwg;
  int out_type;   // 0 fp32, 1 fp16, 2 bf16
};

// fp32 -> bfloat16, round to nearest even (a NaN stays a quiet NaN).
__device__ inline uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int kMaxTreeNodes = 1024;
struct MaskArgs {
  int16_t parents[kMaxTreeNodes];
  float *mask;
  uint32_t q_l, kv_seq_len, mask_stride;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_forward_f32(const FwdArgs &a, uint32_t head_dim,
                              hipStream_t s);
hipError_t launch_forward_f16(const FwdArgs &a, uint32_t head_dim,
                              hipStream_t s);
hipError_t launch_quant_forward(const QuantArgs &a, uint32_t dim,
                                uint32_t bits, uint32_t group, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);
hipError_t launch_tree_mask(const MaskArgs &a, hipStream_t s);
hipError_t launch_mask_range(const MaskRangeArgs &a, hipStream_t s);

// Rows handled by one workgroup of each forward kernel (host-side shape
// planning needs them).
constexpr uint32_t kF32RowsPerWG = 16;
constexpr uint32_t kQuantRowsPerWG = 16;
uint32_t f16_tile_keys(uint32_t head_dim);
// Rows one workgroup of the fp16 forward covers for this shape (group =
// query heads per kv head; implicit = no mask buffer; mask_vec = mask rows
// 16-byte aligned).
uint32_t f16_rows_per_wg(uint32_t head_dim, uint32_t rows, uint32_t group, bool implicit,
                         bool mask_vec);
// The wide fp16 forward (one wavefront per SIMD, 48 rows each): whether it
// serves this shape, and its launcher.
bool wide_applies(uint32_t head_dim, uint32_t rows, uint32_t group, bool implicit, bool mask_vec);
uint32_t wide_rows_per_wg();
hipError_t launch_forward_wide(const FwdArgs &a, uint32_t head_dim, hipStream_t s);
uint32_t f32_tile_keys(uint32_t head_dim);
uint32_t quant_tile_keys(uint32_t dim);
// Resident workgroups per CU of the quantized kernel variant (0: no such
// variant); mask_kind 0 none, 1 additive T, 2 u32; elem 0 fp16, 1 bf16, 2 fp32.
uint32_t quant_wgs_per_cu(uint32_t dim, uint32_t bits, uint32_t group, int mask_kind,
                          int elem);

// Asynchronous global -> LDS copies: every lane moves 16 (or 4) bytes from its
// own global address to lds + 16 * lane (4 * lane), `lds` being the
// wavefront's LDS byte address (wave-uniform).  They are issued from inline
// assembly so that the compiler adds no waits of its own; the kernels wait
// with wait_vm<N>(), N = vector-memory operations the wavefront issued later
// that may stay in flight (an undercount of those is never allowed; extra
// later operations only make the wait stricter).
// (`lds` and a scalar base are wave-uniform by contract; readfirstlane puts
// them in SGPRs even where the compiler cannot prove that uniformity, which
// the "s" operands require.  The LDS address goes to M0 as an operand bound
// to that register, so the compiler writes M0 itself and knows it changed.)
__device__ inline uint32_t sgpr_u32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
// NT: the non-temporal policy, for K/V streamed once into LDS (on the 128K
// chain it raised the forward from 5.6 to 6.2 TB/s).
template <bool NT = false> __device__ inline void dma_b128(const void *g, uint32_t lds) {
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(sgpr_u32(lds)) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(sgpr_u32(lds)) : "memory");
}
__device__ inline void dma_b128_nt(const void *g, uint32_t lds) { dma_b128<true>(g, lds); }
__device__ inline void dma_b32(const void *g, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(sgpr_u32(lds)) : "memory");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (global_load_lds_dwordx4 v_off, s[base]): a loop that walks
// tiles only moves the scalar base, the per-lane offsets stay put.
// The base may reach its SGPRs through v_readfirstlane right before the
// copy, and a vector-memory read of an SGPR that a VALU instruction wrote
// needs 5 wait states, which the compiler does not count for inline
// assembly (without them the copy can read a stale base): hence the s_nop.
template <bool NT = false>
__device__ inline void dma_b128_s(const void *base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t bs = ((uint64_t)sgpr_u32((uint32_t)(b >> 32)) << 32) | sgpr_u32((uint32_t)b);
  if constexpr (NT)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff),
                 "s"((const void *)(uintptr_t)bs), "{m0}"(sgpr_u32(lds))
                 : "memory");
  else
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
                 "s"((const void *)(uintptr_t)bs), "{m0}"(sgpr_u32(lds))
                 : "memory");
}
template <int N> __device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XCD-aware workgroup numbering.  MI355X hands consecutive workgroup ids to
// its 8 XCDs in turn; every row tile of one (kv head, split) unit is placed
// on the same XCD, in consecutive slots, so their shared K/V tiles meet in
// that XCD's L2.
constexpr uint32_t kXcds = 8;
__host__ __device__ inline uint32_t grid_size(uint32_t units,
                                              uint32_t row_tiles) {
  return kXcds * ((units + kXcds - 1) / kXcds) * row_tiles;
}
__device__ inline void decode_block(uint32_t bid, uint32_t row_tiles,
                                    uint32_t &unit, uint32_t &rt) {
  uint32_t xcd = bid % kXcds;
  uint32_t slot = bid / kXcds;
  unit = (slot / row_tiles) * kXcds + xcd;
  rt = slot % row_tiles;
}

// The tiles [lo, hi) of `bn` keys that the splits divide: from tile_lo on
// (the implicit rule's window start), narrowed to the live keys of an
// explicit mask when its range scan is given (empty when no cell is live).
// Every lane of the wavefront gets the same (wave-uniform) result.
__device__ inline void split_tiles(const FwdArgs &a, uint32_t bn, uint32_t tile_lo,
                                   uint32_t &lo, uint32_t &hi) {
  lo = tile_lo;
  hi = a.n_tiles;
  if (a.range == nullptr) return;
  const uint32_t lane = threadIdx.x % kWave;
  uint32_t first = 0xffffffffu, last = 0u;
  for (uint32_t c = lane; c < a.range_chunks; c += kWave) {
    const u32x2 fl = reinterpret_cast<const u32x2 *>(a.range)[c];
    if (fl[0] != 0xffffffffu) {
      first = min(first, fl[0]);
      last = max(last, fl[1]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    first = min(first, (uint32_t)__shfl_xor((int)first, o));
    last = max(last, (uint32_t)__shfl_xor((int)last, o));
  }
  first = __builtin_amdgcn_readfirstlane(first);
  last = __builtin_amdgcn_readfirstlane(last);
  if (first == 0xffffffffu) {
    lo = hi = tile_lo;
    return;
  }
  lo = max(lo, first / bn);
  hi = min(hi, last / bn + 1u);
  if (hi < lo) hi = lo;
}

// Cross-lane maxima in registers (no LDS round trip): DPP within rows of 16
// lanes, v_permlane16_swap / v_permlane32_swap across rows.
// max over lanes l ^ 16 (rows 0 + 1, 2 + 3 of the wavefront)
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max over lanes l ^ 32 (the two halves of the wavefront)
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max over the 32 lanes of the lane's half-wave
__device__ inline float half_wave_max(float x) {
  int v = __float_as_int(x);
  // quad_perm [1,0,3,2] and [2,3,0,1]: lanes l ^ 1, l ^ 2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false)));
  v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false)));
  v = __float_as_int(x);
  // row_ror 4 and 8: the four quads of a 16-lane row
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false)));
  v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false)));
  return max_xor16(x);
}

// Q'^T operand of one 32-dim step for a 16-row block: lane (n, gp) needs
// dims 8gp .. 8gp+7 of its row n as fp16 (times sc).  The global loads take
// dims 4gp .. 4gp+3 and 16+4gp .. 16+4gp+3 instead, so that the four lanes
// of a row read 64 contiguous bytes per instruction; two swaps then regroup
// the halves across the four 16-lane rows (gp): after the 32-lane swap the
// rows of (x, y) hold (A0 A1 B0 B1, A2 A3 B2 B3), after the 16-lane swap
// (A0 A2 B0 B2, A1 A3 B1 B3) -- lane gp's dims 8gp .. 8gp+3 and +4 .. +7.
__device__ inline floatx4 q_fragment(const float *qrow_step, uint32_t gp, float sc) {
  floatx4 a = *reinterpret_cast<const floatx4 *>(qrow_step + 4 * gp);
  floatx4 b = *reinterpret_cast<const floatx4 *>(qrow_step + 16 + 4 * gp);
  a *= sc;
  b *= sc;
  const half4_t ha = {(half_t)a[0], (half_t)a[1], (half_t)a[2], (half_t)a[3]};
  const half4_t hb = {(half_t)b[0], (half_t)b[1], (half_t)b[2], (half_t)b[3]};
  const u32x2 ua = __builtin_bit_cast(u32x2, ha), ub = __builtin_bit_cast(u32x2, hb);
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto s32 = __builtin_amdgcn_permlane32_swap(ua[k], ub[k], false, false);
    const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
    r[k] = s16[0];
    r[2 + k] = s16[1];
  }
  return __builtin_bit_cast(floatx4, r);
}

// Balanced contiguous split of n_tiles tiles into nwg ranges.
__device__ inline void split_range(uint32_t n_tiles, uint32_t nwg, uint32_t s,
                                   uint32_t &t0, uint32_t &t1) {
  t0 = (uint32_t)(((uint64_t)n_tiles * s) / nwg);
  t1 = (uint32_t)(((uint64_t)n_tiles * (s + 1)) / nwg);
}

}  // namespace ta
