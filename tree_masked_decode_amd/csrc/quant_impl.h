// quant_impl.h -- attention over an affine-quantized (4/8-bit) K/V cache:
// the kernel templates.  Each quant_d<dim>.hip instantiates one head dim,
// so that the variants compile in parallel; quant.hip dispatches.
//
// "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0): element d of a token
// is scale_g * code + bias_g with the code taken little-end first from a
// 32-bit word, a query head maps to kv stream q_idx / repeat, an optional
// sink is a virtual key with raw logit sinks[h] and value 0, and an optional
// additive f16 mask biases the logits.  That page runs one 32-lane group per
// query over all tokens; here one wavefront takes up to 16 query rows that
// share a kv stream (heads of the GQA group x tree nodes) over one KV split,
// and the contractions run on v_mfma_f32_16x16x32_f16 with the codes as exact
// fp16 integers.  The affine map is factored out of the contractions:
//
//   q.k_t = sum_g s_tg * (sum_{d in g} q_d c_td) + b_tg * (sum_{d in g} q_d)
//   o_d   = sum_t (p_t s^v_tg) c^v_td + sum_t p_t b^v_tg,      g = group of d
//
// so K codes feed the score MFMA directly (one accumulator per group; Q is
// used exactly as given in fp16 and the attention scale is applied to the
// fp32 dot products), and the PV MFMA takes codes as A and p*scale_g as B
// (one B operand per group, split into an fp16 hi/lo pair so the product
// keeps fp32-like precision); the bias terms are short per-row dot products
// on the VALU.
//
// Memory pipeline: every tile of 32 keys -- K words, V words, the four
// scale/bias slices and the mask cells of the workgroup's rows -- is copied
// global -> LDS with coalesced global_load_lds instructions into a ring of NS
// stages, NS - 1 tiles ahead; the workgroup is one wavefront, so waits are
// its own vmcnt counts and no barrier is needed.  The arithmetic then reads
// the tile from LDS.
//
// Codes become fp16 by OR-ing them into the mantissa of 1024.0 (0x6400) and
// subtracting 1024 (exact).  K codes are read straight into MFMA operands
// (a 32-bit word holds 8 or 4 consecutive dims of one token, and the order of
// the dims inside an MFMA step is free as long as Q uses the same order).
// V must be transposed (the PV operand wants 8 tokens of one dim per lane),
// so each wavefront bounces its V words through LDS as [word][token].
#pragma once

#include "common.h"

namespace ta {

namespace {

constexpr int kThreads = 64;   // one wavefront per workgroup
constexpr int BN = 32;         // keys per tile
constexpr float kLazyQ = 8.0f; // lazy-rescale threshold of the running max (base 2)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ inline uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Two codes (already in bits 0..bits-1 of x0 / x1's lane slots) -> (c0, c1)
// as exact fp16: OR into 1024.0's mantissa, then subtract 1024.
__device__ inline uint32_t codes_to_h2(uint32_t packed_pair) {
  half2_t h = as_h2(packed_pair | 0x64006400u);
  const half2_t k1024 = {(half_t)1024.0f, (half_t)1024.0f};
  return as_u(h - k1024);
}
// The same from an unmasked word: (x & m) | 0x64006400 is one v_and_or_b32
// when the nibble/byte mask m sits in a register (it is kept out of the
// compiler's sight so that it is not folded back into a second literal).
__device__ inline uint32_t masked_codes_to_h2(uint32_t x, uint32_t m) {
  half2_t h = as_h2((x & m) | 0x64006400u);
  const half2_t k1024 = {(half_t)1024.0f, (half_t)1024.0f};
  return as_u(h - k1024);
}
// The same for codes in bits 4..7 of each half, (x & (m << 4)): 1024 + 16c
// as fp16, mapped to c exactly by one packed fma, (y / 16 - 64).
__device__ inline uint32_t masked_hi_codes_to_h2(uint32_t x, uint32_t m4) {
  const half2_t h = as_h2((x & m4) | 0x64006400u);
  const half2_t s = {(half_t)0.0625f, (half_t)0.0625f};
  const half2_t b = {(half_t)-64.0f, (half_t)-64.0f};
  return as_u(h * s + b);
}
template <int BITS> __device__ inline uint32_t code_pair_mask() {
  uint32_t m;
  if (BITS == 4)
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m));
  else
    asm volatile("v_mov_b32 %0, 0x00ff00ff" : "=v"(m));
  return m;
}

// 8 slots of one MFMA step from the lane's words.  4-bit: one word, slots
// [c0 c4 c1 c5 c2 c6 c3 c7].  8-bit: two words, slots [c0 c2 c1 c3] each.
template <int BITS>
__device__ inline half8_t word_codes(const uint32_t *w, uint32_t m) {
  u32x4 r;
  if (BITS == 4) {
    // odd nibbles in place (no shift); one shift brings nibbles 2, 3 (and
    // 6, 7) down to bits 0..7
    const uint32_t w8 = w[0] >> 8;
    r[0] = masked_codes_to_h2(w[0], m);
    r[1] = masked_hi_codes_to_h2(w[0], m << 4);
    r[2] = masked_codes_to_h2(w8, m);
    r[3] = masked_hi_codes_to_h2(w8, m << 4);
  } else {
    r[0] = masked_codes_to_h2(w[0], m);
    r[1] = masked_codes_to_h2(w[0] >> 8, m);
    r[2] = masked_codes_to_h2(w[1], m);
    r[3] = masked_codes_to_h2(w[1] >> 8, m);
  }
  return __builtin_bit_cast(half8_t, r);
}

// Element types of the queries, scales, biases, float mask and output
// ("ffai/flash_quantized_sdpa.rs" kernels are generic in that type T).
enum { kF16 = 0, kBF16 = 1, kF32 = 2 };
template <int ET> struct Elem {
  static constexpr int SZ = ET == kF32 ? 4 : 2;   // bytes
};
// Element i of a T array (global memory, LDS or registers), as fp32.
template <int ET> __device__ inline float elem_f32(const void *base, size_t i) {
  if (ET == kF32) return reinterpret_cast<const float *>(base)[i];
  const uint16_t b = reinterpret_cast<const uint16_t *>(base)[i];
  if (ET == kBF16) return __uint_as_float((uint32_t)b << 16);
  return (float)__builtin_bit_cast(half_t, b);
}
template <int ET> __device__ inline void store_elem(void *base, size_t i, float x) {
  if (ET == kF32)
    reinterpret_cast<float *>(base)[i] = x;
  else if (ET == kBF16)
    reinterpret_cast<uint16_t *>(base)[i] = f32_to_bf16(x);
  else
    reinterpret_cast<half_t *>(base)[i] = (half_t)x;
}

// Dim index of slot j of a step whose first word is w0 (see word_codes).
template <int BITS>
__device__ inline uint32_t slot_dim(uint32_t w0, int j) {
  if (BITS == 4) {
    const int pi4[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    return 8u * w0 + pi4[j];
  }
  const int pi8[4] = {0, 2, 1, 3};
  return 4u * (w0 + (uint32_t)(j >> 2)) + pi8[j & 3];
}

template <int DIM, int BITS, int G, int ET = kF16>
struct QShape {
  static constexpr int ESZ = Elem<ET>::SZ;     // bytes of a scale / bias
  static constexpr int EPW = 4 / ESZ;          // of them per 32-bit word
  static constexpr int WPK = DIM * BITS / 32;  // 32-bit words per token row
  static constexpr int NG = DIM / G;           // scale groups per token
  static constexpr int WPS = BITS / 4;         // words per MFMA step per lane
  static constexpr int SPG = G / 32;           // MFMA steps per group
  static constexpr int RUN = SPG * WPS;        // lane's contiguous words per group
  static constexpr int GW = G * BITS / 32;     // words per group
  static constexpr int STEPS = DIM / 32;       // score MFMA steps
  static constexpr int DB = DIM / 16;          // PV output blocks
  static constexpr int VTOT = BN * WPK / 4;            // V 16-byte chunks of a tile
  static constexpr int VCH = (VTOT + kThreads - 1) / kThreads;  // ... per lane
  static constexpr int RS = BN + 4;            // LDS row stride (words)
  static constexpr int SBW = 4 * NG / EPW;     // u32 words of 4 keys' scales
  static_assert(VCH >= 1, "tile too small");
  static_assert(RUN * 4 == GW, "lane runs must tile a group");
  // LDS stage: K words, V words, K scales, K biases, V scales, V biases, mask
  static constexpr int KT = BN * WPK * 4;              // bytes of a K (or V) tile
  static constexpr int KT_I = (KT + 1023) / 1024;      // 16-byte-per-lane copies
  // bytes of the last copy when a tile is not a whole number of copies
  // (dim 96 at 4 bits: 1.5 KB); its lanes past that leave it alone
  static constexpr int KT_TAIL = KT % 1024;
  static constexpr int SBB = BN * NG * ESZ;            // bytes of one scale/bias slice
  // the four slices back to back (4 SBB = 128 NG ESZ bytes) move in SB_I
  // copies of SB_W bytes per lane; lane l of copy i takes byte SB_W (64 i +
  // l) of that region, i.e. slice SB_W (64 i + l) / SBB.  16-byte copies when
  // a token's values fill whole 16-byte chunks (so that a chunk never
  // straddles two tokens) and the region is whole copies, else 4-byte ones.
  static constexpr bool SB_WIDE = (NG * ESZ) % 16 == 0 && (4 * SBB) % 1024 == 0;
  static constexpr int SB_W = SB_WIDE ? 16 : 4;
  static constexpr int SB_I = 4 * SBB / (64 * SB_W);
  static constexpr int SBP = SBB;
  static constexpr int VL = WPK * RS * 4;              // V transpose area
  static_assert(WPK % 4 == 0, "token rows of whole 16-byte chunks");
};

// Mask modes: none (implicit causal); an additive mask of T cells in
// 16-byte copies (row starts and kv_seq_len multiples of 16 / sizeof(T)
// cells), 4-byte copies (multiples of 4 / sizeof(T)) or per-lane register
// loads (any alignment); or a u32 visibility mask
// ("ffai/flash_quantized_sdpa.rs", bool-mask macro) in 16-byte or 4-byte
// copies.  A copy mode moves the 16 rows x 32 cells of a tile, row r at byte
// 32 r CB (CB = cell bytes), lane l of copy i taking row RPC i + l / LPR and
// cells CPL (l % LPR) .. (CPL cells per lane, LPR lanes per row, RPC rows
// per copy).
enum { kMaskNone = 0, kMaskB128 = 1, kMaskB32 = 2, kMaskReg = 3, kMaskBool = 4,
       kMaskBoolB128 = 5 };
template <int MM, int ET> struct MaskGeom {
  static constexpr bool BOOL = MM == kMaskBool || MM == kMaskBoolB128;
  static constexpr bool DMA = BOOL || MM == kMaskB128 || MM == kMaskB32;
  static constexpr bool WIDE = MM == kMaskB128 || MM == kMaskBoolB128;  // 16-byte copies
  static constexpr int CB = BOOL ? 4 : Elem<ET>::SZ;       // cell bytes
  static constexpr int CPL = (WIDE ? 16 : 4) / CB;         // cells per lane
  static constexpr int LPR = BN / CPL;                     // lanes per row
  static constexpr int RPC = kThreads / LPR;               // rows per copy
  static constexpr int NC = DMA ? 16 / RPC : 0;            // copies per tile
  static constexpr int BYTES = DMA ? 16 * BN * CB : 0;     // per stage
  static constexpr int STEP = WIDE ? 1024 : 256;           // LDS bytes per copy
  static_assert(!DMA || (RPC * LPR == kThreads && NC * RPC == 16), "mask copy geometry");
};
template <int DIM, int BITS, int G, int MM, int ET> struct QStage {
  using S = QShape<DIM, BITS, G, ET>;
  using MG = MaskGeom<MM, ET>;
  static constexpr int MASK_I = MG::NC;
  static constexpr int M_BYTES = MG::BYTES;
  static constexpr int BYTES = 2 * S::KT + 4 * S::SBP + M_BYTES;
  static constexpr int PER_TILE = 2 * S::KT_I + S::SB_I + MASK_I;
  // At dim <= 128 the registers allow three one-wavefront workgroups per
  // SIMD, twelve per CU, so a workgroup keeps within 160 KB / 12 of LDS
  // there (two stages; measured faster than three stages at eight per CU);
  // wider heads run fewer.
  static constexpr int BUDGET = DIM <= 128 ? 160 * 1024 / 12 : 48 * 1024;
  // (and a wavefront's copy counter tracks at most 63 copies in flight)
  static constexpr int NS = (3 * BYTES + S::VL <= BUDGET && 2 * PER_TILE <= 63) ? 3 : 2;
  static constexpr int LDS = NS * BYTES + S::VL;
  static_assert(PER_TILE * (NS - 1) <= 63, "vmcnt range");
};

// Word index of (group g, step-in-group sub, part) for lane group gp.
template <int DIM, int BITS, int G>
__device__ inline uint32_t step_word(int g, int sub, uint32_t gp) {
  using S = QShape<DIM, BITS, G>;
  return (uint32_t)(g * S::GW) + gp * S::RUN + (uint32_t)(sub * S::WPS);
}

// SR (small R): the workgroup's live rows number at most 4 (one decode
// query per head of a GQA group of 4, say).  The score epilogue and softmax
// then run with each lane on one key of two rows (lane & 31, rows
// 2 (lane >> 5) + 0..1) instead of on 8 keys of one MFMA row, 12 of whose 16
// rows would be dead; scores and the p * scale operands pass through LDS.
template <int DIM, int BITS, int G, int MM, int ET, int SR>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantArgs a) {
  using S = QShape<DIM, BITS, G, ET>;
  using ST = QStage<DIM, BITS, G, MM, ET>;
  using MG = MaskGeom<MM, ET>;
  constexpr bool IMPLICIT = MM == kMaskNone;
  constexpr int NG = S::NG, STEPS = S::STEPS, DB = S::DB, NS = ST::NS;
  // SBL: the scales and biases of a tile (8 SBW registers) stay in LDS
  // where they would not fit beside the rest (many groups per token); the
  // stage is then refilled after the tile's arithmetic instead of before.
  constexpr bool SBL = !SR && (S::SBW > 8 || DIM >= 512);
  // FUSE (head dim 512): scores folded per group, P operands built per group
  constexpr bool FUSE = !SR && DIM >= 512;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) char *)lds);
  uint32_t *vlds = reinterpret_cast<uint32_t *>(lds + NS * ST::BYTES);

  uint32_t unit, rt;
  decode_block(blockIdx.x, a.row_tiles, unit, rt);
  if (unit >= a.units) return;
  const uint32_t kv = unit / a.nwg;          // kv stream: b * nkv + hk
  const uint32_t split = unit % a.nwg;
  const uint32_t lane = threadIdx.x;
  const uint32_t n = lane & 15u, gp = lane >> 4;

  const uint32_t gr = rt * 16u + n;          // row: node * repeat + head-in-group
  const bool valid = gr < a.rows;
  const uint32_t node = valid ? gr / a.repeat : 0u;
  const uint32_t qidx = kv * a.repeat + (valid ? gr % a.repeat : 0u);
  // SR roles: key kl of the tile, rows sr_row[0..1] = 2 rp + 0..1 (rt is 0)
  const uint32_t kl = lane & 31u, rp = lane >> 5;
  uint32_t sr_row[2];
  bool sr_valid[2];
  uint32_t sr_qidx[2];
  int64_t sr_last[2];
  size_t sr_mrow[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    sr_row[s2] = 2u * rp + (uint32_t)s2;
    sr_valid[s2] = SR && sr_row[s2] < a.rows;
    const uint32_t nd = sr_valid[s2] ? sr_row[s2] / a.repeat : 0u;
    sr_qidx[s2] = kv * a.repeat + (sr_valid[s2] ? sr_row[s2] % a.repeat : 0u);
    sr_last[s2] = (int64_t)a.kv_seq_len - (int64_t)a.q_l + (int64_t)nd;
    sr_mrow[s2] = (size_t)sr_qidx[s2] * a.mask_head_stride + (size_t)nd * a.mask_stride;
  }

  // ---- Q in the K operand's slot order; the attention scale is applied
  // to the fp32 dot products afterwards.  fp16 Q is used exactly; bf16 Q
  // becomes fp16 (exact for magnitudes in fp16's normal range); fp32 Q is an
  // fp16 hi + lo pair (two matrix instructions per step). ----
  // (loaded once the first tiles' copies are on their way, so that the two
  // memory latencies overlap; a row past the end reads row 0 of its kv
  // stream's first query head, in bounds, and is zeroed)
  constexpr bool QLO = ET == kF32;
  half8_t qf[STEPS], qfl[QLO ? STEPS : 1];
  float qsum[NG];
  auto load_q = [&]() {
#pragma unroll
  for (int g = 0; g < NG; ++g) qsum[g] = 0.0f;
  {
    const size_t qrow = ((size_t)qidx * a.q_l + node) * DIM;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int sub = 0; sub < S::SPG; ++sub) {
        const uint32_t w0 = step_word<DIM, BITS, G>(g, sub, gp);
        half8_t f, fl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xr = elem_f32<ET>(a.q, qrow + slot_dim<BITS>(w0, j));
          const float x = valid ? xr : 0.0f;
          f[j] = (half_t)x;
          if (QLO) fl[j] = (half_t)(x - (float)f[j]);
          qsum[g] += ET == kF16 ? (float)f[j] : x;
        }
        qf[g * S::SPG + sub] = f;
        if (QLO) qfl[(g * S::SPG + sub) % (QLO ? STEPS : 1)] = fl;
      }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    qsum[g] += __shfl_xor(qsum[g], 16);
    qsum[g] += __shfl_xor(qsum[g], 32);
  }
  };

  const size_t kvrow0 = (size_t)kv * a.kv_capacity;
  const uint32_t *KP = a.kp + kvrow0 * S::WPK;
  const uint32_t *VP = a.vp + kvrow0 * S::WPK;
  constexpr int ESZ = S::ESZ;
  const char *KS = reinterpret_cast<const char *>(a.ks) + kvrow0 * NG * ESZ;
  const char *KB = reinterpret_cast<const char *>(a.kb) + kvrow0 * NG * ESZ;
  const char *VS = reinterpret_cast<const char *>(a.vs) + kvrow0 * NG * ESZ;
  const char *VB = reinterpret_cast<const char *>(a.vb) + kvrow0 * NG * ESZ;
  const size_t mrow = (size_t)qidx * a.mask_head_stride + (size_t)node * a.mask_stride;
  const int64_t causal_last = (int64_t)a.kv_seq_len - (int64_t)a.q_l + (int64_t)node;
  const uint32_t L = a.kv_seq_len;
  // sliding window ("ffai/flash_quantized_sdpa.rs" causal / sliding-window
  // gate): tokens below key_lo are never attended; the splits cover the
  // tiles from the one that holds key_lo
  const uint32_t klo = a.key_lo;
  const uint32_t tile_lo = klo / BN;

  // ---- per-tile registers ----
  struct Tile {
    uint32_t kw[2][SBL ? 1 : NG][S::RUN];   // K words: key 16kb+n, group g (SBL: in LDS)
    uint32_t ksb[2][2][SBL ? 1 : S::SBW];   // K scales/biases: keys 16kb+4gp..+3, all groups
    uint32_t vsb[2][2][SBL ? 1 : S::SBW];   // V scales/biases: keys F(gp, 4h..4h+3)
    const char *stp;              // SBL: the tile's LDS stage
    u32x4 vw[SBL ? 1 : S::VCH];   // V words for the LDS transpose (SBL: in LDS)
    float m[2][4];                // mask cells (row n, keys 16kb+4gp+j)
    // SR: scale and bias of the lane's key kl per group, and its mask cells
    // of rows 2 rp + 0..1
    float ksr[SR ? NG : 1], kbr[SR ? NG : 1], vsr[SR ? NG : 1], vbr[SR ? NG : 1];
    float mr[2];
  };
  // ---- copies of tile t into stage (t - t0) % NS ----
  // Keys past kv_seq_len re-read row L - 1 (or the word that holds it), so
  // that nothing outside the buffers is read; they are excluded below.
  uint32_t t0, t1;
  split_range(a.n_tiles - tile_lo, a.nwg, split, t0, t1);
  t0 += tile_lo;
  t1 += tile_lo;
  const uint32_t t_first = t0;
  auto stage_off = [&](uint32_t t) -> uint32_t { return ((t - t_first) % NS) * ST::BYTES; };
  // Per-lane source pointers of the copies: a tile's K words, V words and
  // each scale/bias slice are contiguous in memory, so every copy of a full
  // tile is the lane's pointer plus a wave-uniform tile offset.  A tile that
  // reaches past kv_seq_len takes the clamped path instead.
  const char *kp_l = reinterpret_cast<const char *>(KP) + 16u * lane;
  const char *vp_l = reinterpret_cast<const char *>(VP) + 16u * lane;
  const char *sarr[4] = {KS, KB, VS, VB};
  const char *sb_l[S::SB_I];
#pragma unroll
  for (int i = 0; i < S::SB_I; ++i) {
    const uint32_t o = S::SB_W * (64u * i + lane);
    sb_l[i] = sarr[o / S::SBB] + o % S::SBB;
  }
  // mask copies: the row each copy gives this lane, as a byte pointer to its
  // first cell (rows past the end reuse the workgroup's row 0)
  const char *mbase = MG::BOOL ? reinterpret_cast<const char *>(a.mbool)
                               : reinterpret_cast<const char *>(a.mask);
  const char *m_l[MG::NC > 0 ? MG::NC : 1];
  if (MG::DMA) {
#pragma unroll
    for (int i = 0; i < MG::NC; ++i) {
      uint32_t g2 = rt * 16u + MG::RPC * i + lane / MG::LPR;
      if (g2 >= a.rows) g2 = rt * 16u;
      const uint32_t q2 = kv * a.repeat + g2 % a.repeat;
      m_l[i] = mbase + ((size_t)q2 * a.mask_head_stride +
                        (size_t)(g2 / a.repeat) * a.mask_stride) * MG::CB;
    }
  }
  auto issue = [&](uint32_t t) {
    const uint32_t key0 = t * BN;
    const uint32_t sb = lds0 + stage_off(t);
    if (key0 + BN <= L) {
      const size_t kvo = (size_t)key0 * (4u * S::WPK);
#pragma unroll
      for (int i = 0; i < S::KT_I; ++i) {
        if (S::KT_TAIL == 0 || i + 1 < S::KT_I || 16u * lane < (uint32_t)S::KT_TAIL) {
          dma_b128(kp_l + kvo + 1024u * i, sb + 1024u * i);
          dma_b128(vp_l + kvo + 1024u * i, sb + S::KT + 1024u * i);
        }
      }
      const size_t so = (size_t)key0 * NG * ESZ;
#pragma unroll
      for (int i = 0; i < S::SB_I; ++i) {
        if (S::SB_WIDE)
          dma_b128(sb_l[i] + so, sb + 2u * S::KT + 1024u * i);
        else
          dma_b32(sb_l[i] + so, sb + 2u * S::KT + 256u * i);
      }
    } else {
      // keys past kv_seq_len re-read row L - 1 (or the word that holds it)
#pragma unroll
      for (int i = 0; i < S::KT_I; ++i) {
        const uint32_t o = 1024u * i + 16u * lane;
        if (S::KT_TAIL == 0 || o < (uint32_t)S::KT) {
          uint32_t key = key0 + o / (4u * S::WPK);
          if (key >= L) key = L - 1u;
          const size_t go = (size_t)key * (4u * S::WPK) + o % (4u * S::WPK);
          dma_b128(reinterpret_cast<const char *>(KP) + go, sb + 1024u * i);
          dma_b128(reinterpret_cast<const char *>(VP) + go, sb + S::KT + 1024u * i);
        }
      }
#pragma unroll
      for (int i = 0; i < S::SB_I; ++i) {
        const uint32_t o = S::SB_W * (64u * i + lane);
        const uint32_t e = (o % S::SBB) / ESZ;              // first element of the copy
        const uint32_t key = key0 + e / NG;
        size_t el = (size_t)key * NG + e % NG;                // element of the stream
        // past kv_seq_len: any whole copy inside the stream's first L tokens
        // (never used).  A 4-byte copy of 2-byte values starts on an even
        // element, so the last such pair is elements (L NG - 2) & ~1 and up:
        // with an odd count of values per token, the last token's last value
        // would otherwise pair with token L's first, past a buffer that holds
        // exactly L tokens.
        if (key >= L)
          el = (ESZ == 2 && !S::SB_WIDE) ? (((size_t)L * NG >= 2 ? (size_t)L * NG - 2 : 0) & ~(size_t)1)
                                         : (size_t)(L - 1u) * NG + e % NG;
        const char *g = sarr[o / S::SBB] + el * ESZ;
        if (S::SB_WIDE)
          dma_b128(g, sb + 2u * S::KT + 1024u * i);
        else
          dma_b32(g, sb + 2u * S::KT + 256u * i);
      }
    }
    if (MG::DMA) {
      // past kv_seq_len (a multiple of CPL in these modes): re-read the
      // chunk that ends at cell L - 1 (never used)
      uint32_t cell = key0 + MG::CPL * (lane % MG::LPR);
      if (cell >= L) cell = L - MG::CPL;
#pragma unroll
      for (int i = 0; i < MG::NC; ++i) {
        const char *g = m_l[i] + (size_t)cell * MG::CB;
        const uint32_t la = sb + 2u * S::KT + 4u * S::SBP + MG::STEP * i;
        if (MG::WIDE)
          dma_b128(g, la);
        else
          dma_b32(g, la);
      }
    }
  };
  // wait until tile t has landed; `after` later tiles (0 .. NS - 1) may
  // stay in flight
  auto wait_tile = [&](uint32_t after) {
    if (NS >= 3 && after >= 2)
      wait_vm<(NS >= 3 ? 2 * ST::PER_TILE : 0)>();
    else if (after >= 1)
      wait_vm<ST::PER_TILE>();
    else
      wait_vm<0>();
  };
  auto load_tile = [&](uint32_t t, Tile &T) {
    const uint32_t key0 = t * BN;
    const char *st = lds + stage_off(t);
    T.stp = st;
    const uint32_t *Kl = reinterpret_cast<const uint32_t *>(st);
    const uint32_t *Vl = reinterpret_cast<const uint32_t *>(st + S::KT);
    const uint32_t *SBl[4];
#pragma unroll
    for (int arr = 0; arr < 4; ++arr)
      SBl[arr] = reinterpret_cast<const uint32_t *>(st + 2 * S::KT + arr * S::SBP);
    const char *Ml = st + 2 * S::KT + 4 * S::SBP;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t kr = 16u * kb + n;   // key within the tile
#pragma unroll
      for (int g = 0; g < (SBL ? 0 : NG); ++g)
#pragma unroll
        for (int r = 0; r < S::RUN; ++r)
          T.kw[kb][g][r] = Kl[kr * S::WPK + g * S::GW + gp * S::RUN + r];
      if constexpr (SR) continue;
      // scales/biases of keys 16kb + 4gp + 0..3 (K side) and
      // 16h + 4gp + 0..3 (V side, the keys of B-operand half h)
      const uint32_t k4 = 16u * kb + 4u * gp;
#pragma unroll
      for (int w = 0; w < (SBL ? 0 : S::SBW); ++w) {
        const uint32_t wi = (k4 * NG) / S::EPW + w;
        T.ksb[kb][0][w] = SBl[0][wi];
        T.ksb[kb][1][w] = SBl[1][wi];
        T.vsb[kb][0][w] = SBl[2][wi];
        T.vsb[kb][1][w] = SBl[3][wi];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kk = key0 + k4 + j;
        float mv;
        const bool in = valid && kk < L && kk >= klo;
        if (IMPLICIT) {
          mv = (in && (int64_t)kk <= causal_last) ? 0.0f : kMasked;
        } else if (MM == kMaskReg) {
          mv = in ? elem_f32<ET>(a.mask, mrow + kk) : kMasked;
        } else if (MG::BOOL) {
          mv = (in && reinterpret_cast<const uint32_t *>(Ml)[n * BN + k4 + j] != 0u) ? 0.0f
                                                                                 : kMasked;
        } else {
          const float x = elem_f32<ET>(Ml, n * BN + k4 + j);  // always in the stage
          mv = in ? x : kMasked;
        }
        T.m[kb][j] = mv;
      }
    }
    if constexpr (SR) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        T.ksr[g] = elem_f32<ET>(SBl[0], kl * NG + g);
        T.kbr[g] = elem_f32<ET>(SBl[1], kl * NG + g);
        T.vsr[g] = elem_f32<ET>(SBl[2], kl * NG + g);
        T.vbr[g] = elem_f32<ET>(SBl[3], kl * NG + g);
      }
      const uint32_t kk = key0 + kl;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bool in = sr_valid[s2] && kk < L && kk >= klo;
        const uint32_t r = sr_row[s2];
        float mv;
        if (IMPLICIT) {
          mv = (in && (int64_t)kk <= sr_last[s2]) ? 0.0f : kMasked;
        } else if (MM == kMaskReg) {
          mv = in ? elem_f32<ET>(a.mask, sr_mrow[s2] + kk) : kMasked;
        } else if (MG::BOOL) {
          mv = (in && reinterpret_cast<const uint32_t *>(Ml)[r * BN + kl] != 0u) ? 0.0f
                                                                               : kMasked;
        } else {
          const float x = elem_f32<ET>(Ml, r * BN + kl);  // always in the stage
          mv = in ? x : kMasked;
        }
        T.mr[s2] = mv;
      }
    }
#pragma unroll
    for (int u = 0; u < (SBL ? 0 : S::VCH); ++u) {
      const uint32_t c = lane + kThreads * u;
      const uint32_t key = c / (S::WPK / 4), q4 = c % (S::WPK / 4);
      T.vw[u] = (S::VTOT % kThreads == 0 || c < (uint32_t)S::VTOT)
                    ? *reinterpret_cast<const u32x4 *>(Vl + key * S::WPK + 4 * q4)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // V words -> LDS [word][position]; position of key (16h + 4g4 + j) is
  // 8*g4 + 4h + j, so that lane group gp later reads its 8 keys contiguously.
  auto store_v = [&](const Tile &T) {
#pragma unroll
    for (int u = 0; u < S::VCH; ++u) {
      const uint32_t c = lane + kThreads * u;
      if (S::VTOT % kThreads != 0 && c >= (uint32_t)S::VTOT) continue;
      const uint32_t key = c / (S::WPK / 4), q4 = c % (S::WPK / 4);
      const uint32_t pos = 8u * ((key & 15u) >> 2) + 4u * (key >> 4) + (key & 3u);
      // (SBL: straight from the stage, which stays until the tile is done)
      const u32x4 vv = SBL ? *reinterpret_cast<const u32x4 *>(
                                 reinterpret_cast<const uint32_t *>(T.stp + S::KT) +
                                 key * S::WPK + 4 * q4)
                           : T.vw[SBL ? 0 : u];
#pragma unroll
      for (int e = 0; e < 4; ++e) vlds[(4 * q4 + e) * S::RS + pos] = vv[e];
    }
  };

  // ---- online-softmax state of the lane's row ----
  float Mrow = -INFINITY, Srow = 0.0f;
  float pb[NG];                     // sum_t p_t * vbias_tg (lane's keys)
  // SR state of rows sr_row[0..1]: reference max (the same in every lane of
  // the half-wave), and this lane's shares of S and of the bias sums
  float srM[2] = {-INFINITY, -INFINITY}, srS[2] = {0.0f, 0.0f};
  float srB[2][SR ? NG : 1];
  float sr_qs[2][SR ? NG : 1];      // Q's group sums of the lane's rows
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int g = 0; g < (SR ? NG : 1); ++g) srB[s2][g] = 0.0f;
  float *sx = reinterpret_cast<float *>(lds + ST::LDS);                       // [NG][4][BN]
  half_t *pw = reinterpret_cast<half_t *>(lds + ST::LDS + NG * 4 * BN * 4);  // [NG][4][BN]
  half_t *pwl = pw + NG * 4 * BN;                                            // lo halves
#pragma unroll
  for (int g = 0; g < NG; ++g) pb[g] = 0.0f;
  floatx4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (a.sinks != nullptr && split == 0 && valid) {
    // the sink: a virtual key with raw logit sinks[h] and value zero
    Mrow = a.sinks[qidx % a.nq] * kLog2e;
    Srow = (gp == 0) ? 1.0f : 0.0f;
  }
  if (SR && a.sinks != nullptr && split == 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      if (sr_valid[s2]) {
        srM[s2] = a.sinks[sr_qidx[s2] % a.nq] * kLog2e;
        srS[s2] = (kl == 0u) ? 1.0f : 0.0f;
      }
  }

  const uint32_t cmask = code_pair_mask<BITS>();
  // V code extraction, two keys at a time: v_perm_b32 moves the byte that
  // holds the lane's code (dim 16db + n) out of each key's word into bytes 0
  // and 2; the code mask and 1024.0's exponent turn them into an fp16 pair
  // 1024 + c (low nibble or byte) or 1024 + 16c (high nibble), and one
  // packed fma maps that to c exactly: (y - 1024) or (y / 16 - 64).
  const uint32_t vbyte = (BITS == 4) ? ((n & 7u) >> 1) : (n & 3u);
  const uint32_t vsel = vbyte | (0x0Cu << 8) | ((4u + vbyte) << 16) | (0x0Cu << 24);
  const bool vhi = BITS == 4 && (n & 1u) != 0u;
  const uint32_t vcm = (BITS == 4) ? (vhi ? 0x00F000F0u : 0x000F000Fu) : 0x00FF00FFu;
  const half2_t vmul = vhi ? half2_t{(half_t)0.0625f, (half_t)0.0625f}
                           : half2_t{(half_t)1.0f, (half_t)1.0f};
  const half2_t vadd = vhi ? half2_t{(half_t)-64.0f, (half_t)-64.0f}
                           : half2_t{(half_t)-1024.0f, (half_t)-1024.0f};

  auto compute = [&](const Tile &T) {
    // scores, one accumulator per scale group.  FUSE (wide heads): each
    // group's accumulators are folded into the running logits xf as soon as
    // its matrix instructions are done -- the same operations in the same
    // order as the epilogue below, with one group's registers live at a time
    floatx4 sacc[FUSE ? 1 : NG][2];
    float xf[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int gs = FUSE ? 0 : g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[gs][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sub = 0; sub < S::SPG; ++sub) {
          const uint32_t *kwp =
              SBL ? reinterpret_cast<const uint32_t *>(T.stp) +
                        (16u * kb + n) * S::WPK + g * S::GW + gp * S::RUN + sub * S::WPS
                  : &T.kw[kb][SBL ? 0 : g][sub * S::WPS];
          half8_t kf = word_codes<BITS>(kwp, cmask);
          sacc[gs][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[g * S::SPG + sub],
                                                                sacc[gs][kb], 0, 0, 0);
          if (QLO)
            sacc[gs][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                kf, qfl[(g * S::SPG + sub) % (QLO ? STEPS : 1)], sacc[gs][kb], 0, 0, 0);
        }
      }
      if constexpr (FUSE) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t k4 = 16u * kb + 4u * gp;
          const void *ksc = SBL ? (const void *)(T.stp + 2 * S::KT + k4 * NG * ESZ)
                                : (const void *)T.ksb[kb][0];
          const void *kbi = SBL ? (const void *)(T.stp + 2 * S::KT + S::SBP + k4 * NG * ESZ)
                                : (const void *)T.ksb[kb][1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xf[kb][j] = fmaf(elem_f32<ET>(ksc, j * NG + g), sacc[0][kb][j], xf[kb][j]);
            xf[kb][j] = fmaf(elem_f32<ET>(kbi, j * NG + g), qsum[g], xf[kb][j]);
          }
        }
      }
    }
    half8_t pf[FUSE ? 1 : NG], pl[FUSE ? 1 : NG];
    float pgen[8];             // general path: p of the lane's 8 keys
    float alpha_gen = 1.0f;    // ... and the tile's rescale of the row
    if constexpr (SR) {
      // ---- scores of the (at most 4) live rows, lane = (key kl, rows
      // sr_row[0..1]) ----
      if (n < 4u) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            *reinterpret_cast<floatx4 *>(&sx[(g * 4 + n) * BN + 16 * kb + 4 * gp]) = sacc[g][kb];
      }
      __builtin_amdgcn_wave_barrier();
      float sc[2];
      bool need = false;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float x = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          x = fmaf(T.ksr[g], sx[(g * 4 + sr_row[s2]) * BN + kl], x);
          x = fmaf(T.kbr[g], sr_qs[s2][g], x);
        }
        const float mv = T.mr[s2];
        x = fmaf(x, a.qscale, (mv > kMasked) ? mv * kLog2e : -INFINITY);
        sc[s2] = x;
        need |= x > srM[s2] + kLazyQ;
      }
      // the reference max of a row moves only when one of its scores exceeds
      // it by more than kLazyQ (base 2), as in the general path
      float alpha[2] = {1.0f, 1.0f};
      if (__builtin_expect(__any(need), 0)) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float tmax = half_wave_max(sc[s2]);
          const float m_new = (tmax > srM[s2] + kLazyQ) ? tmax : srM[s2];
          const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
          alpha[s2] = __builtin_amdgcn_exp2f(srM[s2] - m_use);
          srM[s2] = m_new;
        }
        // O of MFMA row n (n < 4) takes the alpha of that row: slot n & 1 of
        // the lanes of half-wave n >> 1 (lanes 0 and 32 hold them)
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[0]), 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[1]), 0));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[0]), 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[1]), 32));
        const float an = n == 0u ? r0 : n == 1u ? r1 : n == 2u ? r2 : n == 3u ? r3 : 1.0f;
        if (!__all(an == 1.0f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= an;
        }
      }
      // p, the lane's shares of S and of the V bias sums, and p * vscale_g
      // into LDS as the PV operands [g][row][slot], an fp16 hi + lo pair as
      // in the general path (8-bit codes reach s c ~ 25, where a single fp16
      // operand would cost ~1e-2).  Slot order is the V operand's: key 16h + 4g4 + j
      // sits at 8 g4 + 4h + j, lane group gp reading slots 8gp .. 8gp+7.
      const uint32_t kpos = 8u * ((kl & 15u) >> 2) + 4u * (kl >> 4) + (kl & 3u);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float m_use = (srM[s2] == -INFINITY) ? 0.0f : srM[s2];
        const float pp = __builtin_amdgcn_exp2f(sc[s2] - m_use);
        srS[s2] = srS[s2] * alpha[s2] + pp;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          srB[s2][g] = fmaf(pp, T.vbr[g], srB[s2][g] * alpha[s2]);
          const float w = pp * T.vsr[g];
          const half_t hi = (half_t)w;
          pw[(g * 4 + sr_row[s2]) * BN + kpos] = hi;
          pwl[(g * 4 + sr_row[s2]) * BN + kpos] = (half_t)(w - (float)hi);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // B operand of row n (rows past 3 read row n & 3: dead columns)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        pf[g] = *reinterpret_cast<const half8_t *>(&pw[(g * 4 + (n & 3u)) * BN + 8 * gp]);
        pl[g] = *reinterpret_cast<const half8_t *>(&pwl[(g * 4 + (n & 3u)) * BN + 8 * gp]);
      }
    } else {
      float s[2][4];
      float tmax = -INFINITY;
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // (SBL: straight from the stage, the key's first element)
        const uint32_t k4 = 16u * kb + 4u * gp;
        const void *ksc = SBL ? (const void *)(T.stp + 2 * S::KT + k4 * NG * ESZ)
                              : (const void *)T.ksb[kb][0];
        const void *kbi = SBL ? (const void *)(T.stp + 2 * S::KT + S::SBP + k4 * NG * ESZ)
                              : (const void *)T.ksb[kb][1];
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = xf[kb][j];
  #pragma unroll
          for (int g = 0; g < (FUSE ? 0 : NG); ++g) {
            x = fmaf(elem_f32<ET>(ksc, j * NG + g), sacc[g][kb][j], x);
            x = fmaf(elem_f32<ET>(kbi, j * NG + g), qsum[g], x);
          }
          const float mv = T.m[kb][j];
          // an excluded cell adds -inf: the arithmetic above stays unconditional
          x = fmaf(x, a.qscale, (mv > kMasked) ? mv * kLog2e : -INFINITY);
          s[kb][j] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = max_xor32(max_xor16(tmax));
      // Lazy rescale: the reference max M moves only when the tile's max
      // exceeds it by more than kLazyQ (base 2); until then p <= 2^kLazyQ, held
      // exactly by the fp32 sums and by the fp16 hi + lo P * scale pair, and
      // O, S and M stay consistent: the same softmax.
      const float m_new = (tmax > Mrow + kLazyQ) ? tmax : Mrow;
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(Mrow - m_use);
      float p[8];
      float psum = 0.0f;
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(s[0][j] - m_use);
        p[4 + j] = __builtin_amdgcn_exp2f(s[1][j] - m_use);
      }
  #pragma unroll
      for (int j = 0; j < 8; ++j) psum += p[j];
      Srow = Srow * alpha + psum;
      Mrow = m_new;
  #pragma unroll
      for (int j = 0; j < 8; ++j) pgen[j] = p[j];
      alpha_gen = alpha;
      // B operands p * vscale_g as an fp16 pair hi + lo (the pair carries
      // about 22 bits of the fp32 product, so the fp16 operand width does not
      // limit the result), and the bias sums
  // (FUSE: built per group inside the PV loop instead)
  #pragma unroll
      for (int g = 0; g < (FUSE ? 0 : NG); ++g) {
        float acc = 0.0f;
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t k4 = 16u * (j >> 2) + 4u * gp;
          const void *vsc = SBL ? (const void *)(T.stp + 2 * S::KT + 2 * S::SBP + k4 * NG * ESZ)
                                : (const void *)T.vsb[j >> 2][0];
          const void *vbi = SBL ? (const void *)(T.stp + 2 * S::KT + 3 * S::SBP + k4 * NG * ESZ)
                                : (const void *)T.vsb[j >> 2][1];
          const float w = p[j] * elem_f32<ET>(vsc, (j & 3) * NG + g);
          const half_t hi = (half_t)w;
          pf[g][j] = hi;
          pl[g][j] = (half_t)(w - (float)hi);
          acc = fmaf(p[j], elem_f32<ET>(vbi, (j & 3) * NG + g), acc);
        }
        pb[g] = pb[g] * alpha + acc;
      }
      if (!__all(alpha == 1.0f)) {
  #pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
    }
    // PV: A = V codes of dim 16db+n for the lane's 8 keys (from LDS)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint32_t w = (16u * db + n) * BITS / 32u;
      const u32x4 lo = *reinterpret_cast<const u32x4 *>(&vlds[w * S::RS + 8u * gp]);
      const u32x4 hi = *reinterpret_cast<const u32x4 *>(&vlds[w * S::RS + 8u * gp + 4u]);
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // keys of slots 2e (low half) and 2e + 1 (high half)
        const uint32_t w0 = e < 2 ? lo[2 * e] : hi[2 * e - 4];
        const uint32_t w1 = e < 2 ? lo[2 * e + 1] : hi[2 * e - 3];
        const uint32_t x = __builtin_amdgcn_perm(w1, w0, vsel);
        const half2_t y = as_h2((x & vcm) | 0x64006400u);
        r[e] = as_u(y * vmul + vadd);
      }
      const int g = (16 * db) / G;
      if constexpr (FUSE) {
        if ((16 * db) % G == 0) {
          // group g's B operands p * vscale_g (hi + lo) and bias sum, as the
          // general epilogue makes them
          float acc = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t k4 = 16u * (j >> 2) + 4u * gp;
            const void *vsc = SBL ? (const void *)(T.stp + 2 * S::KT + 2 * S::SBP + k4 * NG * ESZ)
                                  : (const void *)T.vsb[j >> 2][0];
            const void *vbi = SBL ? (const void *)(T.stp + 2 * S::KT + 3 * S::SBP + k4 * NG * ESZ)
                                  : (const void *)T.vsb[j >> 2][1];
            const float w = pgen[j] * elem_f32<ET>(vsc, (j & 3) * NG + g);
            const half_t hi = (half_t)w;
            pf[0][j] = hi;
            pl[0][j] = (half_t)(w - (float)hi);
            acc = fmaf(pgen[j], elem_f32<ET>(vbi, (j & 3) * NG + g), acc);
          }
          pb[g] = pb[g] * alpha_gen + acc;
        }
      }
      const int gi = FUSE ? 0 : g;
      const half8_t vf = __builtin_bit_cast(half8_t, r);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[gi], oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[gi], oacc[db], 0, 0, 0);
    }
  };

  // ---- main loop: tile t from LDS while tiles t + 1 .. t + NS land ----
  // A tile's stage is copied whole into registers (load_tile), so the copies
  // of tile t + NS go into tile t's own stage as soon as those reads have
  // returned: NS tiles stay in flight behind the arithmetic.
  // Tile t0 first, then Q: the wait for Q's loads (they complete in order)
  // also completes tile t0, and the two latencies overlap.  The other NS - 1
  // tiles go out once Q's sums are in registers, so that wait does not
  // cover them; the first tile's wait below allows exactly those in flight.
  if (t0 < t1) issue(t0);
  load_q();
#pragma unroll
  for (int g = 0; g < NG; ++g) asm volatile("" ::"v"(qsum[g]));
#pragma unroll
  for (int i = 1; i < NS; ++i)
    if (t0 + i < t1) issue(t0 + i);
  if constexpr (SR) {
    // Q's group sums of the lane's SR rows (lane r holds row r's, r < 4)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int g = 0; g < NG; ++g) sr_qs[s2][g] = __shfl(qsum[g], (int)sr_row[s2]);
  }
  Tile cur;
  for (uint32_t t = t0; t < t1; ++t) {
    wait_tile(min(t1 - 1u - t, (uint32_t)(NS - 1)));
    load_tile(t, cur);
    // the reads of tile t's stage have returned before copies refill it
    // (SBL: compute still reads the stage's scales, so its refill waits)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (!SBL && t + NS < t1) issue(t + NS);
    int live = 0;
    if constexpr (SR) {
      live = (cur.mr[0] > kMasked) | (cur.mr[1] > kMasked);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) live |= (cur.m[kb][j] > kMasked);
    }
    if (__any(live)) {
      __builtin_amdgcn_wave_barrier();
      store_v(cur);
      __builtin_amdgcn_wave_barrier();
      compute(cur);
    }
    if (SBL) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (t + NS < t1) issue(t + NS);
    }
  }

  // ---- results ----
  if constexpr (SR) {
    // totals of the SR rows over the half-wave, then to lane (n, gp = 0) of
    // MFMA row n, so that the general reduction below finds them
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        srS[s2] += __shfl_xor(srS[s2], o);
#pragma unroll
        for (int g = 0; g < NG; ++g) srB[s2][g] += __shfl_xor(srB[s2][g], o);
      }
    }
    const int src = (int)(min(n, 3u) >> 1) * 32;
    const bool odd = (n & 1u) != 0u;
    const float s0 = __shfl(srS[0], src), s1 = __shfl(srS[1], src);
    const float m0 = __shfl(srM[0], src), m1 = __shfl(srM[1], src);
    Srow = (gp == 0u) ? (odd ? s1 : s0) : 0.0f;
    Mrow = odd ? m1 : m0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float b0 = __shfl(srB[0][g], src), b1 = __shfl(srB[1][g], src);
      pb[g] = (gp == 0u) ? (odd ? b1 : b0) : 0.0f;
    }
  }
  float stot = Srow + __shfl_xor(Srow, 16);
  stot += __shfl_xor(stot, 32);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    pb[g] += __shfl_xor(pb[g], 16);
    pb[g] += __shfl_xor(pb[g], 32);
  }
  if (!valid) return;
  const size_t rid = (size_t)qidx * a.q_l + node;
  // lane holds O[d = 16db + 4gp + j] of its row
  if (a.nwg == 1) {
    const float inv = (stot > 0.0f) ? 1.0f / stot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int g = (16 * db) / G;
      floatx4 o = (oacc[db] + pb[g]) * inv;
      const size_t off = rid * DIM + 16 * db + 4 * gp;
      if (ET == kF32) {
        *reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(a.out) + off) = o;
      } else if (ET == kBF16) {
        const uint32_t lo = f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        const uint32_t hi = f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + off) = u32x2{lo, hi};
      } else {
        half4_t h = {(half_t)o[0], (half_t)o[1], (half_t)o[2], (half_t)o[3]};
        *reinterpret_cast<half4_t *>(reinterpret_cast<half_t *>(a.out) + off) = h;
      }
    }
  } else {
    const size_t nrows = (size_t)a.batch * a.nq * a.q_l;
    const size_t prow = (size_t)split * nrows + rid;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int g = (16 * db) / G;
      *reinterpret_cast<floatx4 *>(a.part_o + prow * DIM + 16 * db + 4 * gp) = oacc[db] + pb[g];
    }
    if (gp == 0) {
      a.part_sm[prow * 2 + 0] = stot;
      a.part_sm[prow * 2 + 1] = Mrow;
    }
  }
}

// LDS of a variant: the stages and V transpose area, plus (SR) the live
// rows' scores [NG][4][BN] f32 and p * scale operands [NG][4][BN] as fp16
// hi and lo halves
template <int DIM, int BITS, int G, int MM, int ET, int SR> constexpr int quant_lds() {
  using ST = QStage<DIM, BITS, G, MM, ET>;
  constexpr int NG = DIM / G;
  return ST::LDS + (SR ? NG * 4 * BN * 4 + NG * 4 * BN * 2 * 2 : 0);
}

template <int DIM, int BITS, int G, int MM, int ET, int SR>
hipError_t launch_qs(const QuantArgs &a, hipStream_t s) {
  static const bool attr_set = [] {
    (void)hipFuncSetAttribute((const void *)quant_kernel<DIM, BITS, G, MM, ET, SR>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr_set;
  dim3 grid(grid_size(a.units, a.row_tiles));
  constexpr int lds = quant_lds<DIM, BITS, G, MM, ET, SR>();
  hipLaunchKernelGGL((quant_kernel<DIM, BITS, G, MM, ET, SR>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// At most 4 rows per kv stream (decode with a GQA group of up to 4) and
// head dims up to 128 take the SR epilogue.
template <int DIM, int BITS, int G, int MM, int ET>
hipError_t launch_qm(const QuantArgs &a, hipStream_t s) {
  if constexpr (DIM <= 128)
    if (a.rows <= 4u) return launch_qs<DIM, BITS, G, MM, ET, 1>(a, s);
  return launch_qs<DIM, BITS, G, MM, ET, 0>(a, s);
}

template <int DIM, int BITS, int G, int ET>
hipError_t launch_q(const QuantArgs &a, hipStream_t s) {
  if (a.mbool != nullptr) {
    const uint64_t words = a.mask_head_stride | a.mask_stride | a.kv_seq_len |
                           (uint64_t)((uintptr_t)a.mbool / sizeof(uint32_t));
    if (words % 4 == 0) return launch_qm<DIM, BITS, G, kMaskBoolB128, ET>(a, s);
    return launch_qm<DIM, BITS, G, kMaskBool, ET>(a, s);
  }
  if (a.mask == nullptr) return launch_qm<DIM, BITS, G, kMaskNone, ET>(a, s);
  constexpr uint64_t esz = Elem<ET>::SZ;
  const uint64_t all = a.mask_head_stride | a.mask_stride | a.kv_seq_len |
                       (uint64_t)((uintptr_t)a.mask / esz);
  if (all % (16 / esz) == 0) return launch_qm<DIM, BITS, G, kMaskB128, ET>(a, s);
  if (all % (4 / esz) == 0) return launch_qm<DIM, BITS, G, kMaskB32, ET>(a, s);
  if constexpr (ET != kF32) return launch_qm<DIM, BITS, G, kMaskReg, ET>(a, s);
  return hipErrorInvalidValue;   // (4-byte cells always take 4-byte copies)
}

template <int DIM, int BITS, int ET>
hipError_t launch_qg(const QuantArgs &a, uint32_t G, hipStream_t s) {
  switch (G) {
    case 32: return launch_q<DIM, BITS, 32, ET>(a, s);
    case 64:
      if constexpr (DIM % 64 == 0) return launch_q<DIM, BITS, 64, ET>(a, s);
      return hipErrorInvalidValue;
    case 128:
      if constexpr (DIM % 128 == 0) return launch_q<DIM, BITS, 128, ET>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int DIM, int ET>
hipError_t launch_qb(const QuantArgs &a, uint32_t bits, uint32_t G, hipStream_t s) {
  return bits == 4 ? launch_qg<DIM, 4, ET>(a, G, s) : launch_qg<DIM, 8, ET>(a, G, s);
}

// Workgroups of one variant a CU holds: the runtime's occupancy answer for
// the kernel with its LDS, or, with no device to ask, the plan's budgets
// (two wavefronts per SIMD up to dim 128, one above; 160 KB of LDS).
template <int DIM, int BITS, int G, int MM, int ET>
uint32_t wgs_per_cu() {
  using ST = QStage<DIM, BITS, G, MM, ET>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, quant_kernel<DIM, BITS, G, MM, ET, 0>,
                                                   kThreads, ST::LDS) == hipSuccess &&
      n > 0)
    return (uint32_t)n;
  (void)hipGetLastError();
  const uint32_t by_regs = DIM <= 128 ? 8u : 4u;
  const uint32_t by_lds = (160u * 1024u) / (uint32_t)ST::LDS;
  return by_regs < by_lds ? by_regs : by_lds;
}

template <int DIM, int BITS, int G, int ET>
uint32_t wgs_per_cu_m(int mask_kind) {
  // the T mask's copy modes share one footprint (the register-load mode is
  // smaller); both u32 copy modes share one too
  if (mask_kind == 2) return wgs_per_cu<DIM, BITS, G, kMaskBoolB128, ET>();
  if (mask_kind == 1) return wgs_per_cu<DIM, BITS, G, kMaskB128, ET>();
  return wgs_per_cu<DIM, BITS, G, kMaskNone, ET>();
}

template <int DIM, int BITS, int ET>
uint32_t wgs_per_cu_g(uint32_t G, int mask_kind) {
  switch (G) {
    case 32: return wgs_per_cu_m<DIM, BITS, 32, ET>(mask_kind);
    case 64:
      if constexpr (DIM % 64 == 0) return wgs_per_cu_m<DIM, BITS, 64, ET>(mask_kind);
      return 0;
    case 128:
      if constexpr (DIM % 128 == 0) return wgs_per_cu_m<DIM, BITS, 128, ET>(mask_kind);
      return 0;
    default: return 0;
  }
}

template <int DIM, int ET>
uint32_t wgs_per_cu_b(uint32_t bits, uint32_t G, int mask_kind) {
  return bits == 4 ? wgs_per_cu_g<DIM, 4, ET>(G, mask_kind)
                   : bits == 8 ? wgs_per_cu_g<DIM, 8, ET>(G, mask_kind) : 0;
}

}  // namespace
}  // namespace ta
