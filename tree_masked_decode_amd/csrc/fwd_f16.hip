// fwd_f16.hip -- tree-attention forward for fp16 K/V on the matrix cores.
//
// "tree_attention.metal" (mlx-native 0.9.1), tree_attention_impl computes,
// per (query, head), an online softmax over KV chunks with an explicit mask
// and GQA, and writes split-KV partials.  Every query row that shares a kv
// head -- q_l nodes x (n_heads / n_kv_heads) heads -- reads the same K/V, so
// here one workgroup takes up to 192 such rows and turns Q.K^T and P.V into
// dense tiles for v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation):
//
//   S^T[key][row] = K[key][:] . Q'[row][:]       A = K   (LDS), B = Q'^T (VGPRs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  A = V^T (LDS), B = P^T (VGPRs)
//
// With this orientation every lane owns one query row in both the score and
// the output accumulators, so the softmax state (M, S) and the rescale factor
// stay in the lane.  Q' = Q * scale is rounded to fp16 once.  The score
// instruction's accumulator input is the tile's mask (the additive cell, or
// -inf for an excluded key), so S^T comes out with the mask already added;
// p = exp2(s * log2(e) - M * log2(e)).  The row sum S is a matrix
// instruction too: a block of ones times P^T, i.e. the sum of the same fp16
// p that weight O.
//
// Workgroup = W wavefronts; each owns RB blocks of 16 rows and feeds every
// K/V operand it reads from LDS to RB matrix instructions.  head_dim 256
// runs W = 8 (two wavefronts per SIMD, RB = 1): with one barrier per tile
// keeping the wavefronts in step, a second wavefront per SIMD is what lets
// LDS waits and the softmax of one overlap the matrix work of the other.
//
// Memory pipeline: tiles of 32 keys (K, V and the raw mask cells of the
// workgroup's tree nodes) go straight from global memory into a ring of NS
// LDS stages with global_load_lds_dwordx4, NS - 1 tiles ahead of the
// arithmetic, so about (NS - 1) * 32 KB per CU is in flight to cover the
// latency of HBM; no registers hold staged data.  One barrier per tile; a
// tile's K copies go out right after it and its V and mask copies after the
// scores, so that they drain behind the arithmetic rather than in a burst.
// K and V are stored row-major with a 16-byte-chunk XOR swizzle (K: chunk c
// of row r lives at c ^ (r & 15); V: at c ^ 2 (r & 15), for reads of chunk
// pairs): every lane of a copy picks the global chunk that belongs at its LDS
// slot, and the operand reads are free of bank conflicts.
// V^T operands come from ds_read_b64_tr_b16, which transposes 4x16 blocks of
// 16-bit values on the way out of LDS.
//
// A wavefront whose rows have every cell of a tile excluded (mask at or below
// -65504, or past the causal limit) skips that tile's arithmetic
// ("tree_attention.metal" skips fully masked chunks); the tile is still
// fetched for the other wavefronts.
#include "common.h"

#include <type_traits>

namespace ta {

namespace {

constexpr int BN = 32;                // keys per tile
constexpr int kLdsBytes = 160 * 1024;
// Lazy-rescale threshold of the running max, in base-2 logit units.
constexpr float kLazy = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;
// LDS operand reads kept in flight ahead of the matrix instructions
constexpr int kAheadQK = 4;
constexpr int kAheadPV = 4;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int cmin(int x, int y) { return x < y ? x : y; }

// MROWS: tree nodes a stage's mask tile holds (0 for the implicit causal
// mask).  VEC: mask rows 16-byte aligned, copied 16 bytes per lane.
template <int D, int RB, int MROWS, bool VEC, int W> struct F16Shape {
  static constexpr int kThreads = 64 * W;             // W wavefronts
  static constexpr int RPW = W * 16 * RB;             // rows per workgroup
  static constexpr int CH = D / 8;                    // 16-byte chunks per K/V row
  static constexpr int KB = BN / 16;                  // 16-key score blocks
  static constexpr int DS = D / 32;                   // QK steps over d
  static constexpr int DB = D / 16;                   // PV output blocks over d
  static constexpr int KV_BYTES = BN * D * 2;         // K (or V) bytes of a tile
  static constexpr int KV_PW = KV_BYTES / 1024 / W;   // 1 KB copies per wavefront
  static constexpr int M_BYTES = MROWS * BN * 4;      // mask cells of a tile
  static constexpr int M_PW = MROWS == 0 ? 0 : VEC ? M_BYTES / 1024 / W : M_BYTES / 256 / W;
  static constexpr int STAGE = 2 * KV_BYTES + M_BYTES;
  static constexpr int NS = cmin(4, kLdsBytes / STAGE);
  static constexpr int PER_TILE = 2 * KV_PW + M_PW;   // copies per wavefront per tile
  static_assert(KV_PW >= 1 && KV_BYTES % (1024 * W) == 0, "tile / workgroup shape");
  static_assert(MROWS % (VEC ? 8 * W : 2 * W) == 0, "mask rows per wavefront");
  static_assert(NS >= 2, "LDS too small for two stages");
  static_assert(PER_TILE * (NS - 2) <= 63, "vmcnt range");
};

// Q'^T fragments wanted in registers at this point: the compiler waits for
// their loads here rather than where they are first used.
template <int RB, int DS> __device__ inline void hold_q(const half8_t (&q)[RB][DS]) {
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < DS; ++j) asm volatile("" ::"v"(q[i][j]));
}

__device__ inline uint32_t swz(uint32_t row, uint32_t chunk) { return chunk ^ (row & 15u); }
// V tiles use pairs of chunks: the transposing reads take 32 bytes (two
// chunks) from each of four rows per 16 lanes, so rows are spread over chunk
// pairs: chunk c of row r lives at c ^ (2 (r & 15)) (mod chunks per row).
template <int CH> __device__ inline uint32_t swz_v(uint32_t row, uint32_t chunk) {
  return chunk ^ ((2u * (row & 15u)) & (uint32_t)(CH - 1));
}

// Instruction-order hint for a block of LDS operand reads feeding matrix
// instructions: the first AHEAD groups of RD reads go out, then every group
// of MF matrix instructions is followed by the reads of the group AHEAD steps
// later, so that AHEAD operand loads are in flight while the matrix cores
// run instead of each instruction waiting out one LDS round trip.  (Order
// only: the compiler's wait counts keep every use after its load.)
template <int STEPS, int RD, int MF, int AHEAD>
__device__ inline void lds_mfma_pipeline() {
  static_assert(AHEAD >= 1 && AHEAD <= STEPS, "prefetch depth");
  __builtin_amdgcn_sched_group_barrier(0x100, RD * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < STEPS - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MF * AHEAD, 0);
}

// NT: the K/V copies take the non-temporal policy (long K/V streams; the
// planner sets FwdArgs::stream_nt).
template <int D, int RB, int MROWS, bool VEC, int W, bool NT>
__global__ __launch_bounds__(64 * W, 1) void fwd_f16_kernel(FwdArgs a) {
  constexpr bool IMPLICIT = MROWS == 0;
  using S = F16Shape<D, RB, MROWS, VEC, W>;
  constexpr int KB = S::KB, DS = S::DS, DB = S::DB, NS = S::NS;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) char *)lds);

  uint32_t unit, rt;
  decode_block(blockIdx.x, a.row_tiles, unit, rt);
  if (unit >= a.units) return;
  const uint32_t hk = unit / a.nwg;
  const uint32_t split = unit % a.nwg;
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const uint32_t lane = tid % kWave;
  const uint32_t n = lane & 15u;   // the lane's query row within a 16-row block
  const uint32_t gp = lane >> 4;   // lane group

  const uint32_t row0 = rt * S::RPW;
  const uint32_t node0 = row0 / a.group;
  const uint32_t last_row = min(row0 + S::RPW, a.rows) - 1u;
  const uint32_t nnodes = last_row / a.group - node0 + 1u;   // nodes of this workgroup

  // ---- the lane's rows; their Q'^T fragments (row n, d = 32ds + 8gp + 0..7)
  // are loaded once the first tiles' copies are on their way ----
  uint32_t node[RB];
  bool valid[RB];
  half8_t qf[RB][DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t gr = row0 + wave * 16u * RB + 16u * rb + n;
    valid[rb] = gr < a.rows;
    node[rb] = valid[rb] ? gr / a.group : node0;
  }
  auto load_q = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t gr = row0 + wave * 16u * RB + 16u * rb + n;
      const uint32_t head = hk * a.group + (valid[rb] ? gr % a.group : 0u);
      const float *qrow = a.q + ((size_t)head * a.q_l + node[rb]) * D;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        // (a row past the end reads node0's row of its kv head's first head,
        // in bounds, and is zeroed: no branch splits the loads)
        const float sc = valid[rb] ? a.scale : 0.0f;
        qf[rb][ds] = __builtin_bit_cast(half8_t, q_fragment(qrow + 32 * ds, gp, sc));
      }
    }
  };

  const size_t kvbase = (size_t)hk * a.kv_capacity * D;
  const half_t *K = static_cast<const half_t *>(a.k) + kvbase;
  const half_t *V = static_cast<const half_t *>(a.v) + kvbase;
  const uint32_t L = a.kv_seq_len;

  // ---- copies of one tile into its stage ----
  // K/V: copy i of this wavefront fills LDS chunks p = 64 (W_i) + lane of the
  // tile, W_i = wave * KV_PW + i; chunk p is row p / CH, physical chunk
  // p % CH, holding logical chunk (p % CH) ^ (row & 15).
  uint32_t kv_row[S::KV_PW], kv_col[S::KV_PW], v_col[S::KV_PW];
  uint32_t k_off[S::KV_PW], v_off[S::KV_PW];   // byte offsets within a full tile
#pragma unroll
  for (int i = 0; i < S::KV_PW; ++i) {
    const uint32_t p = (wave * S::KV_PW + i) * 64u + lane;
    kv_row[i] = p / S::CH;
    kv_col[i] = 8u * swz(kv_row[i], p % S::CH);
    v_col[i] = 8u * swz_v<S::CH>(kv_row[i], p % S::CH);
    k_off[i] = 2u * (kv_row[i] * D + kv_col[i]);
    v_off[i] = 2u * (kv_row[i] * D + v_col[i]);
  }
  // mask: node rows of BN cells (128 bytes) back to back; a 16-byte copy
  // covers 8 rows (lane / 8, cells 4 (lane % 8) ..), a 4-byte copy 2 rows
  // (lane / 32, cell lane % 32).  Rows past the workgroup's nodes re-read
  // node0's row and are never used.
  constexpr int M_RPC = VEC ? 8 : 2;   // mask rows per copy
  uint32_t m_row[S::M_PW > 0 ? S::M_PW : 1];
  const uint32_t m_col = VEC ? 4u * (lane % 8u) : lane % 32u;
#pragma unroll
  for (int j = 0; j < S::M_PW; ++j) {
    const uint32_t r = (wave * S::M_PW + j) * M_RPC + lane / (64u / M_RPC);
    m_row[j] = r < nnodes ? r : 0u;
  }
  auto stage_addr = [&](uint32_t t, uint32_t t0) -> uint32_t {
    return lds0 + ((t - t0) % NS) * S::STAGE;
  };
  // part 0: the K copies; part 1: the V and mask copies.  The two parts go
  // out at different points of a tile's arithmetic, so that the copies
  // drain behind it instead of queueing in one burst.
  auto issue = [&](uint32_t t, uint32_t t0, auto part) {
    constexpr int PART = decltype(part)::value;
    const uint32_t key0 = t * BN;
    const uint32_t sb = stage_addr(t, t0);
    const bool full = key0 + BN <= L;
    if (full) {
      // every key of the tile is below kv_seq_len: a scalar tile base plus
      // the lane's fixed offset
      const half_t *base = (PART == 0 ? K : V) + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < S::KV_PW; ++i) {
        const uint32_t la = sb + (wave * S::KV_PW + i) * 1024u;
        if (PART == 0)
          dma_b128_s<NT>(base, k_off[i], la);
        else
          dma_b128_s<NT>(base, v_off[i], la + S::KV_BYTES);
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::KV_PW; ++i) {
        // keys past kv_seq_len re-read the last valid row (never used)
        const uint32_t key = min(key0 + kv_row[i], L - 1u);
        const uint32_t la = sb + (wave * S::KV_PW + i) * 1024u;
        if (PART == 0)
          dma_b128<NT>(K + (size_t)key * D + kv_col[i], la);
        else
          dma_b128<NT>(V + (size_t)key * D + v_col[i], la + S::KV_BYTES);
      }
    }
    if (PART == 1) {
#pragma unroll
      for (int j = 0; j < S::M_PW; ++j) {
        uint32_t key = key0 + m_col;
        // past kv_seq_len: stay inside the row (16-byte chunks: the chunk
        // that holds cell L - 1, which ends before mask_stride)
        if (key >= L) key = VEC ? ((L - 1u) & ~3u) : L - 1u;
        const float *g = a.mask + (size_t)(node0 + m_row[j]) * a.mask_stride + key;
        const uint32_t la = sb + 2u * S::KV_BYTES + (wave * S::M_PW + j) * (VEC ? 1024u : 256u);
        if (VEC)
          dma_b128(g, la);
        else
          dma_b32(g, la);
      }
    }
  };
  // wait until tile t has landed; `after` later tiles (0 .. NS - 2) may stay in flight
  auto wait_tile = [&](uint32_t after) {
    if (NS >= 4 && after >= 2)
      wait_vm<(NS >= 4 ? 2 * S::PER_TILE : 0)>();
    else if (NS >= 3 && after >= 1)
      wait_vm<(NS >= 3 ? S::PER_TILE : 0)>();
    else
      wait_vm<0>();
  };

  // ---- online-softmax state of the lane's rows ----
  // M in natural units; nml = -M * log2(e) (0 while M is -inf, when O and S
  // are still zero); S and O accumulate in matrix-core registers.
  float Mrow[RB], nml[RB];
  floatx4 oacc[RB][DB], sacc_sum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    Mrow[rb] = -INFINITY;
    nml[rb] = 0.0f;
    sacc_sum[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  int64_t causal_last[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    causal_last[rb] = (int64_t)L - (int64_t)a.q_l + (int64_t)node[rb];

  // Scores and online softmax of tile t (stage at LDS byte address sb) for the
  // lane's rows.  Sets pf (the P^T operands) and alpha (the rescale of O each
  // row needs, 1 almost always); returns 0 if none of the wavefront's cells
  // is live.  GENERAL: the tile may hold keys past kv_seq_len or (implicit
  // mask) past a row's causal limit, so every cell is checked; otherwise every
  // key is in range and, with the implicit mask, attended by every row.
  auto qk_softmax = [&](uint32_t t, uint32_t sb, float (&alpha_out)[RB], half8_t (&pf)[RB],
                        auto general) -> int {
    constexpr bool GENERAL = decltype(general)::value;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) alpha_out[rb] = 1.0f;
    const half_t *Ks = reinterpret_cast<const half_t *>(lds + (sb - lds0));
    const float *Ms = reinterpret_cast<const float *>(lds + (sb - lds0) + 2 * S::KV_BYTES);
    const uint32_t key0 = t * BN;
    // accumulator inputs: the lane's cells, keys 16kb + 4gp + j -- the
    // additive mask value, or -inf for an excluded key.  Rows past the end
    // use node0's cells; their Q is zero and their results are never written.
    floatx4 sacc[RB][KB];
    if (IMPLICIT && !GENERAL) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[rb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      // A tile wholly before the window start has no live cell.  The fast
      // tiles never are, but the branch keeps the tile loop below nested:
      // without it, at one row block, the compiler folds the rescale exit
      // into the tile loop and copies every O accumulator out of the
      // matrix-core registers once per tile.
      if (key0 + BN <= a.key_lo) return 0;
    } else {
      float mmax = -INFINITY;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          floatx4 x;
          if (!IMPLICIT)
            x = *reinterpret_cast<const floatx4 *>(Ms + (node[rb] - node0) * BN + 16 * kb + 4 * gp);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = key0 + 16u * kb + 4u * gp + j;
            bool in;
            if (IMPLICIT)
              in = key < L && key >= a.key_lo && (int64_t)key <= causal_last[rb];
            else if (GENERAL)
              in = x[j] > kMasked && key < L;
            else
              in = x[j] > kMasked;
            sacc[rb][kb][j] = in ? (IMPLICIT ? 0.0f : x[j]) : -INFINITY;
            mmax = fmaxf(mmax, sacc[rb][kb][j]);
          }
        }
      if (!__any(mmax > -INFINITY)) return 0;
    }

    // S^T (+ mask): each K operand feeds RB instructions
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t row = 16u * kb + n;
        const half8_t kf = *reinterpret_cast<const half8_t *>(
            Ks + row * D + 8 * swz(row, 4u * ds + gp));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[rb][ds], sacc[rb][kb], 0, 0, 0);
      }
    }
    lds_mfma_pipeline<DS * KB, 1, RB, kAheadQK>();
    // online softmax per row block; P^T operands
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = fmaxf(fmaxf(fmaxf(sacc[rb][0][0], sacc[rb][0][1]), fmaxf(sacc[rb][0][2], sacc[rb][0][3])),
                         fmaxf(fmaxf(sacc[rb][1][0], sacc[rb][1][1]), fmaxf(sacc[rb][1][2], sacc[rb][1][3])));
      // the row's 32 cells sit in lanes n, n + 16, n + 32, n + 48
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      // Lazy rescale: the reference max moves (and O, S are rescaled) only
      // when the tile's max exceeds it by more than kLazy (base 2); until
      // then p <= 2^kLazy, exact in fp16 and fp32.  O, S and M stay
      // consistent, so the result is the same softmax.
      float alpha = 1.0f;
      if (tmax > Mrow[rb] + kLazy * kLn2) {
        const float nml_new = -tmax * kLog2e;
        // (O and S are still zero when M is -inf: nothing to rescale)
        alpha = (Mrow[rb] == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(nml_new - nml[rb]);
        Mrow[rb] = tmax;
        nml[rb] = nml_new;
      }
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(fmaf(sacc[rb][0][j], kLog2e, nml[rb]));
        p[4 + j] = __builtin_amdgcn_exp2f(fmaf(sacc[rb][1][j], kLog2e, nml[rb]));
      }
      pf[rb] = half8_t{(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3],
                       (half_t)p[4], (half_t)p[5], (half_t)p[6], (half_t)p[7]};
      alpha_out[rb] = alpha;
    }
    return 1;
  };
  // O^T += V^T P^T and S += 1 P^T for the stage at LDS byte address sb.
  const half8_t ones = {(half_t)1.0f, (half_t)1.0f, (half_t)1.0f, (half_t)1.0f,
                        (half_t)1.0f, (half_t)1.0f, (half_t)1.0f, (half_t)1.0f};
  auto pv = [&](uint32_t sb, const half8_t (&pf)[RB]) {
    const half_t *Vs = reinterpret_cast<const half_t *>(lds + (sb - lds0) + S::KV_BYTES);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sacc_sum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[rb], sacc_sum[rb], 0, 0, 0);
    // V^T operand of d-block db for keys F(gp, 0..7) read as two transposed
    // 4x16 blocks (keys 4gp..4gp+3 and 16+4gp..16+4gp+3)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      short4_t lo, hi;
      {
        const uint32_t r0 = 4u * gp + (n >> 2), r1 = r0 + 16u;
        const uint32_t ch = 2u * db + ((n & 3u) >> 1), half_off = 4u * (n & 1u);
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4 *)(Vs + r0 * D + 8 * swz_v<S::CH>(r0, ch) + half_off));
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4 *)(Vs + r1 * D + 8 * swz_v<S::CH>(r1, ch) + half_off));
      }
      const half8_t vf = __builtin_bit_cast(half8_t,
          (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                      hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rb], oacc[rb][db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);   // the row-sum instructions
    lds_mfma_pipeline<DB, 2, RB, kAheadPV>();
  };
  // The rare rescale of O and S: kept out of the tile loop below so that the
  // accumulators stay in the matrix-core registers inside it.
  auto rescale = [&](const float (&alpha)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sacc_sum[rb] *= alpha[rb];
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha[rb];
    }
  };

  // ---- main loop ----
  // the splits cover the tiles from the one that holds key_lo (the
  // implicit rule's window start; 0 otherwise)
  const uint32_t tile_lo = a.key_lo / BN;
  uint32_t t0, t1;
  uint32_t span_lo, span_hi;
  split_tiles(a, BN, tile_lo, span_lo, span_hi);
  split_range(span_hi - span_lo, a.nwg, split, t0, t1);
  t0 += span_lo;
  t1 += span_lo;
  // Tile t0 first, then Q: the wait the compiler puts before Q's first use
  // (loads complete in order) also completes tile t0, and the two latencies
  // overlap.  The rest of the prologue's tiles go out once Q is in
  // registers, so that wait does not hold up on them; the first tile's wait
  // below then allows exactly those NS - 2 tiles in flight.
  if (t0 < t1) {
    issue(t0, t0, std::integral_constant<int, 0>{});
    issue(t0, t0, std::integral_constant<int, 1>{});
  }
  load_q();
  hold_q(qf);
#pragma unroll
  for (int s = 1; s < NS - 1; ++s)
    if (t0 + s < t1) {
      issue(t0 + s, t0, std::integral_constant<int, 0>{});
      issue(t0 + s, t0, std::integral_constant<int, 1>{});
    }
  // Top of tile t: wait for its copies, barrier (every wavefront is done with
  // tile t - 1), then start refilling tile t - 1's stage with tile t + NS - 1
  // (K now, V and mask once the scores are out: refill_rest).
  // With two stages (the widest heads) the single tile in flight is refilled
  // in one go.
  auto begin_tile = [&](uint32_t t) {
    wait_tile(min(t1 - 1u - t, (uint32_t)(NS - 2)));
    __syncthreads();
    if (t + NS - 1 < t1) {
      issue(t + NS - 1, t0, std::integral_constant<int, 0>{});
      if (NS == 2) issue(t + NS - 1, t0, std::integral_constant<int, 1>{});
    }
  };
  auto refill_rest = [&](uint32_t t) {
    if (NS > 2 && t + NS - 1 < t1) issue(t + NS - 1, t0, std::integral_constant<int, 1>{});
  };
  float alpha[RB];
  half8_t pf[RB];
  // Tiles before `fast` hold only keys below kv_seq_len and, with the
  // implicit mask, keys every row of the workgroup attends: there the mask
  // needs no per-cell key checks.
  uint32_t fast = L / BN;
  // (rows whose last visible key lies before key 0, q_l > kv_seq_len, see
  // nothing: the bound clamps at 0 instead of wrapping)
  if (IMPLICIT)
    fast = min(fast, (uint32_t)(max<int64_t>(0, (int64_t)L - a.q_l + node0 + 1) / BN));
  // a window start inside the first tile: that split checks every cell
  if (IMPLICIT && a.key_lo % BN != 0 && t0 == tile_lo) fast = t0;
  fast = min(max(fast, t0), t1);
  uint32_t t = t0;
  while (t < fast) {
    // Inner loop: nothing but matrix instructions touches O.  A wavefront
    // that must rescale leaves it; every wavefront still passes exactly one
    // barrier per tile.
    bool need = false;
    uint32_t sb = 0;
    for (; t < fast; ++t) {
      begin_tile(t);
      sb = stage_addr(t, t0);
      const int live = qk_softmax(t, sb, alpha, pf, std::false_type{});
      refill_rest(t);
      bool r = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) r |= alpha[rb] != 1.0f;
      if (__builtin_expect(__any(r), 0)) {
        need = true;
        break;
      }
      if (live) pv(sb, pf);
    }
    if (!need) break;
    rescale(alpha);
    pv(sb, pf);
    ++t;
  }
  // the remaining few tiles (at the end of the key range) check every cell
  for (t = fast; t < t1; ++t) {
    begin_tile(t);
    const uint32_t sb = stage_addr(t, t0);
    const int live = qk_softmax(t, sb, alpha, pf, std::true_type{});
    refill_rest(t);
    if (live) {
      rescale(alpha);
      pv(sb, pf);
    }
  }

  // ---- results ----
  const size_t nrows = (size_t)a.n_heads * a.q_l;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float stot = sacc_sum[rb][0];
    if (!valid[rb]) continue;
    const uint32_t gr = row0 + wave * 16u * RB + 16u * rb + n;
    const uint32_t head = hk * a.group + gr % a.group;
    const size_t rid = (size_t)node[rb] * a.n_heads + head;
    if (a.nwg == 1) {
      const float inv = (stot > 0.0f) ? 1.0f / stot : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<floatx4 *>(a.out + rid * D + 16 * db + 4 * gp) = oacc[rb][db] * inv;
    } else {
      const size_t prow = (size_t)split * nrows + rid;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<floatx4 *>(a.part_o + prow * D + 16 * db + 4 * gp) = oacc[rb][db];
      if (gp == 0) {
        // M in base-2 units: p was taken relative to 2^(-nml)
        a.part_sm[prow * 2 + 0] = stot;
        a.part_sm[prow * 2 + 1] = Mrow[rb] == -INFINITY ? -INFINITY : -nml[rb];
      }
    }
  }
}

template <int D, int RB, int MROWS, bool VEC, int W, bool NT>
hipError_t launch_nt(const FwdArgs &a, hipStream_t s) {
  using Sh = F16Shape<D, RB, MROWS, VEC, W>;
  const size_t lds = (size_t)Sh::NS * Sh::STAGE;
  static const bool attr_set = [] {
    (void)hipFuncSetAttribute((const void *)fwd_f16_kernel<D, RB, MROWS, VEC, W, NT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    return true;
  }();
  (void)attr_set;
  dim3 grid(grid_size(a.units, a.row_tiles));
  hipLaunchKernelGGL((fwd_f16_kernel<D, RB, MROWS, VEC, W, NT>), grid, dim3(Sh::kThreads), lds, s, a);
  return hipGetLastError();
}
template <int D, int RB, int MROWS, bool VEC, int W>
hipError_t launch_v(const FwdArgs &a, hipStream_t s) {
  return a.stream_nt ? launch_nt<D, RB, MROWS, VEC, W, true>(a, s)
                     : launch_nt<D, RB, MROWS, VEC, W, false>(a, s);
}

template <int D, int RB, int W>
hipError_t launch_rb(const FwdArgs &a, hipStream_t s) {
  constexpr int RPW = W * 16 * RB;
  constexpr int M0 = 8 * W;  // smallest mask tile the wavefronts split evenly
  if (a.mask == nullptr) return launch_v<D, RB, 0, false, W>(a, s);
  // a row tile spans at most floor((RPW - 1) / group) + 2 tree nodes
  const uint32_t nodes = min((RPW - 1u) / a.group + 2u, a.q_l);
  const bool vec = ((uintptr_t)a.mask % 16u == 0) && (a.mask_stride % 4u == 0);
  if (nodes <= M0)
    return vec ? launch_v<D, RB, M0, true, W>(a, s) : launch_v<D, RB, M0, false, W>(a, s);
  if (nodes <= 2 * M0)
    return vec ? launch_v<D, RB, 2 * M0, true, W>(a, s) : launch_v<D, RB, 2 * M0, false, W>(a, s);
  return vec ? launch_v<D, RB, RPW, true, W>(a, s) : launch_v<D, RB, RPW, false, W>(a, s);
}

}  // namespace

uint32_t f16_tile_keys(uint32_t) { return (uint32_t)BN; }

// Launch plan: W wavefronts of RB 16-row blocks.  head_dim 256 runs two
// wavefronts per SIMD (W = 8, RB = 1) so that one wavefront's softmax and LDS
// waits overlap the other's matrix instructions; 128 and 512 run one per SIMD
// (W = 4) with as many row blocks as registers allow without spilling, fewer
// when that wastes fewer padded rows.
struct F16Plan { uint32_t w, rb; };
static F16Plan f16_plan(uint32_t head_dim, uint32_t rows) {
  if (head_dim == 256) return F16Plan{8u, 1u};
  const uint32_t max_rb = head_dim >= 512 ? 1u : 3u;
  uint32_t best = 1, best_waste = 0xffffffffu;
  for (uint32_t rb = max_rb; rb >= 1; --rb) {
    const uint32_t rpw = 64u * rb;
    const uint32_t waste = ((rows + rpw - 1) / rpw) * rpw - rows;
    if (waste < best_waste) {
      best = rb;
      best_waste = waste;
    }
  }
  return F16Plan{4u, best};
}

uint32_t f16_rows_per_wg(uint32_t head_dim, uint32_t rows, uint32_t group, bool implicit,
                         bool mask_vec) {
  if (wide_applies(head_dim, rows, group, implicit, mask_vec)) return wide_rows_per_wg();
  const F16Plan p = f16_plan(head_dim, rows);
  return 16u * p.w * p.rb;
}

hipError_t launch_forward_f16(const FwdArgs &a, uint32_t head_dim, hipStream_t s) {
  const bool implicit = a.mask == nullptr;
  const bool vec = ((uintptr_t)a.mask % 16u == 0) && (a.mask_stride % 4u == 0);
  if (wide_applies(head_dim, a.rows, a.group, implicit, vec)) return launch_forward_wide(a, head_dim, s);
  const F16Plan p = f16_plan(head_dim, a.rows);
  switch (head_dim) {
    case 128:
      return p.rb == 3 ? launch_rb<128, 3, 4>(a, s) : p.rb == 2 ? launch_rb<128, 2, 4>(a, s)
                                                                : launch_rb<128, 1, 4>(a, s);
    case 256:
      return launch_rb<256, 1, 8>(a, s);
    case 512: return launch_rb<512, 1, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
