// fwd_wide.hip -- tree-attention forward for fp16 K/V when many query rows
// share one K/V stream (the 32K dynamic-tree verify: 384 rows per kv head).
//
// Same computation as fwd_f16.hip ("tree_attention.metal", tree_attention_impl:
// Q.K^T + mask, online softmax, P.V, split partials), organised for the LDS
// bandwidth of a CDNA4 compute unit.  Every wavefront reads the whole K tile
// (ds_read_b128) and V tile (ds_read_b64_tr_b16, which moves half the bytes
// per instruction) of each 32-key step from LDS, and the LDS serves about one
// such read per 8 cycles per CU; the matrix work a read feeds grows with the
// rows a wavefront owns.  Here one wavefront per SIMD owns RB = 3 blocks of
// 16 rows (48 rows, 192 per workgroup): each K or V operand read feeds three
// v_mfma_f32_16x16x32_f16, and LDS reads and matrix work per tile are about
// equal (with 16 rows per wavefront the LDS needs three times the matrix
// time).  O (48 rows x 256 dims, fp32) lives in the accumulation registers.
//
// Per tile t of a split:
//   top     wait for tile t+1's copies, barrier, refill the stage tile t-1
//           used with tile t+3 (global_load_lds_dwordx4, 4 stages)
//   QK      S(t+1) = K(t+1) . Q'^T + C(t+1) for the 48 rows
//   softmax p = 2^S(t) (the scores already have the row reference max
//           subtracted, see below), P in fp16
//   PV      O^T += V(t)^T . P^T, row sums += 1 . P^T
// QK of the next tile is issued in the same block as the softmax of this one,
// so the exponentials overlap matrix work.
//
// Logits are in base-2 units: Q' = Q * scale * log2(e), rounded to fp16 once.
// Each row keeps a reference max M (base 2) that moves only when a tile's
// row max exceeds it by more than 8 (lazy rescale: p <= 2^8 stays exact in
// fp16 and fp32, and O, S and M stay consistent).  The accumulator input
// C(t) of the score instructions is -M for a tile whose mask cells are all
// zero for the wavefront's rows (the common case of a tree mask: the shared
// prefix) and mask * log2(e) - M, or -inf for an excluded cell (at or below
// -65504, past kv_seq_len, or outside the implicit causal rule), otherwise.
// So p = 2^S needs no further arithmetic, and an excluded key gives exactly
// 0.  A tile is softmaxed on the fast path (exp and fp16 conversion only)
// when every row's M is finite and unchanged since the tile's scores were
// issued; the fp16 p are checked against 2^8 with packed integer max
// instructions (p >= 0, so the 16-bit patterns order like the values), and
// a tile that fails the check, or needs a new M, takes the slow path: true
// row max, new M, rescale of O and the row sums, p recomputed.
#include "common.h"

#include <type_traits>

#include "fwd_wide_loop.inc"

namespace ta {

namespace {

constexpr int BN = 32;      // keys per tile
constexpr int W = 4;        // wavefronts per workgroup (one per SIMD)
constexpr int NS = 4;       // LDS stages
constexpr float kLazy2 = 8.0f;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

// ML: 16-byte mask loads per lane that cover the wavefront's tree nodes for
// one tile (0 for the implicit causal rule).
template <int D, int RB, int ML> struct WideShape {
  static constexpr int RPW = W * 16 * RB;         // rows per workgroup
  static constexpr int CH = D / 8;                // 16-byte chunks per K/V row
  static constexpr int DS = D / 32;               // score steps over d
  static constexpr int DB = D / 16;               // output blocks over d
  static constexpr int KVB = BN * D * 2;          // bytes of one K (or V) tile
  static constexpr int KV_PW = KVB / 1024 / W;    // 1 KB copies per wavefront per K (or V) tile
  static constexpr int PER_TILE = 2 * KV_PW + ML; // vector-memory ops per wavefront per tile
  static constexpr int MB = ML * 1024;            // mask bytes per wavefront per tile
  static constexpr int LDS = 2 * NS * KVB + NS * W * MB;
  static_assert(KV_PW >= 1 && KVB % (1024 * W) == 0, "tile / workgroup shape");
  // every LDS operand address is a per-lane register plus an instruction
  // offset below 64 KB: K at stage * KVB + kb * 16 rows, V at the same plus
  // NS * KVB (folded into the V registers)
  static_assert((NS - 1) * KVB + 16 * D * 2 < 65536, "LDS offsets");
};

__device__ inline uint32_t swz(uint32_t row, uint32_t chunk) { return chunk ^ (row & 15u); }
template <int CH> __device__ inline uint32_t swz_v(uint32_t row, uint32_t chunk) {
  return chunk ^ ((2u * (row & 15u)) & (uint32_t)(CH - 1));
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx32 __attribute__((ext_vector_type(32)));

// The registers the tile loop (fwd_wide_loop.inc) writes besides the ones
// bound to its operands: the scores (accumulated in a[212:235], copied to
// v[96:119]) and their -M' input (a[236:247]), P^T fragments, the operand
// ring and softmax temporaries, and its scalar registers.
#define TA_WIDE_CLOBBERS                                                                          \
  "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107",   \
      "v108", "v109", "v110", "v111", "v112", "v113", "v114", "v115", "v116", "v117", "v118",   \
      "v119", "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127", "v128", "v129",   \
      "v130", "v131", "v132", "v133", "v134", "v135", "v136", "v137", "v138", "v139", "v140",   \
      "v141", "v142", "v143", "v144", "v145", "v146", "v147", "v148", "v149", "v150", "v151",   \
      "v152", "v153", "v154", "v155", "v176", "v177", "v178", "v179", "v180", "v181", "v182",   \
      "v183", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193",   \
      "v194", "v195", "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204",   \
      "v205", "v206", "v207", "s80", "s81", "s82", "s83", "s84", "s85", "s86", "s87", "s88",     \
      "s89", "s90", "s91", "s92", "s93", "s94", "s95", "s96", "s97", "s98", "s99", "vcc", "scc", "m0", \
      "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", \
      "a223", "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", \
      "a234", "a235", "a236", "a237", "a238", "a239", "a240", "a241", "a242", "a243", "a244", \
      "a245", "a246", "a247", \
      "memory"

template <int ML>
__device__ inline void wide_loop(floatx32 &O0, floatx32 &O1, floatx32 &O2, floatx32 &O3,
                                 floatx32 &O4, floatx32 &O5, floatx16 &R, floatx16 &CM,
                                 const floatx32 &Q0, const floatx32 &Q1, const floatx32 &Q2,
                                 const floatx4 &ONES, const floatx32 &OFF, const floatx8 &MISC,
                                 const floatx2 &MISC2, const floatx4 &KVROW,
                                 uint32_t t0, uint32_t t1, uint32_t L, uint64_t kb, uint64_t vb,
                                 uint64_t mb, uint32_t m0k, uint32_t m0m, uint32_t keylo,
                                 int32_t climit, uint32_t lclamp) {
  const uint32_t kb0 = sgpr_u32((uint32_t)kb), kb1 = sgpr_u32((uint32_t)(kb >> 32));
  const uint32_t vb0 = sgpr_u32((uint32_t)vb), vb1 = sgpr_u32((uint32_t)(vb >> 32));
  const uint32_t mb0 = sgpr_u32((uint32_t)mb), mb1 = sgpr_u32((uint32_t)(mb >> 32));
#define TA_WIDE_OPERANDS(LOOP)                                                                    \
  asm volatile(LOOP                                                                              \
               : "+{a[0:31]}"(O0), "+{a[32:63]}"(O1), "+{a[64:95]}"(O2), "+{a[96:127]}"(O3),     \
                 "+{a[128:159]}"(O4), "+{a[160:191]}"(O5), "+{a[192:207]}"(R),                    \
                 "+{v[160:175]}"(CM)                                                             \
               : "{v[0:31]}"(Q0), "{v[32:63]}"(Q1), "{v[64:95]}"(Q2), "{v[156:159]}"(ONES),     \
                 "{v[208:239]}"(OFF), "{v[240:247]}"(MISC), "{v[248:249]}"(MISC2),              \
                 "{a[208:211]}"(KVROW), [t0] "s"(sgpr_u32(t0)),                                  \
                 [t1] "s"(sgpr_u32(t1)), [L] "s"(sgpr_u32(L)), [kb0] "s"(kb0), [kb1] "s"(kb1),   \
                 [vb0] "s"(vb0), [vb1] "s"(vb1), [mb0] "s"(mb0), [mb1] "s"(mb1),                 \
                 [m0k] "s"(sgpr_u32(m0k)), [m0m] "s"(sgpr_u32(m0m)), [keylo] "s"(sgpr_u32(keylo)), \
                 [climit] "s"(sgpr_u32((uint32_t)climit)), [lclamp] "s"(sgpr_u32(lclamp))        \
               : TA_WIDE_CLOBBERS)
  if constexpr (ML == 0) TA_WIDE_OPERANDS(TA_WIDE_LOOP_ML0);
  else if constexpr (ML == 1) TA_WIDE_OPERANDS(TA_WIDE_LOOP_ML1);
  else TA_WIDE_OPERANDS(TA_WIDE_LOOP_ML2);
#undef TA_WIDE_OPERANDS
}

// An empty asm that reads three register tuples: the computations that
// produce them cannot sink below it.  (A device function: the host pass of a
// kernel body cannot take "v" operands.)
__device__ __attribute__((always_inline)) inline void hold_vgprs(const floatx32 &a,
                                                                 const floatx32 &b,
                                                                 const floatx32 &c) {
  asm volatile("" ::"v"(a), "v"(b), "v"(c));
}

template <int D, int RB, int ML>
__global__ __launch_bounds__(64 * W, 1) void fwd_wide_kernel(FwdArgs a) {
  static_assert(D == 256 && RB == 3, "the tile loop is generated for head dim 256, 48 rows per wavefront");
  constexpr bool IMPLICIT = ML == 0;
  using S = WideShape<D, RB, ML>;
  constexpr int DS = S::DS, DB = S::DB, KVB = S::KVB;
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
  const uint32_t n = lane & 15u;   // the lane's row within a 16-row block
  const uint32_t gp = lane >> 4;   // lane group
  const uint32_t L = a.kv_seq_len;

  // ---- rows of this wavefront ----
  const uint32_t row0 = rt * S::RPW;
  const uint32_t wrow0 = row0 + wave * 16u * RB;
  // last valid row of the workgroup (padding rows copy its node, so that
  // every row of a wavefront sees some key whenever a real row does)
  const uint32_t wg_last = min(row0 + S::RPW, a.rows) - 1u;
  uint32_t node[RB];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t gr = wrow0 + 16u * rb + n;
    valid[rb] = gr < a.rows;
    node[rb] = (valid[rb] ? gr : wg_last) / a.group;
  }
  // node range of the wavefront (wave-uniform)
  const uint32_t w_first = min(wrow0, wg_last), w_last = min(wrow0 + 16u * RB - 1u, wg_last);
  const uint32_t nlo = __builtin_amdgcn_readfirstlane(w_first / a.group);
  const uint32_t nhi = __builtin_amdgcn_readfirstlane(w_last / a.group);

  const size_t kvbase = (size_t)hk * a.kv_capacity * D;
  const half_t *K = static_cast<const half_t *>(a.k) + kvbase;
  const half_t *V = static_cast<const half_t *>(a.v) + kvbase;

  // ---- per-lane constants of the loop ----
  floatx32 OFF;
  floatx8 MISC;        // v240..v247
  floatx2 MISC2;       // v248..v249
  floatx4 KVROW;       // a208..a211

#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    OFF[ds] = __uint_as_float(lds0 + n * (D * 2) + 16u * swz(n, 4u * ds + gp));
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const uint32_t r0 = 4u * gp + (n >> 2), ch = 2u * db + ((n & 3u) >> 1);
    OFF[8 + db] = __uint_as_float(lds0 + NS * KVB + r0 * (D * 2) + 16u * swz_v<S::CH>(r0, ch) +
                                  8u * (n & 1u));
  }
  uint32_t k_off[S::KV_PW], v_off[S::KV_PW];
#pragma unroll
  for (int i = 0; i < S::KV_PW; ++i) {
    const uint32_t p = (wave * S::KV_PW + i) * 64u + lane;
    const uint32_t row = p / S::CH;
    k_off[i] = 2u * (row * D + 8u * swz(row, p % S::CH));
    v_off[i] = 2u * (row * D + 8u * swz_v<S::CH>(row, p % S::CH));
    OFF[24 + i] = __uint_as_float(k_off[i]);
    OFF[28 + i] = __uint_as_float(v_off[i]);
    KVROW[i] = __uint_as_float(row);
  }
  const uint32_t mask_lds = lds0 + 2 * NS * KVB + wave * S::MB;   // the wavefront's stage-0 mask area
  uint32_t mrow[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < (ML > 0 ? ML : 1); ++j) {
    const uint32_t nd = min(nlo + lane / 8u + 8u * j, nhi);
    mrow[j] = nd * a.mask_stride * 4u + 16u * (lane % 8u);
  }
  MISC[0] = __uint_as_float(mrow[0]);
  MISC[1] = __uint_as_float(mrow[1]);
  MISC[2] = __uint_as_float(mask_lds + 16u * lane);
  MISC[3] = __uint_as_float(16u * (lane % 8u));
  float clim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    MISC[4 + rb] = __uint_as_float(mask_lds + (node[rb] - nlo) * BN * 4u + 16u * gp);
    clim[rb] = __int_as_float((int32_t)((int64_t)L - (int64_t)a.q_l + (int64_t)node[rb]));
  }
  MISC[7] = clim[0];
  MISC2[0] = clim[1];
  MISC2[1] = clim[2];

  // ---- split range ----
  const uint32_t tile_lo = a.key_lo / BN;
  uint32_t t0, t1;
  uint32_t span_lo, span_hi;
  split_tiles(a, BN, tile_lo, span_lo, span_hi);
  split_range(span_hi - span_lo, a.nwg, split, t0, t1);
  t0 += span_lo;
  t1 += span_lo;
  // K (with the mask cells) and V of tile u into stage st of their rings
  auto issue_k = [&](uint32_t u, uint32_t st) __attribute__((always_inline)) {
    const uint32_t key0 = u * BN;
    const uint32_t lk = lds0 + st * KVB + wave * S::KV_PW * 1024u;
#pragma unroll
    for (int i = 0; i < S::KV_PW; ++i) {
      const uint32_t row = __float_as_uint(KVROW[i]);
      const uint32_t key = min(key0 + row, L - 1u);
      dma_b128_nt(reinterpret_cast<const char *>(K + (size_t)key * D) + (k_off[i] - 2u * row * D),
               lk + i * 1024u);
    }
    if constexpr (!IMPLICIT) {
      uint32_t key = key0 + 4u * (lane % 8u);
      if (key >= L) key = (L - 1u) & ~3u;
#pragma unroll
      for (int j = 0; j < ML; ++j)
        dma_b128_nt(reinterpret_cast<const char *>(a.mask) + (mrow[j] - 16u * (lane % 8u)) + 4u * key,
                 mask_lds + st * (W * S::MB) + j * 1024u);
    }
  };
  auto issue_v = [&](uint32_t u, uint32_t st) __attribute__((always_inline)) {
    const uint32_t key0 = u * BN;
    const uint32_t lv = lds0 + NS * KVB + st * KVB + wave * S::KV_PW * 1024u;
#pragma unroll
    for (int i = 0; i < S::KV_PW; ++i) {
      const uint32_t row = __float_as_uint(KVROW[i]);
      const uint32_t key = min(key0 + row, L - 1u);
      dma_b128_nt(reinterpret_cast<const char *>(V + (size_t)key * D) + (v_off[i] - 2u * row * D),
               lv + i * 1024u);
    }
  };

  floatx32 O0 = {}, O1 = {}, O2 = {}, O3 = {}, O4 = {}, O5 = {};
  floatx16 R = {}, CM = {};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) CM[12 + rb] = -INFINITY;
  CM[15] = __uint_as_float(4u * gp);
  if (t0 < t1) {
    const uint32_t tl = t1 - 1u;
    // The loop expects K (and mask cells) of tiles t0 .. t0+3 and V of
    // tiles t0 .. t0+2 in their stages (tiles past the split repeat its
    // last), tile t0's complete and the rest issued in the order
    // K1 V1 K2 V2 K3: its per-step wait then covers each of them in time.
    // Tile t0 goes out first; Q's loads follow it, and waiting for them
    // (loads complete in order) completes tile t0 without holding up on the
    // rest of the ring fill, which is issued after Q is in registers.
    issue_k(t0, 0);
    issue_v(t0, 0);
    // Q'^T fragments (Q * scale * log2(e), fp16): row n of each block,
    // d = 32 ds + 8 gp + 0..7
    floatx32 Qv[RB];
    const float qs = a.scale * kLog2e;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t gr = wrow0 + 16u * rb + n;
      const uint32_t head = hk * a.group + (valid[rb] ? gr % a.group : 0u);
      const float *qrow = a.q + ((size_t)head * a.q_l + node[rb]) * D;
      const float sc = valid[rb] ? qs : 0.0f;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const floatx4 w = q_fragment(qrow + 32 * ds, gp, sc);
#pragma unroll
        for (int k = 0; k < 4; ++k) Qv[rb][4 * ds + k] = w[k];
      }
    }
    // (Q in registers before the rest of the fill goes out)
    hold_vgprs(Qv[0], Qv[1], Qv[2]);
#pragma unroll
    for (uint32_t i = 1; i < 3u; ++i) {
      issue_k(min(t0 + i, tl), i);
      issue_v(min(t0 + i, tl), i);
    }
    issue_k(min(t0 + 3u, tl), 3u);
    const floatx4 ONES = __builtin_bit_cast(floatx4, u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u,
                                                             0x3C003C00u});
    wide_loop<ML>(O0, O1, O2, O3, O4, O5, R, CM, Qv[0], Qv[1], Qv[2], ONES, OFF, MISC, MISC2, KVROW,
                  t0, t1, L,
                  (uint64_t)(uintptr_t)K, (uint64_t)(uintptr_t)V, (uint64_t)(uintptr_t)a.mask,
                  lds0 + wave * S::KV_PW * 1024u, mask_lds, a.key_lo,
                  (int32_t)((int64_t)L - (int64_t)a.q_l + (int64_t)nlo), (L - 1u) & ~3u);
  }

  // ---- results ----
  const size_t nrows = (size_t)a.n_heads * a.q_l;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float stot = R[4 * rb];
    if (!valid[rb]) continue;
    const uint32_t gr = wrow0 + 16u * rb + n;
    const uint32_t head = hk * a.group + gr % a.group;
    const size_t rid = (size_t)node[rb] * a.n_heads + head;
    const floatx32 &Oa = rb == 0 ? O0 : rb == 1 ? O2 : O4;
    const floatx32 &Ob = rb == 0 ? O1 : rb == 1 ? O3 : O5;
    const float inv = (stot > 0.0f) ? 1.0f / stot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const floatx32 &Os = db < 8 ? Oa : Ob;
      const int b = 4 * (db % 8);
      const floatx4 o = {Os[b], Os[b + 1], Os[b + 2], Os[b + 3]};
      if (a.nwg == 1)
        *reinterpret_cast<floatx4 *>(a.out + rid * D + 16 * db + 4 * gp) = o * inv;
      else
        *reinterpret_cast<floatx4 *>(a.part_o + ((size_t)split * nrows + rid) * D + 16 * db + 4 * gp) = o;
    }
    if (a.nwg > 1 && gp == 0) {
      const size_t prow = (size_t)split * nrows + rid;
      a.part_sm[prow * 2 + 0] = stot;
      a.part_sm[prow * 2 + 1] = CM[12 + rb];
    }
  }
}

template <int D, int RB, int ML>
hipError_t launch_w(const FwdArgs &a, hipStream_t s) {
  using Sh = WideShape<D, RB, ML>;
  static const bool attr_set = [] {
    (void)hipFuncSetAttribute((const void *)fwd_wide_kernel<D, RB, ML>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    return true;
  }();
  (void)attr_set;
  dim3 grid(grid_size(a.units, a.row_tiles));
  hipLaunchKernelGGL((fwd_wide_kernel<D, RB, ML>), grid, dim3(64 * W), Sh::LDS, s, a);
  return hipGetLastError();
}

// 16-byte mask copies per lane a wavefront's 48 rows need (their nodes, one
// 32-key tile: 8 nodes per copy); 0 if more than two.  A wavefront's first
// row is a multiple of 48, so when the group divides 48 its rows span exactly
// 48 / group nodes; otherwise at most one more than the rounded-up quotient.
uint32_t wide_mask_loads(uint32_t group) {
  const uint32_t nodes = 48u % group == 0u ? 48u / group : (48u + group - 1u) / group + 1u;
  const uint32_t ml = (nodes + 7u) / 8u;
  return ml <= 2u ? ml : 0u;
}

}  // namespace

constexpr uint32_t kWideRB = 3;

bool wide_applies(uint32_t head_dim, uint32_t rows, uint32_t group, bool implicit, bool mask_vec) {
  if (head_dim != 256) return false;
  if (rows < W * 16u * kWideRB) return false;
  if (implicit) return true;
  return mask_vec && wide_mask_loads(group) != 0u;
}

uint32_t wide_rows_per_wg() { return W * 16u * kWideRB; }

hipError_t launch_forward_wide(const FwdArgs &a, uint32_t head_dim, hipStream_t s) {
  if (head_dim != 256) return hipErrorInvalidValue;
  if (a.mask == nullptr) return launch_w<256, kWideRB, 0>(a, s);
  switch (wide_mask_loads(a.group)) {
    case 1: return launch_w<256, kWideRB, 1>(a, s);
    case 2: return launch_w<256, kWideRB, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
