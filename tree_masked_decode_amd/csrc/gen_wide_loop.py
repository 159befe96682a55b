#!/usr/bin/env python3
"""Generate fwd_wide_loop.inc: the tile loop of the wide fp16 forward
(fwd_wide.hip) as one CDNA4 inline-assembly block per mask mode.

The loop is written out instruction by instruction because its schedule is
the point: one wavefront per SIMD keeps O (48 rows x 256 dims, fp32) in the
accumulation registers, Q'^T (48 rows) in ordinary registers, and streams
each 32-key tile's K and V operands from LDS into a six-slot register ring
four operands ahead of the matrix instructions that use them; the softmax of
tile t (exp2 + fp16 packing + a packed-integer range check) is interleaved
with the score instructions of tile t+1.  The compiler, given the same work
in C++, serialises the LDS reads behind their matrix instructions and moves
accumulators between register files every tile.

Usage: python gen_wide_loop.py  (writes fwd_wide_loop.inc next to itself).

Register map (fixed; fwd_wide.hip binds its variables to these ranges):
  a[0:191]    O^T accumulators, block (rb, db) at a[64 rb + 4 db : +3]
  a[192:203]  row sums (ones . P^T), rb at a[192 + 4 rb : +3]
  a[204:206]  the reference max the pending scores were issued with, saved
              when a slow step moves M (see "stale" below)
  a[212:235]  score accumulators of the next tile, (rb, kb) at a[212 + 8 rb + 4 kb : +3]
  a[236:247]  score accumulator input -M' (four copies), rb at a[236 + 4 rb : +3]
  v[0:95]     Q'^T fragments, (rb, ds) at v[32 rb + 4 ds : +3]
  v[96:119]   the current tile's scores, copied out of a[212:235] at the top
              of each step, (rb, kb) at v[96 + 8 rb + 4 kb : +3]
  v[120:143]  per-cell accumulator inputs, staged for a[212:235] (slow paths)
  v[144:155]  P^T fragments (fp16), rb at v[144 + 4 rb : +3]
  v[156:159]  a half8 of ones (row-sum operand)
  v[160:162]  -M' of each row block (the value a[236:247] holds, for the VALU)
  v[172:174]  reference max M of each row block (base 2; -inf until a key is seen)
  v[175]      4 gp
  v[176:199]  operand ring, 6 slots of 4 registers; temporaries in the slow paths
  v[200:207]  softmax temporaries
  v[208:215]  LDS address of K chunk (n, 4 ds + gp) of stage 0 (with the swizzle)
  v[216:231]  LDS address of the V^T read of d-block db, stage 0
  v[232:235]  byte offset of K copy i within a full tile (V at v[236:239])
  v[240:241]  byte offset of the mask copy j of this lane (its node row + 16 (lane % 8))
  v[242]      LDS address of this lane's 16 bytes of the stage-0 mask area
  v[243]      16 (lane % 8)
  v[244:246]  LDS address of row block rb's mask cells (node - nlo) * 128 + 16 gp, stage 0
  v[247:249]  last key row block rb may see under the implicit rule (L - q_l + node)
  a[208:211]  tile row of K/V copy i
  (v[250:255] stay free for the compiler's whole-wave register needs)
SGPRs s80..s99 are the loop's own (declared clobbered):
  s80 t  s81 last tile  s82 flags (bit 0: every M finite, bit 1: stale)
  s83 s84 temporaries  s85 fetch tile u  s[86:87] K tile pointer
  s[88:89] V tile pointer  s[90:91] mask tile pointer  s92 first key of u
  s93 next tile tn  s94 first key of tn  s95 L - 1  s[96:97] return address
  s[98:99] 64-bit temporary, and the return address of the rescale

Every matrix instruction accumulates in the accumulation registers: a
wavefront that mixes matrix instructions accumulating in ordinary registers
with ones accumulating in accumulation registers issues them at about half
rate (measured: 30 instead of 16 cycles each), so the scores are accumulated
in a[212:235] and copied to ordinary registers for the softmax.

Hazards (gfx950, as the compiler itself spaces them): a matrix result read by
a VALU needs 8 wait states, a VALU result read by a matrix instruction 2, an
exp result read by a VALU 1, a VALU result read by v_permlane*_swap 2.  The
loop never reads a matrix result within 8 instructions of the instruction
that writes it; where the distance is not structural it pads with s_nop.
"""

import os

D, RB, W, NS, BN = 256, 3, 4, 4, 32
KVB = BN * D * 2          # bytes of one K (or V) tile
DS, DB = D // 32, D // 16
KV_PW = KVB // 1024 // W  # 1 KB copies per wavefront per K (or V) tile
# Operand ring slots (4 registers each); the first six double as the slow
# paths' temporaries and the mask words of the class check, the rest as the
# staging of per-cell accumulator inputs (slow paths, no reads in flight).
# AHEAD_A / AHEAD_B: operand reads in flight ahead of the matrix instructions
# in the score / PV region; the ring slot a read fills is that of the step
# before the current one, already consumed.
SLOTS = [176, 180, 184, 188, 192, 196, 120, 124, 128, 132, 136, 140]
AHEAD_A = int(os.environ.get("TA_AHEAD_A", "5"))
AHEAD_B = int(os.environ.get("TA_AHEAD_B", "5"))
RING = max(6, max(AHEAD_A, AHEAD_B) + 1)
assert RING <= len(SLOTS)
assert 2 * AHEAD_B <= 15 and AHEAD_A <= 15   # the LDS counter holds 15
# Cache policy of the K / V / mask copies: non-temporal.  Each 1 KB copy is
# read once into LDS (the other row tile of its tile reads it at about the
# same time); measured on the 32K tree, the tile loop ran 52.8 -> 47.5 us.
CPOL = "nt"
LAZY = 15.0               # the reference max moves when a tile's row max exceeds it by > 15 (base 2)
LAZY_F16 = 0x7800         # 2^15 as fp16 bits: a fast-path p above it needs a new reference

F32_NEG65504 = 0xC77FE000
F32_LOG2E = 0x3FB8AA3B
F32_NEGINF = 0xFF800000
F32_LAZY = 0x41700000     # 15.0


def r4(base):
    return "v[%d:%d]" % (base, base + 3)


def O(rb, db):
    b = 64 * rb + 4 * db
    return "a[%d:%d]" % (b, b + 3)


def RS(rb):
    b = 192 + 4 * rb
    return "a[%d:%d]" % (b, b + 3)


def AREF(rb):
    return "a%d" % (204 + rb)


def Q(rb, ds):
    return r4(32 * rb + 4 * ds)


def SA(rb, kb, j=None):
    b = 212 + 8 * rb + 4 * kb
    return ("a[%d:%d]" % (b, b + 3)) if j is None else "a%d" % (b + j)


def SV(rb, kb, j=None):
    b = 96 + 8 * rb + 4 * kb
    return r4(b) if j is None else "v%d" % (b + j)


def SSTG(rb, kb, j):
    return "v%d" % (120 + 8 * rb + 4 * kb + j)


def P(rb, k=None):
    b = 144 + 4 * rb
    return r4(b) if k is None else "v%d" % (b + k)


ONES = "v[156:159]"


def C(rb, j=None):
    b = 236 + 4 * rb
    return ("a[%d:%d]" % (b, b + 3)) if j is None else "a%d" % (b + j)


def CV(rb):
    return "v%d" % (160 + rb)


def M2(rb):
    return "v%d" % (172 + rb)


def B(i):
    return r4(SLOTS[i % RING])


def Blo(i):
    b = SLOTS[i % RING]
    return "v[%d:%d]" % (b, b + 1)


def Bhi(i):
    b = SLOTS[i % RING]
    return "v[%d:%d]" % (b + 2, b + 3)


def T(k):
    return "v%d" % (200 + k)


def OFFK(ds):
    return "v%d" % (208 + ds)


def OFFV(db):
    return "v%d" % (216 + db)


def KOFF(i):
    return "v%d" % (232 + i)


def VOFF(i):
    return "v%d" % (236 + i)


MROW = ["v240", "v241"]
MCHK = "v242"
M16 = "v243"


def MCELL(rb):
    return "v%d" % (244 + rb)


def CLIM(rb):
    return "v%d" % (247 + rb)


def KVROW(i):
    return "a%d" % (208 + i)


GP4 = "v175"


class Gen:
    def __init__(self, ml):
        self.ml = ml            # 0: implicit causal rule; 1 or 2: mask copies per lane per tile
        self.lines = []

    def e(self, s):
        # labels carry the asm instance's unique number (%=): the three mask
        # modes are three asm statements in one object file
        if s.startswith("s_branch ") or s.startswith("s_cbranch_"):
            s += "_%="
        self.lines.append(s)

    def label(self, name):
        self.lines.append(name + "_%=:")

    @property
    def pt(self):
        return 2 * KV_PW + self.ml

    def mask_stage(self, st):
        return st * W * self.ml * 1024

    # ---- copies: K (+ mask cells) of tile t+4 into K stage st, V of tile
    # t+3 into V stage st+3.  K and V rings are separate, so each part is
    # fetched three steps before the step that reads it: tile t+4's K is read
    # at step t+3 (scores of the next tile) and tile t+3's V at step t+3. ----
    def dma_part(self, st, part, ahead, stage):
        e = self.e
        tag = "%d_%d" % (st, part)
        e("s_add_u32 s85, s80, %d" % ahead)
        e("s_min_u32 s85, s85, s81")
        e("s_lshl_b32 s92, s85, 5")
        e("s_add_u32 s83, s92, 32")
        e("s_cmp_le_u32 s83, %[L]")
        e("s_cbranch_scc0 .Lwpdma%s" % tag)
        off = KOFF if part == 0 else VOFF
        base = ("%[kb0]", "%[kb1]") if part == 0 else ("%[vb0]", "%[vb1]")
        lbase = part * NS * KVB + stage * KVB
        e("s_lshl_b32 s83, s85, 14")
        e("s_add_u32 s86, %s, s83" % base[0])
        e("s_addc_u32 s87, %s, 0" % base[1])
        for i in range(KV_PW):
            e("s_add_u32 m0, %%[m0k], %d" % (lbase + i * 1024))
            e(("global_load_lds_dwordx4 %s, s[86:87] " + CPOL) % off(i))
        if part == 0 and self.ml:
            e("s_lshl_b32 s83, s92, 2")
            e("s_add_u32 s90, %[mb0], s83")
            e("s_addc_u32 s91, %[mb1], 0")
            for j in range(self.ml):
                e("s_add_u32 m0, %%[m0m], %d" % (self.mask_stage(stage) + j * 1024))
                e(("global_load_lds_dwordx4 %s, s[90:91] " + CPOL) % MROW[j])
        e("s_branch .Lwdmad%s" % tag)
        # a tile that ends past kv_seq_len: per-lane rows clamped to L - 1
        self.label(".Lwpdma%s" % tag)
        e("s_mov_b32 s98, %s" % base[0])
        e("s_mov_b32 s99, %s" % base[1])
        for i in range(KV_PW):
            e("v_accvgpr_read_b32 %s, %s" % (T(5), KVROW(i)))
            e("v_lshlrev_b32 %s, 9, %s" % (T(0), T(5)))
            e("v_sub_u32 %s, %s, %s" % (T(0), off(i), T(0)))
            e("v_add_u32 %s, s92, %s" % (T(1), T(5)))
            e("v_min_u32 %s, s95, %s" % (T(1), T(1)))
            e("v_lshl_add_u32 %s, %s, 9, %s" % (T(1), T(1), T(0)))
            e("s_add_u32 m0, %%[m0k], %d" % (lbase + i * 1024))
            e(("global_load_lds_dwordx4 %s, s[98:99] " + CPOL) % T(1))
        if part == 0 and self.ml:
            # key of the lane's chunk, clamped to the chunk that holds L - 1
            e("v_lshrrev_b32 %s, 2, %s" % (T(2), M16))
            e("v_add_u32 %s, s92, %s" % (T(2), T(2)))
            e("v_cmp_gt_u32_e32 vcc, %%[L], %s" % T(2))
            e("v_mov_b32 %s, %%[lclamp]" % T(3))
            e("v_cndmask_b32_e32 %s, %s, %s, vcc" % (T(2), T(3), T(2)))
            e("v_lshlrev_b32 %s, 2, %s" % (T(2), T(2)))
            e("s_mov_b32 s98, %[mb0]")
            e("s_mov_b32 s99, %[mb1]")
            for j in range(self.ml):
                e("v_sub_u32 %s, %s, %s" % (T(4), MROW[j], M16))
                e("v_add_u32 %s, %s, %s" % (T(4), T(4), T(2)))
                e("s_add_u32 m0, %%[m0m], %d" % (self.mask_stage(stage) + j * 1024))
                e(("global_load_lds_dwordx4 %s, s[98:99] " + CPOL) % T(4))
        self.label(".Lwdmad%s" % tag)

    def dma(self, st):
        self.dma_part(st, 0, 4, st)
        self.dma_part(st, 1, 3, (st + 3) % NS)

    # ---- the same copies spread over the score instructions: issued as one
    # burst at the top of a step they held the wavefront's in-order issue
    # (no matrix instruction can pass a copy waiting for the address unit),
    # with all four wavefronts bursting at once.  dma_setup computes both
    # parts' scalar bases, or branches to `partial` when either tile reaches
    # past kv_seq_len (those steps keep the burst with per-lane clamping);
    # dma_list gives the (M0, copy) pairs that region_a interleaves. ----
    def dma_setup(self, st, partial):
        e = self.e
        e("s_add_u32 s85, s80, 4")          # K (and mask) tile of this step
        e("s_min_u32 s85, s85, s81")
        e("s_lshl_b32 s92, s85, 5")
        e("s_add_u32 s83, s92, 32")
        e("s_cmp_le_u32 s83, %[L]")
        e("s_cbranch_scc0 %s" % partial)
        e("s_add_u32 s84, s80, 3")          # V tile of this step
        e("s_min_u32 s84, s84, s81")
        e("s_lshl_b32 s83, s84, 5")
        e("s_add_u32 s83, s83, 32")
        e("s_cmp_le_u32 s83, %[L]")
        e("s_cbranch_scc0 %s" % partial)
        e("s_lshl_b32 s83, s85, 14")
        e("s_add_u32 s86, %[kb0], s83")
        e("s_addc_u32 s87, %[kb1], 0")
        e("s_lshl_b32 s83, s84, 14")
        e("s_add_u32 s88, %[vb0], s83")
        e("s_addc_u32 s89, %[vb1], 0")
        if self.ml:
            e("s_lshl_b32 s83, s92, 2")
            e("s_add_u32 s90, %[mb0], s83")
            e("s_addc_u32 s91, %[mb1], 0")

    def dma_list(self, st):
        pairs = []
        kl = st * KVB
        for i in range(KV_PW):
            pairs.append(["s_add_u32 m0, %%[m0k], %d" % (kl + i * 1024),
                          ("global_load_lds_dwordx4 %s, s[86:87] " + CPOL) % KOFF(i)])
        for j in range(self.ml):
            pairs.append(["s_add_u32 m0, %%[m0m], %d" % (self.mask_stage(st) + j * 1024),
                          ("global_load_lds_dwordx4 %s, s[90:91] " + CPOL) % MROW[j]])
        vl = NS * KVB + ((st + 3) % NS) * KVB
        for i in range(KV_PW):
            pairs.append(["s_add_u32 m0, %%[m0k], %d" % (vl + i * 1024),
                          ("global_load_lds_dwordx4 %s, s[88:89] " + CPOL) % VOFF(i)])
        return pairs

    def class_read(self, stn):
        """Issue the mask-word reads of tile tn's class check (into the idle
        operand ring) so that their latency hides behind the copy issue."""
        if self.ml:
            self.e("ds_read_b128 v[176:179], %s offset:%d" % (MCHK, self.mask_stage(stn)))
            if self.ml == 2:
                self.e("ds_read_b128 v[180:183], %s offset:%d" % (MCHK, self.mask_stage(stn) + 1024))

    def class_check(self, tag, stn, slow_label, read_done=False):
        e = self.e
        if self.ml and not read_done:
            self.class_read(stn)
        e("s_add_u32 s83, s94, 32")
        e("s_cmp_le_u32 s83, %[L]")
        if self.ml:
            # (the mask words may still be arriving in the ring that the
            # per-cell path reuses)
            e("s_waitcnt lgkmcnt(0)")
        e("s_cbranch_scc0 %s" % slow_label)
        if self.ml == 0:
            e("s_cmp_lt_u32 s94, %[keylo]")
            e("s_cbranch_scc1 %s" % slow_label)
            e("s_add_u32 s83, s94, 31")
            e("s_cmp_gt_i32 s83, %[climit]")
            e("s_cbranch_scc1 %s" % slow_label)
        else:
            e("s_waitcnt lgkmcnt(0)")
            e("v_or3_b32 %s, v176, v177, v178" % T(0))
            e("v_or_b32_e32 %s, %s, v179" % (T(0), T(0)))
            if self.ml == 2:
                e("v_or3_b32 %s, %s, v180, v181" % (T(0), T(0)))
                e("v_or3_b32 %s, %s, v182, v183" % (T(0), T(0)))
            e("v_cmp_ne_u32_e32 vcc, 0, %s" % T(0))
            e("s_cmp_eq_u64 vcc, 0")
            e("s_cbranch_scc0 %s" % slow_label)

    # ---- per-cell accumulator inputs of tile tn into score buffer nxt ----
    def slow_class(self, stn, nxt):
        e = self.e
        e("v_add_u32 %s, s94, %s" % (T(0), GP4))        # key of the lane's first cell (kb 0, j 0)
        if self.ml:
            e("v_sub_u32 %s, %%[L], %s" % (T(1), T(0)))  # keys left in range from there (signed)
            for rb in range(RB):
                for kb in range(2):
                    e("ds_read_b128 %s, %s offset:%d" % (B(2 * rb + kb), MCELL(rb), self.mask_stage(stn) + 64 * kb))
            e("s_waitcnt lgkmcnt(0)")
            e("s_mov_b32 s83, 0x%08x" % F32_NEG65504)
            e("s_mov_b32 s84, 0x%08x" % F32_LOG2E)
            e("v_mov_b32_e32 %s, 0x%08x" % (T(3), F32_NEGINF))
            for rb in range(RB):
                for kb in range(2):
                    xb = SLOTS[2 * rb + kb]
                    for j in range(4):
                        x = "v%d" % (xb + j)
                        e("v_cmp_gt_i32_e64 s[98:99], %s, %d" % (T(1), 16 * kb + j))
                        e("v_cmp_lt_f32_e32 vcc, s83, %s" % x)
                        e("s_and_b64 vcc, vcc, s[98:99]")
                        e("v_fma_f32 %s, %s, s84, %s" % (T(2), x, CV(rb)))
                        e("v_cndmask_b32_e32 %s, %s, %s, vcc" % (SSTG(rb, kb, j), T(3), T(2)))
        else:
            e("v_mov_b32_e32 %s, 0x%08x" % (T(3), F32_NEGINF))
            for rb in range(RB):
                for kb in range(2):
                    for j in range(4):
                        e("v_add_u32 %s, %d, %s" % (T(2), 16 * kb + j, T(0)))
                        e("v_cmp_ge_i32_e64 s[98:99], %s, %s" % (CLIM(rb), T(2)))
                        e("v_cmp_gt_u32_e32 vcc, %%[L], %s" % T(2))
                        e("s_and_b64 vcc, vcc, s[98:99]")
                        e("v_cmp_le_u32_e64 s[98:99], %%[keylo], %s" % T(2))
                        e("s_and_b64 vcc, vcc, s[98:99]")
                        e("v_cndmask_b32_e32 %s, %s, %s, vcc" % (SSTG(rb, kb, j), T(3), CV(rb)))
        for rb in range(RB):
            for kb in range(2):
                for j in range(4):
                    e("v_accvgpr_write_b32 %s, %s" % (SA(rb, kb, j), SSTG(rb, kb, j)))
        e("s_nop 2")

    # ---- the fast softmax of buffer cur: exp2, fp16 packing, range check ----
    def softmax_list(self, cur):
        L = []
        for rb in range(RB):
            for kb in range(2):
                for j in range(4):
                    L.append("v_exp_f32_e32 %s, %s" % (T(4 * kb + j), SV(rb, kb, j)))
            for k in range(4):
                L.append("v_cvt_pk_f16_f32 %s, %s, %s" % (P(rb, k), T(2 * k), T(2 * k + 1)))
        words = [P(rb, k) for rb in range(RB) for k in range(4)]
        L.append("v_pk_max_u16 %s, %s, %s" % (T(0), words[0], words[1]))
        for w in words[2:]:
            L.append("v_pk_max_u16 %s, %s, %s" % (T(0), T(0), w))
        # both halves saturate to 0 unless above the bound
        L.append("v_pk_sub_u16 %s, %s, s84 clamp" % (T(1), T(0)))
        L.append("v_cmp_ne_u32_e32 vcc, 0, %s" % T(1))
        return L

    # ---- scores of tile tn (stage stn) into buffer nxt, with the softmax of cur interleaved ----
    def region_a(self, stn, nxt, cur, fast_c, with_softmax, dma=()):
        e = self.e
        valu = self.softmax_list(cur) if with_softmax else []
        if with_softmax:
            e("s_mov_b32 s84, 0x%04x%04x" % (LAZY_F16, LAZY_F16))
        per = [[] for _ in range(16)]
        # spread the copies (one per operand step from the first) and the
        # VALU work over the 16 operand steps
        for idx, pair in enumerate(dma):
            per[min(15, idx * 16 // max(1, len(dma)))].extend(pair)
        for idx, ins in enumerate(valu):
            per[min(15, idx * 16 // max(1, len(valu)))].append(ins)
        nread = 16

        def kread(i):
            ds, kb = i >> 1, i & 1
            e("ds_read_b128 %s, %s offset:%d" % (B(i), OFFK(ds), stn * KVB + kb * 16 * D * 2))
        for i in range(AHEAD_A):
            kread(i)
        for i in range(16):
            ds, kb = i >> 1, i & 1
            # one wait covers two steps (steps i and i+1)
            if i % 2 == 0:
                issued = min(nread, i + AHEAD_A)
                e("s_waitcnt lgkmcnt(%d)" % max(0, issued - min(nread, i + 2)))
            for rb in range(RB):
                src_c = C(rb) if fast_c and ds == 0 else SA(rb, kb)
                e("v_mfma_f32_16x16x32_f16 %s, %s, %s, %s" % (SA(rb, kb), B(i), Q(rb, ds), src_c))
            if i + AHEAD_A < nread:
                kread(i + AHEAD_A)
            for ins in per[i]:
                e(ins)

    # ---- O^T += V^T P^T and the row sums, stage st ----
    def region_b(self, st):
        e = self.e
        e("s_nop 1")
        for rb in range(RB):
            e("v_mfma_f32_16x16x32_f16 %s, %s, %s, %s" % (RS(rb), ONES, P(rb), RS(rb)))

        def vread(db):
            e("ds_read_b64_tr_b16 %s, %s offset:%d" % (Blo(db), OFFV(db), st * KVB))
            e("ds_read_b64_tr_b16 %s, %s offset:%d" % (Bhi(db), OFFV(db), st * KVB + 16 * D * 2))
        for db in range(AHEAD_B):
            vread(db)
        for db in range(DB):
            # one wait covers two d-blocks
            if db % 2 == 0:
                issued = 2 * min(DB, db + AHEAD_B)
                e("s_waitcnt lgkmcnt(%d)" % max(0, issued - 2 * min(DB, db + 2)))
            for rb in range(RB):
                e("v_mfma_f32_16x16x32_f16 %s, %s, %s, %s" % (O(rb, db), B(db), P(rb), O(rb, db)))
            if db + AHEAD_B < DB:
                vread(db + AHEAD_B)

    def step(self, st):
        e = self.e
        cur, nxt, stn = st & 1, (st & 1) ^ 1, (st + 1) % NS
        self.label(".Lwstep%d" % st)
        # tile t's scores out of the accumulation registers (region A below
        # overwrites them with tile t+1's); before the wait, which they overlap
        for rb in range(RB):
            for kb in range(2):
                for j in range(4):
                    e("v_accvgpr_read_b32 %s, %s" % (SV(rb, kb, j), SA(rb, kb, j)))
        e("s_waitcnt vmcnt(%d)" % (2 * self.pt))
        e("s_barrier")
        self.class_read(stn)
        e("s_add_u32 s93, s80, 1")
        e("s_min_u32 s93, s93, s81")
        e("s_lshl_b32 s94, s93, 5")
        self.dma_setup(st, ".Lwdmap%d" % st)
        dl = self.dma_list(st)
        self.class_check(st, stn, ".Lwcslow%d" % st, read_done=True)
        self.region_a(stn, nxt, cur, True, True, dl)
        e("s_branch .Lwadone%d" % st)
        self.label(".Lwcslow%d" % st)
        self.slow_class(stn, nxt)
        self.region_a(stn, nxt, cur, False, True, dl)
        e("s_branch .Lwadone%d" % st)
        # a copy tile reaches past kv_seq_len (the last tiles of a split):
        # the burst with per-lane clamping, then the per-cell scores (the
        # class words may still be landing in the operand ring)
        self.label(".Lwdmap%d" % st)
        e("s_waitcnt lgkmcnt(0)")
        self.dma(st)
        self.slow_class(stn, nxt)
        self.region_a(stn, nxt, cur, False, True)
        self.label(".Lwadone%d" % st)
        # fast path kept iff no p above the bound, every M finite and none stale
        e("s_cmp_eq_u64 vcc, 0")
        e("s_cselect_b32 s83, s82, 0")
        e("s_cmp_eq_u32 s83, 1")
        e("s_cbranch_scc1 .Lwpv%d" % st)
        e("s_getpc_b64 s[96:97]")
        e("s_add_u32 s96, s96, 12")
        e("s_addc_u32 s97, s97, 0")
        e("s_branch .Lwsslow%d" % cur)
        self.label(".Lwpv%d" % st)
        self.region_b(st)
        e("s_add_u32 s80, s80, 1")
        e("s_cmp_ge_u32 s80, %[t1]")
        e("s_cbranch_scc1 .Lwend")

    # ---- slow softmax of buffer cur (called; returns through s[96:97]) ----
    def slow_softmax(self, cur):
        e = self.e
        self.label(".Lwsslow%d" % cur)
        ref, tmx, tmp, mnew, msub = "v176", "v177", "v178", "v180", "v181"
        e("s_mov_b64 s[86:87], 0")          # rows whose M moves
        e("s_mov_b64 s[88:89], 0")          # rows that need O rescaled
        e("s_mov_b64 s[90:91], exec")       # rows whose M is finite
        e("s_mov_b32 s84, 0x%08x" % F32_NEGINF)
        for rb in range(RB):
            alpha = "v%d" % (184 + rb)
            # the reference the scores were issued with
            e("s_bitcmp1_b32 s82, 1")
            e("s_cbranch_scc1 .Lwref%d_%d" % (cur, rb))
            e("v_sub_f32_e32 %s, 0, %s" % (ref, CV(rb)))
            e("s_branch .Lwrefd%d_%d" % (cur, rb))
            self.label(".Lwref%d_%d" % (cur, rb))
            e("v_accvgpr_read_b32 %s, %s" % (ref, AREF(rb)))
            self.label(".Lwrefd%d_%d" % (cur, rb))
            for kb in range(2):
                for j in range(4):
                    e("v_add_f32_e32 %s, %s, %s" % (T(4 * kb + j), SV(rb, kb, j), ref))
            e("v_max3_f32 %s, %s, %s, %s" % (tmx, T(0), T(1), T(2)))
            e("v_max3_f32 %s, %s, %s, %s" % (tmx, tmx, T(3), T(4)))
            e("v_max3_f32 %s, %s, %s, %s" % (tmx, tmx, T(5), T(6)))
            e("v_max_f32_e32 %s, %s, %s" % (tmx, tmx, T(7)))
            for sw in ("v_permlane16_swap_b32_e32", "v_permlane32_swap_b32_e32"):
                e("v_mov_b32_e32 %s, %s" % (tmp, tmx))
                e("s_nop 1")
                e("%s %s, %s" % (sw, tmx, tmp))
                e("v_max_f32_e32 %s, %s, %s" % (tmx, tmx, tmp))
            # mnew = tmax if tmax > M + LAZY (also when M is -inf and tmax is not), else M
            e("v_add_f32_e32 %s, 0x%08x, %s" % (tmp, F32_LAZY, M2(rb)))
            e("v_cmp_gt_f32_e32 vcc, %s, %s" % (tmx, tmp))
            e("v_cndmask_b32_e32 %s, %s, %s, vcc" % (mnew, M2(rb), tmx))
            # alpha = 2^(M - mnew) where a finite M moves, else 1 (O and the
            # row sum are still zero while M is -inf)
            e("v_sub_f32_e32 %s, %s, %s" % (alpha, M2(rb), mnew))
            e("v_exp_f32_e32 %s, %s" % (alpha, alpha))
            e("v_cmp_neq_f32_e32 vcc, %s, %s" % (mnew, M2(rb)))
            e("s_or_b64 s[86:87], s[86:87], vcc")
            e("v_cmp_neq_f32_e64 s[98:99], s84, %s" % M2(rb))
            e("s_and_b64 vcc, vcc, s[98:99]")
            e("v_cndmask_b32_e32 %s, 1.0, %s, vcc" % (alpha, alpha))
            e("v_cmp_neq_f32_e32 vcc, 1.0, %s" % alpha)
            e("s_or_b64 s[88:89], s[88:89], vcc")
            # the scores of the next tile were issued with the current -C
            e("v_sub_f32_e32 %s, 0, %s" % (tmp, CV(rb)))
            e("v_accvgpr_write_b32 %s, %s" % (AREF(rb), tmp))
            e("v_mov_b32_e32 %s, %s" % (M2(rb), mnew))
            # reference used from now on: mnew, or 0 while it is -inf
            e("v_cmp_neq_f32_e32 vcc, 0x%08x, %s" % (F32_NEGINF, mnew))
            e("s_and_b64 s[90:91], s[90:91], vcc")
            e("v_cndmask_b32_e32 %s, 0, %s, vcc" % (msub, mnew))
            e("v_sub_f32_e32 %s, 0, %s" % (CV(rb), msub))
            for j in range(4):
                e("v_accvgpr_write_b32 %s, %s" % (C(rb, j), CV(rb)))
            for k in range(8):
                e("v_sub_f32_e32 %s, %s, %s" % (T(k), T(k), msub))
            for k in range(8):
                e("v_exp_f32_e32 %s, %s" % (T(k), T(k)))
            e("s_nop 0")
            for k in range(4):
                e("v_cvt_pk_f16_f32 %s, %s, %s" % (P(rb, k), T(2 * k), T(2 * k + 1)))
        # flags: bit 0 every M finite, bit 1 some M moved (pending scores stale)
        e("s_cmp_eq_u64 s[90:91], exec")
        e("s_cselect_b32 s82, 1, 0")
        e("s_cmp_lg_u64 s[86:87], 0")
        e("s_cselect_b32 s83, 2, 0")
        e("s_or_b32 s82, s82, s83")
        e("s_cmp_eq_u64 s[88:89], 0")
        e("s_cbranch_scc1 .Lwsret%d" % cur)
        e("s_getpc_b64 s[98:99]")
        e("s_add_u32 s98, s98, 12")
        e("s_addc_u32 s99, s99, 0")
        e("s_branch .Lwrescale")
        self.label(".Lwsret%d" % cur)
        e("s_nop 1")
        e("s_setpc_b64 s[96:97]")

    # ---- O and the row sums times alpha (v184..v186), through ordinary registers ----
    def rescale(self):
        e = self.e
        self.label(".Lwrescale")
        e("s_nop 7")
        regs = ["v188", "v189", "v190", "v191"]
        blocks = [(rb, 64 * rb + 4 * db) for rb in range(RB) for db in range(DB)]
        blocks += [(rb, 192 + 4 * rb) for rb in range(RB)]
        for rb, a0 in blocks:
            for j in range(4):
                e("v_accvgpr_read_b32 %s, a%d" % (regs[j], a0 + j))
            for j in range(4):
                e("v_mul_f32_e32 %s, %s, v%d" % (regs[j], regs[j], 184 + rb))
            for j in range(4):
                e("v_accvgpr_write_b32 a%d, %s" % (a0 + j, regs[j]))
        e("s_nop 3")
        e("s_setpc_b64 s[98:99]")

    def build(self):
        e = self.e
        e("s_mov_b32 s80, %[t0]")
        e("s_sub_u32 s81, %[t1], 1")
        e("s_sub_u32 s95, %[L], 1")
        e("s_mov_b32 s82, 0")
        # -M' = 0 while every M is -inf (the ordinary-register copy v[160:162]
        # comes in as zero)
        for rb in range(RB):
            for j in range(4):
                e("v_accvgpr_write_b32 %s, 0" % C(rb, j))
        e("s_barrier")
        # scores of the first tile (stage 0)
        e("s_mov_b32 s93, s80")
        e("s_lshl_b32 s94, s93, 5")
        self.class_check("p", 0, ".Lwpcslow")
        self.region_a(0, 0, 1, True, False)
        e("s_branch .Lwpdone")
        self.label(".Lwpcslow")
        self.slow_class(0, 0)
        self.region_a(0, 0, 1, False, False)
        self.label(".Lwpdone")
        # (step 0 reads those scores at once: the matrix results' wait states)
        e("s_nop 7")
        e("s_nop 7")
        e("s_nop 7")
        for st in range(NS):
            self.step(st)
        e("s_branch .Lwstep0")
        for cur in range(2):
            self.slow_softmax(cur)
        self.rescale()
        self.label(".Lwend")
        e("s_waitcnt vmcnt(0)")
        e("s_nop 7")
        e("s_nop 7")
        return self.lines


def render():
    """The text of fwd_wide_loop.inc."""
    out = ["// Generated by gen_wide_loop.py -- do not edit.  The tile loop of the",
           "// wide fp16 forward, one string per mask mode (0: implicit causal rule,",
           "// 1 / 2: mask cells copied per tile, 16 bytes per lane per copy).",
           "#pragma once"]
    for ml in (0, 1, 2):
        lines = Gen(ml).build()
        out.append("#define TA_WIDE_LOOP_ML%d \\" % ml)
        for ln in lines:
            out.append('  "%s\\n" \\' % ln.replace('"', '\\"'))
        out.append('  ""')
    return "\n".join(out) + "\n"


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "fwd_wide_loop.inc"), "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
