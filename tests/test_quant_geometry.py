"""Host-side model of the quantized kernel's copy geometry and copy waits.

The quantized forward copies every 32-key tile global -> LDS with
global_load_lds instructions (16 or 4 bytes per lane) into a ring of NS
stages and waits for them with hand-counted vmcnt values; no barrier or
compiler-inserted wait guards those reads.  This module restates, in Python,
the kernel's stage layout, the per-lane source and destination of every copy
of a tile (full and partial tiles), the LDS words the arithmetic then reads,
and the order of copies and waits of the tile loop, and checks for each
configuration:

  * every copy stays inside the caller's buffers (packed codes, scales,
    biases, mask) and inside its own LDS stage;
  * every LDS byte read for a key below kv_seq_len was written by a copy of
    the same tile, from that key's own row (K / V words, scales, biases,
    mask cells of the right row);
  * when tile t is read, the wait before it leaves in flight only copies
    issued after tile t's last copy (loads complete in order), and never
    more than the 63 that a wavefront's counter tracks;
  * a tile's copy count is the PER_TILE the waits are counted with.

The configurations are the quantized GPU tests', the workloads', and the
geometry of a reverted variant that failed one parity case (head dim 512,
8-bit codes, group 32, u32 mask with 4-byte copies, kv_seq_len 97, two
splits).  The constants restate the shape structs of the kernel source
(QShape, MaskGeom, QStage); a change there must be mirrored here.
"""

import itertools
import math

import pytest

BN, LANES = 32, 64
F16, BF16, F32 = 0, 1, 2
NONE, B128, B32, REG, BOOL, BOOLB128 = range(6)


def shape(dim, bits, G, et, mm):
    S = {}
    S["ESZ"] = 4 if et == F32 else 2
    S["EPW"] = 4 // S["ESZ"]
    S["WPK"] = dim * bits // 32
    S["NG"] = dim // G
    S["KT"] = BN * S["WPK"] * 4
    S["KT_I"] = (S["KT"] + 1023) // 1024
    S["KT_TAIL"] = S["KT"] % 1024
    S["SBB"] = BN * S["NG"] * S["ESZ"]
    S["SB_WIDE"] = (S["NG"] * S["ESZ"]) % 16 == 0 and (4 * S["SBB"]) % 1024 == 0
    S["SB_W"] = 16 if S["SB_WIDE"] else 4
    S["SB_I"] = 4 * S["SBB"] // (64 * S["SB_W"])
    S["RS"] = BN + 4
    S["VL"] = S["WPK"] * S["RS"] * 4
    S["VTOT"] = BN * S["WPK"] // 4
    is_bool = mm in (BOOL, BOOLB128)
    dma = is_bool or mm in (B128, B32)
    wide = mm in (B128, BOOLB128)
    S["BOOL"], S["DMA"], S["WIDE"] = is_bool, dma, wide
    S["CB"] = 4 if is_bool else S["ESZ"]
    S["CPL"] = (16 if wide else 4) // S["CB"]
    S["LPR"] = BN // S["CPL"]
    S["RPC"] = LANES // S["LPR"]
    S["NC"] = 16 // S["RPC"] if dma else 0
    S["MBYTES"] = 16 * BN * S["CB"] if dma else 0
    S["MSTEP"] = 1024 if wide else 256
    if dma:
        assert S["RPC"] * S["LPR"] == LANES and S["NC"] * S["RPC"] == 16
    S["BYTES"] = 2 * S["KT"] + 4 * S["SBB"] + S["MBYTES"]
    S["PER_TILE"] = 2 * S["KT_I"] + S["SB_I"] + S["NC"]
    budget = 160 * 1024 // 12 if dim <= 128 else 48 * 1024
    S["NS"] = 3 if (3 * S["BYTES"] + S["VL"] <= budget and 2 * S["PER_TILE"] <= 63) else 2
    assert S["PER_TILE"] * (S["NS"] - 1) <= 63
    return S


def mask_mode(et, mask_kind, mhs, stride, L):
    """The launcher's choice of mask copy mode (16-byte aligned bases)."""
    if mask_kind is None:
        return NONE
    if mask_kind == "bool":
        return BOOLB128 if (mhs | stride | L) % 4 == 0 else BOOL
    esz = 4 if et == F32 else 2
    a = mhs | stride | L
    if a % (16 // esz) == 0:
        return B128
    if a % (4 // esz) == 0:
        return B32
    assert et != F32
    return REG


def tile_copies(S, t, L, cap, stream, rt, rows, repeat, kv, mhs, stride):
    """(buffer, src byte, lds byte, width) of every lane of every copy of
    tile t, copy by copy; LDS bytes relative to the stage."""
    key0 = t * BN
    WPK, NG, ESZ = S["WPK"], S["NG"], S["ESZ"]
    copies = []
    row = 4 * WPK                       # bytes of a token's codes
    base = stream * cap * row
    sbase = stream * cap * NG * ESZ
    full = key0 + BN <= L
    # K and V copies interleave per i: K_i, V_i
    for i in range(S["KT_I"]):
        ck, cv = [], []
        for lane in range(LANES):
            o = 1024 * i + 16 * lane
            if S["KT_TAIL"] and o >= S["KT"]:
                continue
            if full:
                src = base + key0 * row + o
            else:
                key = min(key0 + o // row, L - 1)
                src = base + key * row + o % row
            ck.append(("kp", src, 1024 * i + 16 * lane, 16))
            cv.append(("vp", src, S["KT"] + 1024 * i + 16 * lane, 16))
        copies += [ck, cv]
    arrs = ("ks", "kb", "vs", "vb")
    for i in range(S["SB_I"]):
        c = []
        for lane in range(LANES):
            o = S["SB_W"] * (64 * i + lane)
            arr = arrs[o // S["SBB"]]
            if full:
                src = sbase + key0 * NG * ESZ + o % S["SBB"]
            else:
                e = (o % S["SBB"]) // ESZ
                key = key0 + e // NG
                el = key * NG + e % NG
                if key >= L:
                    el = (max(L * NG - 2, 0) & ~1) if (ESZ == 2 and not S["SB_WIDE"]) else (
                        (L - 1) * NG + e % NG)
                src = sbase + el * ESZ
            step = 1024 if S["SB_WIDE"] else 256
            c.append((arr, src, 2 * S["KT"] + step * i + S["SB_W"] * lane, S["SB_W"]))
        copies.append(c)
    if S["DMA"]:
        for i in range(S["NC"]):
            c = []
            for lane in range(LANES):
                cell = key0 + S["CPL"] * (lane % S["LPR"])
                if cell >= L:
                    cell = L - S["CPL"]
                g2 = rt * 16 + S["RPC"] * i + lane // S["LPR"]
                if g2 >= rows:
                    g2 = rt * 16
                q2 = kv * repeat + g2 % repeat
                mrow = q2 * mhs + (g2 // repeat) * stride
                w = 16 if S["WIDE"] else 4
                c.append(("mask", (mrow + cell) * S["CB"],
                          2 * S["KT"] + 4 * S["SBB"] + S["MSTEP"] * i + w * lane, w))
            copies.append(c)
    return copies


def stage_reads(S, t, L, rt, rows, repeat, kv, mhs, stride, stream, cap):
    """(lds byte, width, buffer, expected src byte) for every byte range the
    arithmetic of tile t reads that must hold a real key's data."""
    key0 = t * BN
    WPK, NG, ESZ = S["WPK"], S["NG"], S["ESZ"]
    row = 4 * WPK
    base = stream * cap * row
    sbase = stream * cap * NG * ESZ
    out = []
    for key in range(BN):
        if key0 + key >= L:
            continue
        # K and V words of the key (every word of the row is read by some lane)
        for wd in range(WPK):
            out.append((key * row + 4 * wd, 4, "kp", base + (key0 + key) * row + 4 * wd))
            out.append((S["KT"] + key * row + 4 * wd, 4, "vp",
                        base + (key0 + key) * row + 4 * wd))
        for a, arr in enumerate(("ks", "kb", "vs", "vb")):
            for g in range(NG):
                e = key * NG + g
                out.append((2 * S["KT"] + a * S["SBB"] + e * ESZ, ESZ, arr,
                            sbase + ((key0 + key) * NG + g) * ESZ))
        if S["DMA"]:
            for r in range(16):
                g2 = rt * 16 + r
                if g2 >= rows:
                    continue
                q2 = kv * repeat + g2 % repeat
                mrow = q2 * mhs + (g2 // repeat) * stride
                out.append((2 * S["KT"] + 4 * S["SBB"] + (r * BN + key) * S["CB"], S["CB"],
                            "mask", (mrow + key0 + key) * S["CB"]))
    return out


def check(dim, bits, G, et, mask_kind, B, nQ, nKV, L, q_l, nwg, window=0, cap=None,
          wait_slack=0):
    cap = cap or L
    if ((dim // G) * (4 if et == F32 else 2)) % 4 and cap % 2:
        cap += 1          # the capacity the library requires there (even)
    repeat = nQ // nKV
    rows = q_l * repeat
    stride = L
    mhs = q_l * stride
    mm = mask_mode(et, mask_kind, mhs, stride, L)
    S = shape(dim, bits, G, et, mm)
    ESZ, NG = S["ESZ"], S["NG"]
    sizes = {"kp": B * nKV * cap * 4 * S["WPK"], "vp": B * nKV * cap * 4 * S["WPK"],
             "ks": B * nKV * cap * NG * ESZ, "kb": B * nKV * cap * NG * ESZ,
             "vs": B * nKV * cap * NG * ESZ, "vb": B * nKV * cap * NG * ESZ,
             "mask": (B * nQ * mhs) * S["CB"]}
    n_tiles = math.ceil(L / BN)
    klo = max(0, L - window) if window and window < L else 0
    tile_lo = klo // BN
    row_tiles = math.ceil(rows / 16)
    for stream, rt in itertools.product(range(B * nKV), range(row_tiles)):
        kv = stream
        for split in range(nwg):
            t0 = (n_tiles - tile_lo) * split // nwg + tile_lo
            t1 = (n_tiles - tile_lo) * (split + 1) // nwg + tile_lo
            issued = []       # tile of each copy, in issue order
            NS = S["NS"]

            def issue(t):
                cps = tile_copies(S, t, L, cap, stream, rt, rows, repeat, kv, mhs, stride)
                assert len(cps) == S["PER_TILE"], (len(cps), S["PER_TILE"])
                lds = {}
                for c in cps:
                    assert c, "a copy with no active lane"
                    for buf, src, dst, w in c:
                        assert 0 <= src and src + w <= sizes[buf], (buf, src, w, sizes[buf])
                        assert 0 <= dst and dst + w <= S["BYTES"], (dst, w)
                        for b in range(w):
                            lds[dst + b] = (buf, src + b)
                    issued.append(t)
                return lds

            content = {}
            for i in range(NS):
                if t0 + i < t1:
                    content[(t0 + i) % NS] = (t0 + i, issue(t0 + i))
            for t in range(t0, t1):
                after = min(t1 - 1 - t, NS - 1)
                n_ok = 2 * S["PER_TILE"] if (NS >= 3 and after >= 2) else (
                    S["PER_TILE"] if after >= 1 else 0)
                n_ok += wait_slack
                assert n_ok <= 63
                last = max(i for i, tt in enumerate(issued) if tt == t)
                assert last < len(issued) - n_ok, "tile %d read while its copies may fly" % t
                tt, lds = content[t % NS]
                assert tt == t
                for dst, w, buf, src in stage_reads(S, t, L, rt, rows, repeat, kv, mhs,
                                                    stride, stream, cap):
                    for b in range(w):
                        got = lds.get(dst + b)
                        assert got == (buf, src + b), (t, dst + b, got, buf, src + b)
                if t + NS < t1:
                    content[(t + NS) % NS] = (t + NS, issue(t + NS))


# (dim, bits, G, elem, mask, B, nQ, nKV, L, q_l, nwg, window)
CASES = [
    # the reverted variant's failing geometry
    (512, 8, 32, F16, "bool", 1, 2, 1, 97, 1, 2, 0),
    (512, 8, 32, F16, "bool", 1, 2, 1, 97, 1, 1, 0),
    (512, 4, 32, F16, None, 1, 2, 1, 97, 1, 2, 0),
    # quantized GPU test shapes
    (128, 4, 64, F16, None, 1, 4, 1, 100, 1, 1, 0),
    (128, 4, 64, F16, "alibi", 2, 8, 2, 333, 1, 3, 0),
    (64, 8, 32, F16, None, 1, 4, 4, 257, 1, 2, 0),
    (256, 4, 128, F16, "alibi", 2, 6, 2, 190, 1, 4, 0),
    (512, 4, 32, F16, None, 1, 2, 1, 97, 1, 2, 0),
    (512, 8, 128, F16, "alibi", 1, 2, 2, 65, 1, 1, 0),
    (64, 4, 64, F16, None, 1, 4, 2, 1000, 3, 5, 0),
    (128, 4, 32, F16, "alibi", 3, 4, 1, 77, 5, 2, 0),
    (96, 4, 32, F16, "alibi", 1, 4, 1, 333, 1, 3, 0),
    (96, 8, 32, F16, None, 2, 4, 2, 190, 2, 2, 0),
    (128, 4, 64, F16, "bool", 2, 8, 2, 333, 1, 3, 0),
    (128, 8, 64, F16, "bool", 1, 4, 1, 500, 1, 3, 33),
    (64, 4, 32, F16, "alibi", 2, 4, 2, 1000, 1, 4, 320),
    (256, 4, 64, F16, "bool", 1, 2, 1, 333, 3, 2, 100),
    (512, 4, 128, F16, None, 1, 2, 1, 161, 2, 3, 70),
    (96, 4, 32, F16, "bool", 1, 4, 2, 300, 1, 2, 0),
    (128, 4, 64, BF16, "alibi", 2, 8, 2, 333, 1, 3, 0),
    (64, 8, 32, BF16, "bool", 1, 4, 4, 257, 2, 2, 0),
    (512, 8, 32, BF16, None, 1, 2, 1, 97, 1, 2, 0),
    (128, 4, 64, F32, "alibi", 2, 8, 2, 333, 1, 3, 0),
    (256, 4, 32, F32, "alibi", 2, 6, 2, 190, 1, 4, 0),
    (512, 8, 32, F32, "alibi", 1, 2, 1, 97, 1, 2, 0),
    (96, 4, 32, F32, None, 1, 4, 2, 300, 3, 3, 77),
    (64, 4, 64, F32, "alibi", 1, 2, 1, 101, 1, 2, 0),
    # odd mask alignments: 4-byte copies and per-lane loads
    (128, 4, 64, F16, "alibi", 1, 4, 1, 203, 1, 2, 0),
    (128, 4, 64, F16, "alibi", 1, 4, 1, 204, 1, 2, 0),
    (128, 4, 64, F16, "bool", 1, 4, 1, 203, 1, 2, 0),
]


@pytest.mark.parametrize("dim,bits,G,et,mask,B,nQ,nKV,L,q_l,nwg,window", CASES)
def test_copy_geometry_and_waits(dim, bits, G, et, mask, B, nQ, nKV, L, q_l, nwg, window):
    check(dim, bits, G, et, mask, B, nQ, nKV, L, q_l, nwg, window)


def test_workload_geometry_first_streams():
    # the 4-bit workload's shape (16384 tokens, 64 splits) on its first two
    # kv streams: full tiles only, and a capacity equal to the length
    check(128, 4, 64, F16, "alibi", 1, 8, 2, 16384, 1, 64)


def test_model_catches_a_miscounted_wait():
    # the model is not vacuous: a wait that lets one more copy fly leaves a
    # tile's last copy possibly unfinished when the tile is read
    with pytest.raises(AssertionError, match="copies may fly"):
        check(128, 4, 64, F16, "alibi", 1, 4, 1, 333, 1, 2, wait_slack=1)


def test_model_catches_a_wrong_source_row():
    # and a copy that takes a neighbouring token's row is caught too
    orig = tile_copies

    def shifted(S, t, *a):
        cps = orig(S, t, *a)
        return [[(b, src + (4 * S["WPK"] if b == "kp" and src >= 4 * S["WPK"] else 0), d, w)
                 for (b, src, d, w) in c] for c in cps]
    globals()["tile_copies"] = shifted
    try:
        with pytest.raises(AssertionError):
            check(128, 4, 64, F16, None, 1, 4, 1, 100, 1, 1)
    finally:
        globals()["tile_copies"] = orig
