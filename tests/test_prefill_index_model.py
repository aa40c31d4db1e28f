"""CPU model of the index math of the grouped MFMA kernels (csrc/k_prefill.h,
16x16x32 form; csrc/k_prefill32.h, 32x32x32 form): the direct-to-LDS staging
of a stage (weight rows, activation rows, block scales, each 16-byte piece at
a per-row XOR-swizzled position) and the operand reads of the K loop.

For every wave, lane, stage and block of ragged shapes (row tiles shorter
than the tile, items shorter than the item size, rows whose block count is
no multiple of the stage) the model checks that
  - every staged byte lands inside its region of the slot and no two lanes
    write the same LDS bytes (a stage is a bijection);
  - global reads stay inside their row (the last stage's pieces are clamped);
  - the bytes each lane reads for its A operand are the weights of the row,
    block and k range the MFMA layout gives that lane, its B operand the same
    k range of the token's activation block, its scale the token's scale of
    that block; blocks past the row's end read the zero scale, so the clamped
    pieces add nothing;
  - the 16 (32) lanes reading one operand hit 16 (32) distinct 16-byte piece
    positions within each 256-byte span (the purpose of the swizzle).
The formulas are those of the kernels' Plan/Plan32 init and issue and the
lane bases of mm_loop/mm_loop32, transcribed; the GPU parity tests check the
kernels' results end to end.

It also models work_of, the XCD-aware order of the gate/up workgroups: over
the items the bucketing makes (each expert's tokens cut into chunks of the
item size, experts in ascending order) every (item, row tile) is taken by
exactly one block of the launch grid, whatever upper bound on the items the
grid was sized for, and each XCD's run holds an expert's items side by side
per row tile; and k_bucket_fill, whose per-expert sums give the slot
offsets, items and slot maps of an exclusive scan with a binary-search owner
per slot.
"""
import itertools

import pytest


def wkey(r, ks, npc):
    return (r // ks) % npc


# ---------------------------------------------------------------------------
# geometry
# ---------------------------------------------------------------------------

def geo16(bits, kt):
    CH = 4
    WB = 4 * bits
    RB = CH * WB
    g = dict(CH=CH, WB=WB, RB=RB, NPC=RB // 16, KS=1 if RB >= 256 else 256 // RB,
             RPI=1024 // RB, WBYTES=32 * RB, ARB=CH * 32, TILE=16, ROWS_PER_WAVE=32)
    g["WINSTR"] = g["WBYTES"] // 1024
    g["ANPC"] = g["ARB"] // 16
    g["AKS"] = 1 if g["ARB"] >= 256 else 256 // g["ARB"]
    g["ARPI"] = 1024 // g["ARB"]
    g["A_OFF"] = 4 * g["WBYTES"]
    g["D_OFF"] = g["A_OFF"] + kt * g["ARB"]
    g["SLOT"] = (g["D_OFF"] + kt * CH * 4 + 255) & ~255
    return g


def geo32(bits, kt):
    CH = 16 // bits
    g = dict(CH=CH, WB=4 * bits, RB=64, NPC=4, KS=4, RPI=16, WBYTES=64 * 64, ARB=CH * 32,
             TILE=32, ROWS_PER_WAVE=64)
    g["WINSTR"] = g["WBYTES"] // 1024
    g["ANPC"] = g["ARB"] // 16
    g["AKS"] = 1 if g["ARB"] >= 256 else 256 // g["ARB"]
    g["ARPI"] = 1024 // g["ARB"]
    g["AINSTR"] = kt * g["ARB"] // 1024
    g["AIW"] = (g["AINSTR"] + 3) // 4
    g["TPI"] = 64 // CH
    g["SINSTR"] = kt // g["TPI"]
    g["SIW"] = (g["SINSTR"] + 3) // 4
    g["A_OFF"] = 4 * g["WBYTES"]
    g["D_OFF"] = g["A_OFF"] + kt * g["ARB"]
    g["SLOT"] = (g["D_OFF"] + kt * CH * 4 + 255) & ~255
    return g


# ---------------------------------------------------------------------------
# staging: LDS byte -> ("w"|"a"|"s", global tag, byte) for one stage
# ---------------------------------------------------------------------------

ZERO = ("zero",)


def stage_map(form, bits, kt, ng, c, nrow, n, NB, rowb, arowb):
    """Writes of stage c by the 4 waves: dict LDS offset -> source, where the
    source of a weight byte is ("w", wave, tile, row, global byte in row), of
    an activation byte ("a", token row, byte in row), of a scale byte
    ("s", token row, block) or ZERO."""
    g = geo16(bits, kt) if form == 16 else geo32(bits, kt)
    lds = {}
    rows_of = list(range(n))  # the item's token rows (slot order)

    def put(off, src):
        assert off not in lds, ("two writes to one LDS byte", off, src, lds[off])
        lds[off] = src

    for wave, lane in itertools.product(range(4), range(64)):
        # weights
        for i in range(g["WINSTR"]):
            r = i * g["RPI"] + lane // g["NPC"]
            t = r // g["TILE"]
            rr = min(r % g["TILE"], nrow[t] - 1)
            piece = (lane % g["NPC"]) ^ wkey(r, g["KS"], g["NPC"])
            gofs = min(c * g["RB"] + piece * 16, rowb - 16)
            assert 0 <= gofs and gofs + 16 <= rowb
            base = wave * g["WBYTES"] + i * 1024 + 16 * lane
            for k in range(16):
                put(base + k, ("w", wave, t, rr, gofs + k))
        # activations
        if form == 16:
            aiw = (ng * g["ARB"] + 255) // 256
            act = True
        else:
            aiw = g["AIW"]
            act = wave * aiw < g["AINSTR"]
        if act:
            for i in range(aiw):
                j = (wave * aiw + i) * g["ARPI"] + lane // g["ANPC"]
                piece = (lane % g["ANPC"]) ^ wkey(j, g["AKS"], g["ANPC"])
                gofs = min(c * g["ARB"] + piece * 16, arowb - 16)
                assert 0 <= gofs and gofs + 16 <= arowb
                base = g["A_OFF"] + (wave * aiw + i) * 1024 + 16 * lane
                for k in range(16):
                    put(base + k, ("a", rows_of[min(j, n - 1)], gofs + k))
        # block scales
        if form == 16 and NB % g["CH"] == 0:
            # one 16-byte load per token by wave 0 (lane j: token j's CH
            # scales of the stage), lanes past the item size idle
            if wave == 0 and lane < kt:
                tok = rows_of[min(lane, n - 1)]
                for bk in range(g["CH"]):
                    for k in range(4):
                        put(g["D_OFF"] + 16 * lane + 4 * bk + k, ("s", tok, c * g["CH"] + bk, k))
        elif form == 16:
            TPI = 64 // g["CH"]
            if wave * TPI < kt:
                js = min(wave * TPI, kt - TPI) + lane // g["CH"]
                sbk = lane % g["CH"]  # skey is 0 for 4-block stages
                b = c * g["CH"] + sbk
                src = ("s", rows_of[min(js, n - 1)], b) if b < NB else ZERO
                for k in range(4):
                    put(g["D_OFF"] + wave * TPI * g["CH"] * 4 + 4 * lane + k, src + (k,))
        elif g["CH"] == 4 and NB % 4 == 0:
            # 32x32 form, int4: one 16-byte load per token by wave 0
            if wave == 0 and lane < kt:
                tok = rows_of[min(lane, n - 1)]
                for bk in range(4):
                    for k in range(4):
                        put(g["D_OFF"] + 16 * lane + 4 * bk + k, ("s", tok, c * 4 + bk, k))
        else:
            if wave * g["SIW"] < g["SINSTR"]:
                for i in range(g["SIW"]):
                    js = min((wave * g["SIW"] + i) * g["TPI"], kt - g["TPI"]) + lane // g["CH"]
                    b = c * g["CH"] + lane % g["CH"]
                    src = ("s", rows_of[min(js, n - 1)], b) if b < NB else ZERO
                    for k in range(4):
                        put(g["D_OFF"] + (wave * g["SIW"] + i) * 256 + 4 * lane + k, src + (k,))
    assert all(0 <= off < g["SLOT"] for off in lds)
    return g, lds


# ---------------------------------------------------------------------------
# operand reads of the K loop
# ---------------------------------------------------------------------------

def reads16(g, bits, wave, lane, bi, grp):
    """(A tile-0 bytes, A tile-1 bytes, B bytes, scale bytes) LDS offsets of
    one lane for block bi and 16-token group grp (mm_loop)."""
    lr, q = lane & 15, lane >> 4
    if bits == 4:
        wq, wbx, na = 0, 4 * q, 4
    elif bits == 8:
        wq, wbx, na = q >> 1, 8 * (q & 1), 8
    else:
        wq, wbx, na = 0, 4 * (q >> 1), 4
    r0k = wkey(lr, g["KS"], g["NPC"])
    a0k = wkey(lr, g["AKS"], g["ANPC"])
    wbase = wave * g["WBYTES"] + lr * g["RB"] + ((wq ^ r0k) << 4) + wbx
    abase = g["A_OFF"] + lr * g["ARB"] + (((q >> 1) ^ a0k) << 4) + 8 * (q & 1)
    dbase = g["D_OFF"] + lr * g["CH"] * 4
    pb = bi if bits == 4 else 2 * bi if bits == 8 else bi >> 1
    ib = 8 * (bi & 1) if bits == 2 else 0
    wo = (wbase ^ (pb << 4)) + ib
    ao = abase ^ (bi << 5)
    do = dbase ^ (bi << 2)
    a0 = [wo + k for k in range(na)]
    a1 = [wo + 16 * g["RB"] + k for k in range(na)]
    b = [ao + grp * 16 * g["ARB"] + k for k in range(8)]
    s = [do + grp * 16 * g["CH"] * 4 + k for k in range(4)]
    return a0, a1, b, s


def reads32(g, bits, wave, lane, bi, grp):
    """The same for mm_loop32 (32-token groups)."""
    lr, q = lane & 31, lane >> 5
    if bits == 4:
        piece, byte, na = bi, 8 * q, 8
    elif bits == 8:
        piece, byte, na = 2 * bi + q, 0, 16
    else:
        piece, byte, na = bi >> 1, 8 * (bi & 1) + 4 * q, 4
    r0k = wkey(lr, g["KS"], g["NPC"])
    a0k = wkey(lr, g["AKS"], g["ANPC"])
    wo = wave * g["WBYTES"] + lr * g["RB"] + ((piece ^ r0k) << 4) + byte
    ao = g["A_OFF"] + lr * g["ARB"] + (((2 * bi + q) ^ a0k) << 4)
    do = g["D_OFF"] + lr * g["CH"] * 4 + 4 * bi
    a0 = [wo + k for k in range(na)]
    a1 = [wo + 32 * g["RB"] + k for k in range(na)]
    b = [ao + grp * 32 * g["ARB"] + k for k in range(16)]
    s = [do + grp * 32 * g["CH"] * 4 + k for k in range(4)]
    return a0, a1, b, s


def expected(form, bits, g, wave, lane, c, bi, grp, nrow, n, NB):
    """What the MFMA layout needs in each read: (weight row of tile 0 and 1,
    the byte range of the block's k range in the packed row), the token and
    activation byte range, the token and block of the scale."""
    tile = g["TILE"]
    lr, q = (lane & 15, lane >> 4) if form == 16 else (lane & 31, lane >> 5)
    kspan = 8 if form == 16 else 16           # k values per lane
    blk = c * g["CH"] + bi
    k0 = q * kspan                            # first k (in storage order) of the lane
    wbytes = [blk * g["WB"] + (k0 * bits) // 8 + k for k in range(kspan * bits // 8)]
    rows = [min(lr, nrow[t] - 1) for t in range(2)]
    tok = min(grp * tile + lr, n - 1)
    abytes = [blk * 32 + k0 + k for k in range(kspan)]
    return rows, wbytes, tok, abytes, blk


CASES16 = [(bits, kt, ng) for bits in (4, 8, 2) for kt, ng in ((32, 1), (32, 2), (64, 4), (64, 2))]
CASES32 = [(bits, kt) for bits in (4, 8, 2) for kt in (32, 64)]
# (blocks per row, rows of tile 0 / tile 1, tokens of the item)
SHAPES = [(192, (16, 16), 32), (6, (16, 5), 7), (2, (3, 1), 1), (64, (16, 16), 17), (10, (9, 16), 64)]


def _check(form, bits, kt, ng, NB, nrow, n):
    g = geo16(bits, kt) if form == 16 else geo32(bits, kt)
    tile = g["TILE"]
    nrow = tuple(min(v, tile) for v in nrow) if form == 16 else tuple(
        min(2 * v, tile) for v in nrow)
    n = min(n, kt)
    rowb = NB * g["WB"]
    arowb = NB * 32
    nst = (NB + g["CH"] - 1) // g["CH"]
    n_groups = ng if form == 16 else (1 if n <= 32 else 2)
    for c in range(nst):
        _, lds = stage_map(form, bits, kt, ng, c, nrow, n, NB, rowb, arowb)
        for wave, lane, bi, grp in itertools.product(range(4), range(64), range(g["CH"]),
                                                     range(n_groups)):
            a0, a1, b, s = (reads16 if form == 16 else reads32)(g, bits, wave, lane, bi, grp)
            rows, wbytes, tok, abytes, blk = expected(form, bits, g, wave, lane, c, bi, grp,
                                                       nrow, n, NB)
            scale_src = [lds[o] for o in s]
            if blk >= NB:
                # past the row's end: the scale is the zero in global memory
                assert all(v[:1] == ("zero",) for v in scale_src), (c, bi, scale_src)
                continue
            assert all(v[:3] == ("s", tok, blk) for v in scale_src), (wave, lane, c, bi, scale_src)
            for t, rd in ((0, a0), (1, a1)):
                got = [lds[o] for o in rd]
                want = [("w", wave, t, rows[t], x) for x in wbytes]
                if bits == 2:
                    # int2: the lane reads the dword of 16 codes holding its k range
                    half = (lane >> (4 if form == 16 else 5))
                    d0 = blk * 8 + 4 * (half >> 1 if form == 16 else half)
                    want = [("w", wave, t, rows[t], d0 + k) for k in range(4)]
                assert got == want, (form, bits, wave, lane, c, bi, t, got[:2], want[:2])
            got = [lds[o] for o in b]
            assert got == [("a", tok, x) for x in abytes], (wave, lane, c, bi, got[:2])


@pytest.mark.parametrize("bits,kt,ng", CASES16)
@pytest.mark.parametrize("shape", SHAPES)
def test_16x16_staging_and_operand_reads(bits, kt, ng, shape):
    NB, nrow, n = shape
    _check(16, bits, kt, ng, NB, nrow, n)


@pytest.mark.parametrize("bits,kt", CASES32)
@pytest.mark.parametrize("shape", SHAPES)
def test_32x32_staging_and_operand_reads(bits, kt, shape):
    NB, nrow, n = shape
    _check(32, bits, kt, kt // 32, NB, nrow, n)


@pytest.mark.parametrize("form", [16, 32])
@pytest.mark.parametrize("bits", [4, 8, 2])
def test_operand_reads_spread_over_piece_positions(form, bits):
    # the lanes reading one operand (16 rows / tokens, or 32) touch distinct
    # 16-byte piece positions of every 256-byte span: the swizzle's purpose
    g = geo16(bits, 64) if form == 16 else geo32(bits, 64)
    tile = g["TILE"]
    for bi in range(g["CH"]):
        for half in range(64 // tile):
            lanes = [half * tile + lr for lr in range(tile)]
            for which in (0, 2):  # A tile 0, B
                offs = [(reads16 if form == 16 else reads32)(g, bits, 0, l, bi, 0)[which][0]
                        for l in lanes]
                spans = {}
                for o in offs:
                    spans.setdefault(o // 256, []).append((o % 256) // 16)
                for pos in spans.values():
                    assert len(pos) == len(set(pos)), (form, bits, bi, which, pos)


def test_integer_block_scales_are_exact():
    # k_scale_int: d_b = M_b 2^e_b (M the 24-bit significand) -> m_b = M_b <<
    # (e_b - e0) with e0 the least exponent of the row's nonzero scales; rows
    # whose exponents span more than 7 (or hold a non-finite value) are
    # marked wide. Then sum_b d_b I_b = 2^e0 sum_b m_b I_b exactly.
    import random
    import struct
    from fractions import Fraction

    def parts(d):
        u = struct.unpack("<I", struct.pack("<f", d))[0]
        E = u >> 23
        if u & 0x7FFFFFFF == 0:
            return None
        M = (u & 0x7FFFFF) if E == 0 else (u & 0x7FFFFF) | 0x800000
        return M, (-149 if E == 0 else E - 150)

    rng = random.Random(5)
    for trial in range(300):
        nb = rng.choice([2, 6, 64, 192])
        base = rng.choice([1e-3, 2.0, 1e-39, 3e38 / 127])
        spread = rng.choice([0, 3, 7, 8, 12])
        ds = []
        for _ in range(nb):
            v = base * 2.0 ** rng.uniform(0, spread) * rng.uniform(1, 2)
            v = struct.unpack("<f", struct.pack("<f", min(v, 3.4e38)))[0]
            ds.append(0.0 if rng.random() < 0.05 else v)
        ps = [parts(d) for d in ds]
        es = [p[1] for p in ps if p]
        if not es:
            continue
        e0, wide = min(es), max(es) - min(es) > 7
        if wide:
            continue
        ms = [0 if p is None else p[0] << (p[1] - e0) for p in ps]
        assert all(0 <= m < 2 ** 31 for m in ms)
        dots = [rng.randint(-28448 * 16, 28448 * 16) for _ in range(nb)]
        exact = sum(Fraction(d) * I for d, I in zip(ds, dots))
        assert Fraction(sum(m * I for m, I in zip(ms, dots))) * Fraction(2) ** e0 == exact
        assert abs(sum(m * I for m, I in zip(ms, dots))) < 2 ** 63


def bucket_items(counts, ch):
    """The items of k_bucket_fill, (expert, first slot, n) in expert order, and
    the slot offsets (expert e owns slots offs[e] .. offs[e + 1] - 1)."""
    offs, items, o = [], [], 0
    for e, c in enumerate(counts):
        offs.append(o)
        for j in range((c + ch - 1) // ch):
            items.append((e, o + j * ch, min(ch, c - j * ch)))
        o += c
    offs.append(o)
    return items, offs


def work_of(b, n_items, nrt, items, offs, kt):
    N = n_items * nrt
    L = (N + 7) >> 3
    l = b >> 3
    p = (b & 7) * L + l
    if l >= L or p >= N:
        return None
    i0 = p // nrt
    e = items[i0][0]
    io = i0 - (items[i0][1] - offs[e]) // kt
    m = (offs[e + 1] - offs[e] + kt - 1) // kt
    q = p - nrt * io
    rt = q // m
    return io + (q - rt * m), rt


WORK_CASES = [
    # (tokens per expert, routed then shared; item size; row tiles per item)
    ([3, 0, 40, 1, 64, 65, 0, 7], 32, 32),
    ([0] * 255 + [1, 512], 32, 32),
    ([128] * 16 + [4096], 64, 16),
    ([33] * 5 + [0, 2], 32, 3),
    ([1], 32, 1),
    ([0, 0, 5], 64, 7),
]


@pytest.mark.parametrize("case", range(len(WORK_CASES)))
def test_xcd_work_order_covers_every_item_and_tile_once(case):
    counts, kt, nrt = WORK_CASES[case]
    items, offs = bucket_items(counts, kt)
    n = len(items)
    for n_max in (n, n + 5):  # the host sizes the grid for an upper bound
        grid = (nrt * n_max + 7) // 8 * 8
        seen = {}
        for b in range(grid):
            w = work_of(b, n, nrt, items, offs, kt)
            if w is None:
                continue
            it, rt = w
            assert 0 <= it < n and 0 <= rt < nrt
            assert w not in seen, (w, b, seen.get(w))
            seen[w] = b
        assert len(seen) == n * nrt
        # per XCD in dispatch order: experts ascending; within an expert row
        # tiles ascending, and its items side by side at each row tile
        for x in range(8):
            run = [work_of(b, n, nrt, items, offs, kt) for b in range(x, grid, 8)]
            run = [w for w in run if w is not None]
            for (i1, r1), (i2, r2) in zip(run, run[1:]):
                e1, e2 = items[i1][0], items[i2][0]
                assert e1 <= e2
                if e1 == e2:
                    assert (r1, i1) < (r2, i2)


def bucket_fill(counts, lists, T, KS, ch):
    """k_bucket_fill, transcribed: workgroup e sums the counts and item counts
    of the experts before it, then writes its items and slot maps."""
    NE = len(counts)
    offs = [0] * (NE + 1)
    items, slot_of, slot_tok = {}, {}, {}
    n_items = 0
    for e in range(NE):
        so = sum(counts[:e])
        io = sum((c + ch - 1) // ch for c in counts[:e])
        c = counts[e]
        ni = (c + ch - 1) // ch
        offs[e] = so
        if e == NE - 1:
            offs[NE] = so + c
            n_items = io + ni
        for j in range(ni):
            items[io + j] = (e, so + j * ch, min(ch, c - j * ch))
        for p in range(c):
            entry = lists[e][p]
            slot_of[entry] = so + p
            slot_tok[so + p] = entry // KS
    return offs, [items[i] for i in range(n_items)], slot_of, slot_tok


@pytest.mark.parametrize("seed", range(6))
def test_bucket_fill_matches_the_scan_definition(seed):
    import random
    rng = random.Random(seed)
    E, S = rng.choice([(16, 1), (256, 1), (5, 0), (64, 2)])
    K = rng.randint(1, min(E, 8))
    T = rng.choice([1, 3, 17, 300])
    KS = K + S
    ch = rng.choice([4, 32, 64])
    # routing: K distinct experts per token; shared experts take every token
    lists = [[] for _ in range(E + S)]
    for t in range(T):
        for k, e in enumerate(rng.sample(range(E), K)):
            lists[e].append(t * KS + k)
        for s in range(S):
            lists[E + s].append(t * KS + K + s)
    counts = [len(l) for l in lists]
    offs, items, slot_of, slot_tok = bucket_fill(counts, lists, T, KS, ch)
    # definition: exclusive scan of the counts; each slot's owner is the last
    # expert whose offset is at or below it
    scan = [0]
    for c in counts:
        scan.append(scan[-1] + c)
    assert offs == scan
    want_items = [(e, scan[e] + j * ch, min(ch, c - j * ch))
                  for e, c in enumerate(counts) for j in range((c + ch - 1) // ch)]
    assert items == want_items
    for g in range(scan[-1]):
        e = max(i for i in range(E + S) if scan[i] <= g and counts[i] > 0)
        entry = lists[e][g - scan[e]]
        assert slot_of[entry] == g and slot_tok[g] == entry // KS
    assert sorted(slot_of) == sorted(x for l in lists for x in l)
