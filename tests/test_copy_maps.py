"""CPU models of the bf16 GEMM kernel's index maps (csrc/gemm_bf16_dma.h,
csrc/gemm_bf16_impl.h), checked before any GPU run.

The kernel moves operand tiles into LDS with 1 KiB global->LDS copies (lane t's
16 bytes land at base + 16 t, so the LDS layout is fixed by which global 16
bytes each lane fetches) and reads MFMA fragments back with ds_read_b128 or
ds_read_b64_tr_b16.  These tests restate the kernel's per-lane formulas in
Python and check, over all waves, lanes and k-tiles:

  * the tile orders are bijections onto the tile grid;
  * every copy source lies inside its operand, ragged shapes included;
  * every fragment read returns exactly the (row, k) elements the MFMA
    operand layout asks for (v_mfma_f32_32x32x16: lane l, row row0 + l % 32,
    k 16 s + 8 (l / 32) .. +7; v_mfma_f32_16x16x32, the kernels' MF16 mode:
    lane l, row row0 + l % 16, k 8 (l / 16) .. +7), and the lanes one read
    cycle serves hit distinct banks;
  * MF16: the MFMA result (lane l holds rows 4 (l / 16) .. +3 of column
    l % 16 of operand 0 x operand 1, the weight fragment first) lands where
    the epilogues and the fp32 LDS restaging expect it;
  * the paired stages' issue schedule never overwrites a stage that is
    still to be read, and the constant vmcnt waits cover every published
    k-tile under in-order completion.

The transposing read follows its measured behaviour: within each 16-lane
group, lane 4r + c supplies the address of 4 consecutive bf16 of row r of a
4 x 16 block (columns 4c .. 4c+3), and lane i receives column i.
"""
import itertools
import random

import pytest

KBK = 32        # k per k-tile
XCDS = 8


# ---- tile orders (tile_coords / tile_coords_rounds) ---------------------------

def tile_coords(bid, nblk, tiles_m, tiles_n, group_m=8):
    pid = bid
    if nblk % XCDS == 0:
        pid = (bid % XCDS) * (nblk // XCDS) + bid // XCDS
    width = group_m * tiles_n
    group = pid // width
    first_m = group * group_m
    gsize = min(tiles_m - first_m, group_m)
    in_group = pid - group * width
    return first_m + in_group % gsize, in_group // gsize


def tile_coords_rounds(bid, nblk, tiles_m, tiles_n):
    if tiles_n not in (8, 16, 32):
        return None
    rows = 256 // tiles_n
    if nblk != tiles_m * tiles_n or tiles_m % rows:
        return None
    xcd, k = bid % XCDS, bid // XCDS
    rnd, s = k // 32, k % 32
    xr = rows // 4
    return rnd * rows + (xcd % xr) * 4 + s % 4, (xcd // xr) * 8 + s // 4


@pytest.mark.parametrize("tiles_m,tiles_n", [(64, 16), (64, 32), (16, 16), (32, 8), (63, 9), (17, 3), (1, 1)])
def test_tile_orders_are_bijections(tiles_m, tiles_n):
    n = tiles_m * tiles_n
    got = {tile_coords(b, n, tiles_m, tiles_n) for b in range(n)}
    assert len(got) == n and all(0 <= a < tiles_m and 0 <= c < tiles_n for a, c in got)
    if tile_coords_rounds(0, n, tiles_m, tiles_n) is not None:
        got = {tile_coords_rounds(b, n, tiles_m, tiles_n) for b in range(n)}
        assert len(got) == n and all(0 <= a < tiles_m and 0 <= c < tiles_n for a, c in got)


# ---- single k-tile stages (OperandTile) ----------------------------------------

def kswz(krow, mf16=False):
    """Chunk swizzle of a k-major tile (OperandTile::kswz)."""
    return ((krow & 3) << 2) ^ ((((krow >> 3) & 1) << 1) if mf16 else 0)


def single_copies(R, NW, kmajor, r0, rows, K, kc, mf16=False):
    """{LDS 16-byte chunk index: (row or k-row, first k or first column)} of
    k-tile kc's copies.  K not a multiple of 32 (KTAIL): the last k-tile is
    the window of the last 32 k, starting at kbase = max(K - 32, 0) (the
    uniform min(32 kc, kbase)), and each lane's k is clamped to the last
    valid one (a no-op unless K < 32)."""
    ktail = K % KBK != 0
    kstart = min(kc * KBK, max(K - KBK, 0)) if ktail else kc * KBK
    Q = R * KBK * 2 // 1024 // NW
    cb = R // 8
    lds = {}
    for wave, i, lane in itertools.product(range(NW), range(Q), range(64)):
        slot = (wave * Q + i) * 64 + lane
        if not kmajor:
            row = slot >> 2
            kin = 8 * ((slot & 3) ^ ((row >> 2) & 3))
            lds[slot] = (min(r0 + row, rows - 1), kstart + (min(kin, K - 8) if ktail else kin))
        else:
            krow = slot // cb
            c = (slot % cb) ^ kswz(krow, mf16)
            lds[slot] = (kstart + (min(krow, K - 1) if ktail else krow), min(r0 + 8 * c, rows - 8))
    assert len(lds) == R * KBK * 2 // 16
    return lds


def tail_mask(K, kc, place):
    """Whether the kernel keeps window place `place` (0 .. 31) of k-tile kc:
    for the last k-tile of a K with a tail, lo <= place < hi with
    lo = klast - kbase, hi = K - kbase; every place of the other k-tiles."""
    nk = -(-K // KBK)
    if K % KBK == 0 or kc != nk - 1:
        return True
    kbase, klast = max(K - KBK, 0), (nk - 1) * KBK
    return klast - kbase <= place < K - kbase


@pytest.mark.parametrize("R,NW,kmajor,rows,K", [
    (256, 8, False, 300, 200), (256, 8, False, 16, 8), (256, 8, True, 264, 300), (256, 8, True, 8, 1),
    (128, 4, False, 300, 136), (128, 4, True, 1000, 40), (256, 8, False, 257, 40), (384, 8, True, 3072, 8192),
    (64, 4, False, 100, 72), (64, 4, False, 2048, 4096),
])
def test_single_stage_sources_in_bounds(R, NW, kmajor, rows, K):
    nk = -(-K // KBK)
    for r0 in range(0, rows, R):
        for kc in sorted({0, nk - 1, nk // 2}):
            for a, b in single_copies(R, NW, kmajor, r0, rows, K, kc).values():
                if not kmajor:
                    assert 0 <= a < rows and 0 <= b and b + 8 <= K
                else:
                    assert 0 <= a < K and 0 <= b and b + 8 <= rows


@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("K", [8, 16, 24, 40, 56, 64, 72, 200, 1000, 1024, 16376])
def test_ktail_window_adds_every_k_once(kmajor, K):
    """Over all k-tiles of a row (k-contiguous) or column (k-major), the k
    that survive the last k-tile's mask are exactly 0 .. K-1, each once; the
    lane's data at window place p of k-tile kc is k = kstart + p (clamped
    copies only at masked places).  k-major operands also take K % 8 != 0."""
    Ks = [K] + ([K - 3, K + 5] if kmajor and K > 8 else [])
    for K in Ks:
        nk = -(-K // KBK)
        R, NW = 256, 8
        seen = []
        for kc in range(nk):
            lds = single_copies(R, NW, kmajor, 0, 10**6, K, kc)
            cb = R // 8
            for slot, (a, b) in lds.items():
                if not kmajor:
                    row = slot >> 2
                    logical = 8 * ((slot & 3) ^ ((row >> 2) & 3))
                    if row != 5:
                        continue
                    for e in range(8):
                        if tail_mask(K, kc, logical + e):
                            assert 0 <= b + e < K
                            seen.append(b + e)
                else:
                    krow = slot // cb
                    c = (slot % cb) ^ kswz(krow)
                    if c != 3:
                        continue
                    if tail_mask(K, kc, krow):
                        assert 0 <= a < K
                        seen.append(a)
        assert sorted(seen) == list(range(K))


def test_kcontig_fragments():
    R, NW = 256, 8
    lds = single_copies(R, NW, False, 0, 10**6, 1024, 3)
    for row0, s in itertools.product(range(0, R, 32), range(2)):
        banks = {}
        for lane in range(64):
            chunk = (2 * s + (lane >> 5)) ^ ((lane >> 2) & 3)
            off = (row0 + (lane & 31)) * 64 + chunk * 16
            assert lds[off // 16] == (row0 + (lane & 31), 3 * KBK + 16 * s + 8 * (lane >> 5))
            banks.setdefault(lane // 16, set()).add((off // 16) % 16)
        assert all(len(b) == 16 for b in banks.values())


def test_kmajor_fragments_through_the_transposing_read():
    R, NW = 256, 8
    cb = R // 8
    lds = single_copies(R, NW, True, 0, 10**6, 1024, 5)

    def element(krow, byte):               # (k, column) of the bf16 at byte `byte` of LDS k-row `krow`
        kr, col0 = lds[(krow * R * 2 + byte) // 16]
        return kr, col0 + (byte % 16) // 2

    for row0, s in itertools.product(range(0, R, 32), range(2)):
        for H in range(2):
            addr = {}
            for lane in range(64):
                gi = lane & 15
                row_lane = (lane >> 5) * 8 + (gi >> 2)
                chunk = ((row0 >> 3) + ((lane >> 4) & 1) * 2 + ((gi & 3) >> 1)) ^ ((gi >> 2) << 2)
                addr[lane] = (s * 16 + H * 4 + row_lane, chunk * 16 + (gi & 1) * 8)
            for lane in range(64):
                g0, gi = lane & ~15, lane & 15
                for r in range(4):             # lane gi receives column gi of the 4 x 16 block
                    src = g0 + 4 * r + (gi >> 2)
                    krow, byte = addr[src]
                    k, col = element(krow, byte + 2 * (gi & 3))
                    assert (k, col) == (5 * KBK + 16 * s + 8 * (lane >> 5) + 4 * H + r, row0 + (lane & 31))
            # the four k-rows of one read fall in four different 64-byte bank windows
            for g in range(4):
                wins = {((addr[g * 16 + 4 * r][0] * R * 2 + addr[g * 16 + 4 * r][1]) // 64) % 4 for r in range(4)}
                assert len(wins) == 4


# ---- LDS layout of the single-stage kernels (DmaLayout) --------------------------

@pytest.mark.parametrize("BM,BN,WGM,WGN", [(256, 256, 2, 4), (128, 128, 2, 2), (128, 384, 2, 4)])
def test_stage_windows_and_staging_slabs(BM, BN, WGM, WGN):
    """A's stages, then B's: on the 256 x 256 and 128 x 128 tiles each
    operand's four stages lie within 64 KiB of its first stage, so one
    register plus the LDS read's 16-bit immediate reaches every stage (the
    128 x 384 tile's B stages span 96 KiB; that kernel has registers to
    spare for a second base).  The fp32 staging slab of each wave lies in A's
    last stage, B's last stage or past the stages: never in a stage that the
    next tile's first STAGES-1 k-tiles fill during the epilogue, never in
    another wave's slab, and inside the 160 KiB of LDS."""
    S = 4
    a_bytes, b_bytes = BM * KBK * 2, BN * KBK * 2
    b_at = S * a_bytes
    stage_bytes = S * (a_bytes + b_bytes)
    if BN <= 256:
        assert S * a_bytes <= 65536 and S * b_bytes <= 65536
    waves = WGM * WGN
    tn = BN // WGN // 32
    staged = 64 % (BN // WGN // 4) == 0
    if not staged:
        assert stage_bytes <= 160 * 1024
        return
    slab = 32 * tn * 32 * 4
    in_a, in_b = a_bytes // slab, b_bytes // slab

    def slab_at(w):
        if w < in_a:
            return (S - 1) * a_bytes + w * slab
        if w < in_a + in_b:
            return b_at + (S - 1) * b_bytes + (w - in_a) * slab
        return stage_bytes + (w - in_a - in_b) * slab

    lds_bytes = max(stage_bytes, stage_bytes + max(0, waves - in_a - in_b) * slab)
    assert lds_bytes <= 160 * 1024
    busy = [(s * a_bytes, (s + 1) * a_bytes) for s in range(S - 1)]
    busy += [(b_at + s * b_bytes, b_at + (s + 1) * b_bytes) for s in range(S - 1)]
    spans = []
    for w in range(waves):
        lo = slab_at(w)
        hi = lo + slab
        assert 0 <= lo and hi <= lds_bytes
        assert all(hi <= b0 or lo >= b1 for b0, b1 in busy)
        assert all(hi <= s0 or lo >= s1 for s0, s1 in spans)
        spans.append((lo, hi))


# ---- paired stages (OperandPairTile) --------------------------------------------

def pair_copies(R, NW, r0, rows, K, j):
    Q = R * 2 * KBK * 2 // 1024 // NW
    lds = {}
    for wave, i, lane in itertools.product(range(NW), range(Q), range(64)):
        slot = (wave * Q + i) * 64 + lane
        row = slot >> 3
        kin = 8 * ((slot & 7) ^ ((row >> 1) & 7))
        src_row, k = min(r0 + row, rows - 1), j * 2 * KBK + kin
        assert 0 <= src_row < rows and 0 <= k and k + 8 <= K
        lds[slot] = (src_row, k)
    assert len(lds) == R * 128 // 16
    return lds


@pytest.mark.parametrize("R,NW", [(256, 8), (128, 8), (128, 4), (64, 4)])
@pytest.mark.parametrize("rows,K,r0,j", [(8192, 4096, 0, 0), (8192, 4096, 7936, 63), (300, 128, 256, 1), (260, 64, 256, 0)])
def test_pair_fragments(R, NW, rows, K, r0, j):
    """B pairs of the 256 x 256 tile (8 waves), A pairs of the 256 x 256 and
    128 x 384 (8 waves), 128 x 128 and 64 x 128 (4 waves) tiles."""
    lds = pair_copies(R, NW, r0, rows, K, j)
    for row0, h, s in itertools.product(range(0, R, 32), range(2), range(2)):
        banks = {}
        for lane in range(64):
            r = lane & 31
            chunk = (4 * h + 2 * s + (lane >> 5)) ^ ((r >> 1) & 7)
            off = (row0 + r) * 128 + chunk * 16
            assert lds[off // 16] == (min(r0 + row0 + r, rows - 1), j * 64 + 32 * h + 16 * s + 8 * (lane >> 5))
            banks.setdefault(lane // 16, set()).add((off // 16) % 16)
        assert all(len(b) == 16 for b in banks.values())


@pytest.mark.parametrize("QA,QP", [(2, 4), (3, 2)])
@pytest.mark.parametrize("nk", [2, 4, 6, 8, 10, 12, 14, 16, 24, 26, 30, 128, 256])
def test_pair_schedule_and_waits(nk, QA, QP):
    """Iteration kt publishes k-tile kt+1, then issues the single-stage
    operand's k-tile kt+3 ("A" below) and, for even kt, the pair (kt+4, kt+5)
    into pair stage (kt/2 + 2) % 3; pairs past the end re-read the last one.
    Prologue: single 0, pair 0, single 1, single 2, pair 1.  Copies per wave:
    (single, pair) = (2, 4) for B pairs of 256 x 256 and A pairs of 128 x 128,
    (3, 2) for A pairs of 128 x 384."""
    pairs = nk // 2
    held = {}                                   # pair stage -> requested pair index
    queue = []                                  # issued copies in order: (kind, requested index)

    def issue_a(t):
        queue.extend([("A", t)] * QA)

    def issue_pair(jr):
        st = jr % 3
        if st in held:                          # everything in the old pair has been read
            for t in (2 * held[st], 2 * held[st] + 1):
                assert t >= nk or t <= last_read[0], ("overwritten before read", nk, jr)
        held[st] = jr
        queue.extend([("P", jr)] * QP)

    def wait(n, t):                             # in-order completion: all but the last n landed
        landed = queue[:len(queue) - n]
        for kind, idx in (("A", t), ("P", t // 2)):
            assert queue.count((kind, idx)) and landed.count((kind, idx)) == queue.count((kind, idx))
        st = (t // 2) % 3
        assert held[st] == t // 2 and t // 2 < pairs

    last_read = [-1]
    issue_a(0); issue_pair(0); issue_a(1); issue_a(2); issue_pair(1)
    wait(2 * QA + QP, 0)
    for kt in range(nk - 1):
        wait(QA + QP, kt + 1)                   # the barrier of iteration kt
        last_read[0] = kt - 1                   # every wave has read tile kt-1 by now
        issue_a(kt + 3)
        if kt % 2 == 0:
            issue_pair(kt // 2 + 2)


def test_random_ragged_sources():
    rng = random.Random(1)
    for _ in range(12):
        R, NW = rng.choice([(256, 8), (128, 4)])
        kmajor = rng.random() < 0.5
        rows = 8 * rng.randint(1, 90) if kmajor else rng.randint(1, 700)
        K = rng.randint(1, 300) if kmajor else 8 * rng.randint(1, 40)
        nk = -(-K // KBK)
        r0 = R * rng.randrange(-(-rows // R))
        for kc in (0, nk - 1):
            for a, b in single_copies(R, NW, kmajor, r0, rows, K, kc).values():
                assert (0 <= a < K and 0 <= b and b + 8 <= rows) if kmajor else (0 <= a < rows and 0 <= b and b + 8 <= K)


# ---- the 16 x 16 x 32 MFMA (MF16) -----------------------------------------------

def test_kcontig_fragments16():
    """OperandTile::frag16, k-contiguous: one ds_read_b128, lane l gets row
    row0 + l % 16, k 8 (l / 16) .. +7; each 16-lane group (one k-chunk) hits
    16 distinct 16-byte bank groups."""
    R, NW = 256, 8
    lds = single_copies(R, NW, False, 0, 10**6, 1024, 3, mf16=True)
    for row0 in range(0, R, 16):
        banks = {}
        for lane in range(64):
            chunk = (lane >> 4) ^ ((lane >> 2) & 3)
            off = (row0 + (lane & 15)) * 64 + chunk * 16
            assert lds[off // 16] == (row0 + (lane & 15), 3 * KBK + 8 * (lane >> 4))
            banks.setdefault(lane // 16, set()).add((off // 16) % 16)
        assert all(len(b) == 16 for b in banks.values())


@pytest.mark.parametrize("R,NW", [(256, 8), (128, 4), (384, 8)])
def test_kmajor_fragments16_through_the_transposing_read(R, NW):
    """OperandTile::frag16, k-major: two transposing reads; lane l receives
    column row0 + l % 16, k 8 (l / 16) + 4 H .. +3.  One read serves 32 lanes
    (256 bytes) per cycle; with the MF16 swizzle their 64 banks are
    distinct, without the extra bit groups 0 and 1 would collide."""
    lds = single_copies(R, NW, True, 0, 10**6, 1024, 5, mf16=True)

    def element(krow, byte):
        kr, col0 = lds[(krow * R * 2 + byte) // 16]
        return kr, col0 + (byte % 16) // 2

    def addresses(row0, H, mf16):
        addr = {}
        for lane in range(64):
            gi = lane & 15
            krow = 8 * (lane >> 4) + 4 * H + (gi >> 2)
            chunk = ((row0 >> 3) + ((gi & 3) >> 1)) ^ kswz(krow, mf16)
            addr[lane] = (krow, chunk * 16 + (gi & 1) * 8)
        return addr

    def banks_distinct(addr, half):
        banks = []
        for lane in range(32 * half, 32 * half + 32):
            krow, byte = addr[lane]
            b = (krow * R * 2 + byte) // 4 % 64
            banks += [b, (b + 1) % 64]
        return len(set(banks)) == 64

    for row0, H in itertools.product(range(0, R, 16), range(2)):
        addr = addresses(row0, H, True)
        for lane in range(64):
            g0, gi = lane & ~15, lane & 15
            for r in range(4):
                krow, byte = addr[g0 + 4 * r + (gi >> 2)]
                assert element(krow, byte + 2 * (gi & 3)) == (5 * KBK + 8 * (lane >> 4) + 4 * H + r, row0 + gi)
        assert banks_distinct(addr, 0) and banks_distinct(addr, 1)
    # the extra swizzle bit is what separates groups 0 and 1
    assert not banks_distinct(addresses(0, 0, False), 0)


@pytest.mark.parametrize("R,NW", [(256, 8), (128, 8), (128, 4), (64, 4)])
@pytest.mark.parametrize("rows,K,r0,j", [(8192, 4096, 0, 0), (300, 128, 256, 1)])
def test_pair_fragments16(R, NW, rows, K, r0, j):
    """OperandPairTile::frag16: half h of pair j, lane l gets row row0 + l % 16,
    k 64 j + 32 h + 8 (l / 16) .. +7."""
    lds = pair_copies(R, NW, r0, rows, K, j)
    for row0, h in itertools.product(range(0, R, 16), range(2)):
        banks = {}
        for lane in range(64):
            r = lane & 15
            chunk = (4 * h + (lane >> 4)) ^ ((r >> 1) & 7)
            off = (row0 + r) * 128 + chunk * 16
            assert lds[off // 16] == (min(r0 + row0 + r, rows - 1), j * 64 + 32 * h + 8 * (lane >> 4))
            banks.setdefault(lane // 16, set()).add((off // 16) % 16)
        assert all(len(b) == 16 for b in banks.values())


@pytest.mark.parametrize("WM,WN", [(128, 64), (64, 64), (64, 96)])
def test_mf16_result_lands_where_the_epilogues_expect(WM, WN):
    """mfmas16_col: half h multiplies A fragment i (rows h WM/2 + 16 i) with
    B fragment j (columns 16 j) into acc[j / 2][h TM/2 + i / 2], sub-block
    q = 2 (i % 2) + j % 2.  The MFMA puts D[4 (l / 16) + r][l % 16] (rows of
    operand 0 = columns n, columns of operand 1 = rows m) in lane l, register
    r.  store_tile reads acc[J][I][4 q + r] as m = 32 I + row_of(q) + l % 16,
    n = 32 J + col_of(q) + 4 (l / 16) + r; the restaging slab puts it at
    row row_of(q) + l % 16 of block I, 16-byte chunk 8 J + col_of(q) / 4 +
    l / 16, and every (m, n) of the wave tile is written exactly once."""
    TM, TN = WM // 32, WN // 32
    row_of = lambda q: 16 * (q >> 1)
    col_of = lambda q: 16 * (q & 1)
    seen = {}
    for h, i, j, lane, r in itertools.product(range(2), range(TM), range(2 * TN), range(64), range(4)):
        m = h * (WM // 2) + 16 * i + (lane & 15)           # MFMA result position
        n = 16 * j + 4 * (lane >> 4) + r
        J, I, q = j // 2, h * (TM // 2) + i // 2, 2 * (i % 2) + j % 2
        assert (32 * I + row_of(q) + (lane & 15), 32 * J + col_of(q) + 4 * (lane >> 4) + r) == (m, n)
        slab_row, chunk = row_of(q) + (lane & 15), 8 * J + col_of(q) // 4 + (lane >> 4)
        assert (32 * I + slab_row, 4 * chunk + r) == (m, n)
        assert (m, n) not in seen
        seen[(m, n)] = (J, I, 4 * q + r)
    assert len(seen) == WM * WN
