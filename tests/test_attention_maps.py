"""CPU model of the attention kernel's key-block and query maps
(csrc/attention.hip), checked before any GPU run.

The kernel processes key blocks of 32 in two groups of waves (group g takes
blocks b = 2 it + g, it < nit = ceil(nblk / 2)); block kb is copied from the
window of 32 keys starting at kbase = min(32 kb, seq - 32), and its window
place p (0 .. 31) holds key kbase + p.  A place is masked when it precedes
the block (p < 32 kb - kbase: already counted, or a phantom block) or, with
the causal mask, when its key is later than the query.  These tests restate
those formulas and check, for ragged sequence lengths, that every copy row
stays inside the batch's sequence and that each key a query may attend is
counted exactly once.
"""
import pytest

KBKV, KBQ = 32, 128


def blocks(seq, qb, causal):
    nblk_all = -(-seq // KBKV)
    nblk = min(nblk_all, (qb + 1) * (KBQ // KBKV)) if causal else nblk_all
    return nblk, -(-nblk // 2)


def key_base(kb, seq):
    return min(kb * KBKV, seq - KBKV)


@pytest.mark.parametrize("seq", [32, 33, 40, 63, 64, 96, 100, 127, 128, 129, 160, 200, 333, 1000, 4095, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_every_key_once_and_copies_in_bounds(seq, causal):
    batch = 2
    nqb = -(-seq // KBQ)
    for b in range(batch):
        row0 = b * seq
        for qb in (range(nqb) if nqb <= 8 else (0, 1, nqb // 2, nqb - 2, nqb - 1)):
            nblk, nit = blocks(seq, qb, causal)
            # copies: iterations issue blocks 2 it, 2 it + 1 for it < nit + 3
            for j in range(2 * (nit + 3)):
                kc = min(j, nblk - 1)
                base = row0 + key_base(kc, seq)
                assert row0 <= base and base + KBKV <= row0 + seq
            for query in range(qb * KBQ, qb * KBQ + KBQ):
                qrow = row0 + min(query, seq - 1)
                assert row0 <= qrow < row0 + seq
                if query >= seq:
                    continue           # loads the last query's row, stores nothing
                seen = []
                for g in range(2):
                    for it in range(nit):
                        kb = 2 * it + g
                        kbase = key_base(kb, seq)
                        lo = kb * KBKV - kbase
                        for p in range(KBKV):
                            key = kbase + p
                            if p < lo or (causal and key > query):
                                continue
                            seen.append(key)
                want = list(range(query + 1 if causal else seq))
                assert sorted(seen) == want, (seq, qb, query)


@pytest.mark.parametrize("seq", [100, 4096])
def test_the_mask_threshold_forms_agree(seq):
    """The kernel takes the masks as thresholds on c(R) = 8 (R / 4) + R % 4
    against lo - 4 h and query - kbase - 4 h (lane half h): the same places
    as the key comparisons they stand for."""
    for kb in range(-(-seq // KBKV) + 1):
        kbase = key_base(kb, seq)
        lo = kb * KBKV - kbase
        for h in range(2):
            for query in (0, 5, kbase + 7, kbase + 31, seq - 1):
                for r in range(16):
                    c = 8 * (r // 4) + r % 4
                    place = 4 * h + c
                    key = kbase + place
                    assert (c < lo - 4 * h) == (key < kb * KBKV)
                    assert (c > query - kbase - 4 * h) == (key > query)


def grid_map(i, batch, heads, nqb, causal):
    """Workgroup id -> (batch, head, query block), as the kernel derives it."""
    head = i % heads
    if causal:
        return (i // heads) % batch, head, nqb - 1 - i // (heads * batch)
    return i // (heads * nqb), head, (i // heads) % nqb


@pytest.mark.parametrize("batch,heads,nqb", [(1, 8, 32), (3, 5, 7), (2, 16, 1), (4, 1, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_grid_map_covers_every_block_once(batch, heads, nqb, causal):
    """Every (batch, head, query block) gets exactly one workgroup; heads
    vary fastest (one head per XCD with 8 local heads); causal grids run the
    query blocks, whose rows grow with the index, from the last to the first."""
    n = batch * heads * nqb
    got = [grid_map(i, batch, heads, nqb, causal) for i in range(n)]
    assert sorted(got) == [(b, h, q) for b in range(batch) for h in range(heads) for q in range(nqb)]
    assert all(got[i][1] == i % heads for i in range(n))
    if causal:
        assert all(got[i][2] >= got[i + 1][2] for i in range(n - 1))


@pytest.mark.parametrize("seq", [128, 129, 200, 256, 333, 1000, 4095, 4096])
def test_split_rows_count_every_key_once(seq):
    """Causal launches that fit one round split each query block's key
    iterations into two halves (the first rounded up; blk0 = twice the first
    half's count for the second workgroup): both halves are non-empty from
    128 keys on, and together they count every key a query may attend once."""
    nqb = -(-seq // KBQ)
    for qb in range(nqb):
        nblk, nit_row = blocks(seq, qb, True)
        first = (nit_row + 1) // 2
        halves = [(0, first), (2 * first, nit_row - first)]
        assert all(n >= 1 for _, n in halves)
        for query in range(qb * KBQ, min(qb * KBQ + KBQ, seq)):
            seen = []
            for blk0, nit in halves:
                for g in range(2):
                    for it in range(nit):
                        kb = blk0 + 2 * it + g
                        kc = min(kb, nblk - 1)              # the block copied
                        assert 0 <= key_base(kc, seq) <= seq - KBKV
                        kbase = key_base(kb, seq)
                        lo = kb * KBKV - kbase
                        seen += [kbase + p for p in range(KBKV) if p >= lo and kbase + p <= query]
            assert sorted(seen) == list(range(query + 1)), (seq, qb, query)
