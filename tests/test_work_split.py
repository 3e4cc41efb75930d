"""CPU model of how the persistent blocks of the grouped matrix-core kernel split a launch's work (split_item in
q4_grouping.h: run by the blocks themselves, or by the grouping launch to write one descriptor per block): the
shared matrix's (token chunk, step) pairs and the routed chunks' steps.  The function below restates the
integer arithmetic; the tests check that every piece of work is done exactly once for grids of 2 to 1024
blocks and 0 to 700 routed chunks, that a block never holds more than one item unless there are more chunks
(or token chunks) than blocks, that the host's single-item check (split_single_item) agrees with that, and
that the token chunks of one shared step range run on one XCD (block b runs on XCD b mod 8) wherever the
ranges fill octets, and on 8 / L XCDs for the L ranges after the last full octet when that divides evenly."""
import itertools

import pytest


def next_item(b, nb, it, T, steps_shared, steps_routed, ng):
    """(shared, chunk or token chunk, s0, s1) of item `it` of block b, or None; the kernel's arithmetic."""
    ng = ng if steps_routed > 0 else 0
    ss, tc = steps_shared, (T + 15) // 16
    nsb, rs = 0, 1
    if ss > 0:
        if ng <= 0:
            nsb = nb
        else:
            us, ur = ss * tc, steps_routed * ng
            nsb = (nb * us + (us + ur) // 2) // (us + ur)
            nsb = max(1, min(nsb, nb - 1))
        rs = max(1, nsb // tc)
        nsb = nsb if nsb < tc else rs * tc
    if b < nsb:
        if nsb < tc:
            c = b + it * nsb
            return None if c >= tc else (True, c, 0, ss)
        if it > 0:
            return None
        full = (rs // 8) * 8
        L = rs - full
        if b < full * tc:
            o, w = divmod(b, 8 * tc)
            c, r = w // 8, 8 * o + w % 8
        else:
            b2 = b - full * tc
            g = 8 // L
            if 8 % L == 0 and tc % g == 0:
                m, x = b2 // 8, b2 % 8
                r, c = full + x % L, (x // L) * (tc // g) + m
            else:
                c, r = b2 % tc, full + b2 // tc
        return True, c, r * ss // rs, (r + 1) * ss // rs
    if ng <= 0:
        return None
    o, R, steps = b - nsb, nb - nsb, steps_routed
    s0, s1 = 0, steps
    if ng <= R:
        if it > 0:
            return None
        q, rem = divmod(R, ng)
        if o < rem * (q + 1):
            j, part, parts = o // (q + 1), o % (q + 1), q + 1
        else:
            o2 = o - rem * (q + 1)
            j, part, parts = rem + o2 // q, o2 % q, q
        s0, s1 = part * steps // parts, (part + 1) * steps // parts
    else:
        j = o + it * R
        if j >= ng:
            return None
    return False, j, s0, s1


def items_of(nb, T, ss, sr, ng):
    out = {}
    for b in range(nb):
        lst = []
        for it in itertools.count():
            x = next_item(b, nb, it, T, ss, sr, ng)
            if x is None:
                break
            lst.append(x)
        out[b] = lst
    return out


def check(nb, T, ss, sr, ng):
    tc = (T + 15) // 16
    items = items_of(nb, T, ss, sr, ng)
    shared, routed = {}, {}
    for b, lst in items.items():
        for sh, j, s0, s1 in lst:
            assert 0 <= s0 <= s1
            for s in range(s0, s1):
                key = (j, s)
                d = shared if sh else routed
                assert key not in d, f"nb={nb} T={T}: {('shared', 'routed')[not sh]} {key} twice"
                d[key] = b
    if ss > 0:
        assert set(shared) == {(c, s) for c in range(tc) for s in range(ss)}
    else:
        assert not shared
    if sr > 0 and ng > 0:
        assert set(routed) == {(j, s) for j in range(ng) for s in range(sr)}
    else:
        assert not routed
    return items, shared


CASES = [(nb, T, ss, sr, ng)
         for nb in (2, 3, 8, 64, 255, 512, 1024)
         for T in (2, 16, 17, 32, 128, 300)
         for ss, sr in ((0, 88), (352, 0), (352, 88), (176, 44), (1, 1), (704, 22))
         for ng in (0, 1, 5, 107, 135, 700)]


@pytest.mark.parametrize("nb,T,ss,sr,ng", CASES)
def test_every_step_once(nb, T, ss, sr, ng):
    if ss == 0 and (sr == 0 or ng == 0):
        return
    check(nb, T, ss, sr, ng)


@pytest.mark.parametrize("T,ng", [(32, 107), (128, 135), (64, 120), (256, 128)])
def test_token_chunks_of_a_range_share_an_xcd(T, ng):
    """The bench's launches (512 blocks; gate/up: 352 shared steps and 88 per routed chunk; down: 176 and
    44): in every octet of full step ranges, the tc token chunks of a range are on blocks with the same
    index mod 8, so that the L2 of one XCD serves the matrix's rows to all of them."""
    for ss, sr in ((352, 88), (176, 44)):
        nb, tc = 512, (T + 15) // 16
        items, shared = check(nb, T, ss, sr, ng)
        by_range = {}
        for b, lst in items.items():
            for sh, c, s0, s1 in lst:
                if sh:
                    by_range.setdefault((s0, s1), set()).add(b % 8)
        nsb = sum(1 for lst in items.values() if lst and lst[0][0])
        rs = nsb // tc
        full = (rs // 8) * 8
        assert full >= 1 or rs < 8
        ranges = sorted(by_range)
        for r in range(full):
            assert len(by_range[ranges[r]]) == 1, f"T={T}: range {ranges[r]} on XCDs {by_range[ranges[r]]}"
        L = rs - full
        if L and 8 % L == 0 and tc % (8 // L) == 0:
            for r in range(full, rs):
                assert len(by_range[ranges[r]]) == 8 // L, f"T={T}: range {ranges[r]} on XCDs {by_range[ranges[r]]}"


def test_one_item_per_block_when_blocks_suffice():
    """With at least as many routed blocks as chunks (the bench's launches), every block holds one item, so
    no block pays a second chunk's setup."""
    for T, ss, sr, ng in ((32, 352, 88, 107), (128, 352, 88, 135), (32, 176, 44, 107), (128, 176, 44, 135)):
        items = items_of(512, T, ss, sr, ng)
        assert max(len(v) for v in items.values()) == 1
        assert sum(len(v) for v in items.values()) == 512


def split_counts(nb, T, ss, sr, ng):
    ng = ng if sr > 0 else 0
    tc = (T + 15) // 16
    nsb, rs = 0, 1
    if ss > 0:
        if ng <= 0:
            nsb = nb
        else:
            us, ur = ss * tc, sr * ng
            nsb = max(1, min((nb * us + (us + ur) // 2) // (us + ur), nb - 1))
        rs = max(1, nsb // tc)
        nsb = nsb if nsb < tc else rs * tc
    return nsb, rs


def split_single_item(nb, T, ss, sr, ng_max):
    """The host's check (q4_grouping.h) that no block gets a second item for any chunk count up to ng_max."""
    tc = (T + 15) // 16
    for ng in (range(1, ng_max + 1) if sr > 0 else [0]):
        nsb, rs = split_counts(nb, T, ss, sr, ng)
        if ss > 0 and nsb < tc and tc > 1:
            return False
        if ng > nb - nsb:
            return False
    return True


@pytest.mark.parametrize("nb,T,ss,sr", [(512, 32, 352, 88), (512, 128, 176, 44), (64, 300, 352, 88), (8, 2, 44, 88),
                                        (512, 4096, 16, 16), (3, 17, 1, 1), (512, 1000, 352, 88)])
def test_single_item_check_matches_the_split(nb, T, ss, sr):
    """Whenever the host's check passes for chunk counts up to ng_max, every block of every such launch holds at
    most one item (the descriptor launch would be exact); when it fails, some chunk count needs a second item."""
    for ng_max in (1, 5, 107, 145, 193, 600):
        ok = split_single_item(nb, T, ss, sr, ng_max)
        worst = max(max(len(v) for v in items_of(nb, T, ss, sr, ng).values()) for ng in range(1, ng_max + 1))
        assert ok == (worst <= 1), (nb, T, ss, sr, ng_max, ok, worst)


def grouping_chunks(ids, n_valid):
    """The grouping's chunk table: experts in order (ids outside the pool last), each expert's pairs in runs of
    16: (record or n_valid, first index into the grouped pair order, count)."""
    bucket = [i if 0 <= i < n_valid else n_valid for i in ids]
    cnt = [bucket.count(b) for b in range(n_valid + 1)]
    out, start = [], 0
    for b in range(n_valid + 1):
        for c in range(0, cnt[b], 16):
            out.append((b, start + c, min(16, cnt[b] - c)))
        start += cnt[b]
    return out


def plan_share_descriptor(ids, n_valid, nb, T, ss, sr, b):
    """One block's descriptor as a descriptor block writes it (plan_share in q4_grouping.h): the chunk table
    rebuilt from per-expert counts and their prefix sums, chunk j found by a binary search for the last
    expert whose first chunk is at most j; the item from split_item."""
    nbk = n_valid + 1
    pcnt = [0] * nbk
    for i in ids:
        pcnt[i if 0 <= i < n_valid else n_valid] += 1
    pre_x, pre_z, x, z = [], [], 0, 0
    for b2 in range(nbk):
        pre_x.append(x)
        pre_z.append(z)
        x += pcnt[b2]
        z += (pcnt[b2] + 15) // 16
    ng = z
    item = next_item(b, nb, 0, T, ss, sr, ng)
    if item is None or item[2] >= item[3]:
        return None
    shared, j, s0, s1 = item
    if shared:
        return (True, 0, 16 * j, min(16, T - 16 * j), s0, s1)
    lo, hi = 0, nbk - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if pre_z[mid] <= j:
            lo = mid
        else:
            hi = mid - 1
    k0 = (j - pre_z[lo]) * 16
    return (False, lo, pre_x[lo] + k0, min(16, pcnt[lo] - k0), s0, s1)


@pytest.mark.parametrize("T,k,E,ss,sr,kind", [(32, 8, 128, 352, 88, "perm"), (128, 8, 128, 176, 44, "zipf"),
                                              (24, 2, 8, 4, 4, "perm"), (7, 2, 8, 4, 4, "invalid"),
                                              (200, 4, 16, 352, 88, "zipf")])
def test_descriptors_equal_the_grouping(T, k, E, ss, sr, kind):
    """Every block's descriptor, as the descriptor blocks rebuild it from the ids, names the chunk of the
    grouping's own table that split_item assigns to the block (record, first pair, count) and its steps."""
    import numpy as np
    rng = np.random.default_rng(T * 7 + k)
    if kind == "perm":
        ids = np.concatenate([rng.permutation(E)[:k] for _ in range(T)])
    elif kind == "zipf":
        r = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        ids = rng.choice(E, size=T * k, p=r / r.sum())
    else:
        ids = rng.integers(-2, E + 2, size=T * k)
    ids = ids.tolist()
    table = grouping_chunks(ids, E)
    ng = len(table)
    nb = 512
    assert split_single_item(nb, T, ss, sr, ng)
    for b in range(nb):
        d = plan_share_descriptor(ids, E, nb, T, ss, sr, b)
        it = next_item(b, nb, 0, T, ss, sr, ng)
        if d is None:
            assert it is None or it[2] >= it[3]
            continue
        shared, rec, start, count, s0, s1 = d
        assert (shared, s0, s1) == (it[0], it[2], it[3])
        if not shared:
            assert (rec, start, count) == table[it[1]], (b, it)
