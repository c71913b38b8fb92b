"""Pins for the oracle's dispatch metadata (histogram, scan, stable placement).

Checked against numpy.bincount / cumsum / stable argsort, against the
per-expert boolean-mask gather of the lpnh.cn deep dive (section 3.2,
redistribute_tokens), and against the bijection / inverse properties that the
saved indices and locations of the DeepEP notes (section 7.5(2)) must have.
"""

import numpy as np
import pytest

import oracle
from moe_workloads import make_routing


@pytest.mark.parametrize("T,E,k,skew", [(1, 1, 1, 0), (257, 8, 2, 0), (1000, 32, 8, 0),
                                        (3000, 128, 4, 1.2), (500, 5, 5, 0), (0, 4, 2, 0)])
def test_dispatch_against_library_routines(T, E, k, skew):
    idx = make_routing(T, E, k, seed=T + E, skew=skew)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert counts.sum() == T * k and offsets[E] == T * k
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(idx.ravel(), kind="stable")  # expert-major, (token, slot) order kept
    assert np.array_equal(src, order // k)
    flat_dest = dest.ravel()
    assert np.array_equal(flat_dest[order], np.arange(T * k))
    # bijection onto [0, T*k) and src_token inverts dest_row
    assert np.array_equal(np.sort(flat_dest), np.arange(T * k))
    if T:
        assert np.array_equal(src[dest], np.repeat(np.arange(T), k).reshape(T, k))


def test_dispatch_equals_per_expert_mask_gather():
    T, E, k, d = 300, 12, 3, 5
    idx = make_routing(T, E, k, seed=4, skew=0.8)
    x = np.random.default_rng(0).standard_normal((T, d)).astype(np.float32)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    x_perm = x[src]
    # lpnh.cn 3.2: tokens[expert_ids == i] for each expert i, concatenated
    naive = np.concatenate([x[(idx == i).any(axis=1)] for i in range(E)])
    assert np.array_equal(x_perm, naive)
    # un-permute(permute(x)) == x, bit for bit
    for j in range(k):
        assert np.array_equal(x_perm[dest[:, j]], x)


def test_dispatch_rejects_bad_routing():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 4]], dtype=np.int32), 4)   # id out of range
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[1, 1]], dtype=np.int32), 4)   # same expert twice
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[-1, 0]], dtype=np.int32), 4)


def test_skewed_routing_leaves_empty_experts():
    idx = make_routing(4000, 128, 4, seed=2, skew=2.5)
    counts, offsets, _, _ = oracle.dispatch(idx, 128)
    assert (counts == 0).sum() > 0
    # empty experts have empty ranges
    assert np.all(offsets[1:][counts == 0] == offsets[:-1][counts == 0])


# ------------------------------------------------------- capacity limit ----
# The hard per-expert cap of the DeepEP notes (V3 load balancing, part A):
# in token order, an expert that already holds `cap` rows turns later tokens
# away (dropped here). Pinned by a per-expert rule written with numpy (the
# first `cap` tokens, by token id, among those that picked the expert), by
# the plain dispatch when the cap never binds, and by closed forms.

def _kept_by_rule(idx, E, cap):
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for e in range(E):
        t_hit, j_hit = np.nonzero(idx == e)          # row-major: ascending token id
        keep[t_hit[:cap], j_hit[:cap]] = True
    return keep


@pytest.mark.parametrize("T,E,k,cap,skew", [(200, 8, 2, 30, 0), (1000, 32, 8, 200, 0.7),
                                            (3000, 128, 4, 50, 2.5), (64, 4, 4, 1, 0),
                                            (300, 6, 3, 7, 1.0)])
def test_capacity_dispatch_against_per_expert_rule(T, E, k, cap, skew):
    idx = make_routing(T, E, k, seed=T + cap, skew=skew)
    counts, offsets, dest, src = oracle.dispatch(idx, E, capacity=cap)
    keep = _kept_by_rule(idx, E, cap)
    assert np.array_equal(dest >= 0, keep)
    assert np.array_equal(counts, np.minimum(np.bincount(idx.ravel(), minlength=E), cap))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    n = int(offsets[E])
    assert n == keep.sum() and n <= E * cap
    # kept slots: a bijection onto [0, n), expert-major and token-ascending
    kd = dest[keep]
    assert np.array_equal(np.sort(kd), np.arange(n))
    order = np.argsort(np.where(keep, idx, E).ravel(), kind="stable")[:n]
    assert np.array_equal(src[:n], order // k)
    assert np.array_equal(src[dest[keep]], np.nonzero(keep)[0])
    assert np.all(src[n:] == -1)


def test_capacity_that_never_binds_is_the_plain_dispatch():
    idx = make_routing(2000, 16, 4, seed=7, skew=1.5)
    plain = oracle.dispatch(idx, 16)
    capped = oracle.dispatch(idx, 16, capacity=int(plain[0].max()))
    for a, b in zip(plain, capped):
        assert np.array_equal(a, b)


def test_capacity_one_keeps_each_experts_first_token():
    idx = make_routing(500, 10, 3, seed=3)
    counts, offsets, dest, src = oracle.dispatch(idx, 10, capacity=1)
    for e in range(10):
        first = np.nonzero((idx == e).any(axis=1))[0]
        if len(first):
            assert counts[e] == 1 and src[offsets[e]] == first[0]
        else:
            assert counts[e] == 0


def test_capacity_rejects_bad_routing_and_negative_cap():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[1, 1]], dtype=np.int32), 4, capacity=2)
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 1]], dtype=np.int32), 4, capacity=-1)


# --------------------------------------------------- reassignment mode -----
# Overflow handed one at a time, in token order, to the least-loaded expert
# (ties to the lower id) while any expert is below the cap. Pinned by the
# closed form of that water-filling rather than by replaying it: with
# first-pass loads L_e = min(count_e, cap) and O overflowing assignments,
# N(v) = sum_e max(0, v - L_e) assignments raise every expert to level v, so
# the o-th overflow lands at the level v with N(v) <= o < N(v+1), on the
# (o - N(v))-th expert in id order among those with L_e <= v, as that
# expert's row v. The notes' claim that a cap at the average load makes the
# per-expert counts "rectangular" (all equal) is checked as well.

def _water_fill(L, O, cap):
    """expert and rank of each overflow index 0..O-1 (-1, -1 once all full)."""
    L = np.asarray(L, dtype=np.int64)
    N = lambda v: int(np.maximum(0, v - L).sum())
    out = []
    for o in range(O):
        if o >= N(cap):
            out.append((-1, -1))
            continue
        v = int(L.min())
        while N(v + 1) <= o:
            v += 1
        cand = np.nonzero(L <= v)[0]
        out.append((int(cand[o - N(v)]), v))
    return out


@pytest.mark.parametrize("T,E,k,cap,skew", [(200, 8, 2, 60, 1.0), (1000, 16, 4, 200, 2.0),
                                            (600, 32, 8, 130, 1.5), (300, 6, 3, 100, 0.3),
                                            (400, 10, 2, 30, 2.5)])
def test_reassignment_matches_water_filling(T, E, k, cap, skew):
    idx = make_routing(T, E, k, seed=T + k, skew=skew)
    counts, offsets, dest, src, route = oracle.dispatch(idx, E, capacity=cap, reassign=True,
                                                        return_route=True)
    first = _kept_by_rule(idx, E, cap)
    L = np.minimum(np.bincount(idx.ravel(), minlength=E), cap)
    over_t, over_j = np.nonzero(~first)                  # overflow in token order
    fill = _water_fill(L, len(over_t), cap)
    # first-pass slots keep their expert and rank
    assert np.array_equal(route[first], idx[first])
    exp_counts = L.copy()
    for (t, j), (e, v) in zip(zip(over_t, over_j), fill):
        assert route[t, j] == e
        if e >= 0:
            assert dest[t, j] == offsets[e] + v
            exp_counts[e] += 1
        else:
            assert dest[t, j] == -1
    assert np.array_equal(counts, exp_counts)
    assert counts.max() <= cap and counts.sum() == min(T * k, E * cap)
    n = int(offsets[E])
    kept = dest >= 0
    assert np.array_equal(np.sort(dest[kept]), np.arange(n))
    assert np.array_equal(src[dest[kept]], np.nonzero(kept)[0])


def test_cap_at_the_average_load_gives_equal_counts():
    T, E, k = 512, 16, 4
    cap = T * k // E
    idx = make_routing(T, E, k, seed=1, skew=2.0)
    counts, offsets, dest, _ = oracle.dispatch(idx, E, capacity=cap, reassign=True)
    assert np.all(counts == cap) and np.all(dest >= 0)


def test_reassignment_with_a_cap_that_never_binds_is_the_plain_dispatch():
    idx = make_routing(800, 12, 3, seed=5, skew=1.0)
    plain = oracle.dispatch(idx, 12)
    re = oracle.dispatch(idx, 12, capacity=int(plain[0].max()), reassign=True)
    for a, b in zip(plain, re):
        assert np.array_equal(a, b)
