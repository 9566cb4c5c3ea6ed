"""Pins of the oracle's routing and plan against brute force and invariants (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import build_plan, route_from_logits, route_from_logits_fast


def _brute_topk(row, k):
    # full sort by (logit descending, index ascending)
    return [e for _, e in sorted(((-float(v), e) for e, v in enumerate(row)))][:k]


@pytest.mark.parametrize("seed,T,E,k", [(0, 7, 8, 2), (1, 5, 16, 4), (2, 3, 5, 5), (3, 9, 128, 4)])
def test_topk_matches_full_sort(seed, T, E, k):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route_from_logits(lg, k)
    for t in range(T):
        assert idx[t].tolist() == _brute_topk(lg[t], k)
    idx2, w2 = route_from_logits_fast(lg, k)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w, w2, rtol=0, atol=1e-15)


def test_topk_ties_go_to_lower_index():
    lg = np.array([[1, 3, 3, 0, 3], [0, 0, 0, 0, 0]], dtype=np.float32)
    idx, w = route_from_logits(lg, 3)
    assert idx.tolist() == [[1, 2, 4], [0, 1, 2]]
    assert np.allclose(w, 1.0 / 3, rtol=0, atol=1e-15)


def test_bias_hand_case():
    # a large bias on expert 0 ranks it first although its logit is the smallest;
    # the weights are the softmax of the two selected *unbiased* logits (1 and 4)
    lg = np.array([[1, 2, 3, 4]], dtype=np.float32)
    bias = np.array([10, 0, 0, 0], dtype=np.float32)
    idx, w = route_from_logits(lg, 2, bias)
    assert idx.tolist() == [[0, 3]]
    e1, e4 = np.exp(1.0), np.exp(4.0)
    assert np.allclose(w[0], [e1 / (e1 + e4), e4 / (e1 + e4)], rtol=0, atol=1e-15)


def test_bias_zero_is_unbiased_and_bias_only_ranks():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((9, 24)).astype(np.float32)
    idx0, w0 = route_from_logits(lg, 4)
    idx1, w1 = route_from_logits(lg, 4, np.zeros(24, dtype=np.float32))
    assert np.array_equal(idx0, idx1) and np.array_equal(w0, w1)
    # with a random bias: the selection is the brute-force top-k of the fp32 sum,
    # and the weights are a softmax over the selected raw logits
    bias = rng.standard_normal(24).astype(np.float32)
    idx, w = route_from_logits(lg, 4, bias)
    key = (lg + bias[None, :]).astype(np.float32)
    for t in range(9):
        assert idx[t].tolist() == _brute_topk(key[t], 4)
        sel = lg[t, idx[t]].astype(np.float64)
        assert np.allclose(w[t], np.exp(sel) / np.exp(sel).sum(), rtol=0, atol=1e-14)
    idx2, w2 = route_from_logits_fast(lg, 4, bias)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w, w2, rtol=0, atol=1e-15)


def test_softmax_over_topk_equals_renormalised_full_softmax():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((6, 10)).astype(np.float32)
    idx, w = route_from_logits(lg, 3)
    for t in range(6):
        full = np.exp(lg[t].astype(np.float64))
        full /= full.sum()
        sel = full[idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-14
        assert np.all(np.diff(w[t]) <= 0)


def _check_plan_invariants(ids, E, plan):
    flat = np.asarray(ids).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = plan["expert_counts"]
    start = plan["expert_start_indices"]
    src = plan["src_info"]
    pr = plan["pair_row"]
    assert counts.sum() == valid.sum() == start[-1] == src.size
    assert start[0] == 0 and np.all(np.diff(start) == counts)
    # inverse maps
    assert np.array_equal(pr[src], np.arange(src.size))
    assert np.all(pr[~valid] == -1)
    # each segment holds its expert's pairs in ascending pair order
    for e in range(E):
        seg = src[start[e]:start[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    # equals a stable argsort of the valid pairs by expert
    vp = np.nonzero(valid)[0]
    assert np.array_equal(src, vp[np.argsort(flat[vp], kind="stable")])
    act = [e for e in range(E) if counts[e] > 0]
    assert plan["num_active"] == len(act)
    assert plan["expert_ids"].tolist() == act + [-1] * (E - len(act))
    assert plan["status"] == int(np.sum(~valid & (flat != -1)))


@pytest.mark.parametrize("case", ["random", "one_expert", "masked", "bad_ids", "dups", "empty", "all_masked"])
def test_plan_invariants(case):
    rng = np.random.default_rng(11)
    T, k, E = 37, 4, 9
    ids = rng.integers(0, E, size=(T, k))
    if case == "one_expert":
        ids[:] = 3
    elif case == "masked":
        ids[rng.random((T, k)) < 0.3] = -1
    elif case == "bad_ids":
        ids[0, 0], ids[5, 2], ids[7, 1] = E, -5, 1000
    elif case == "dups":
        ids[:, 1] = ids[:, 0]
    elif case == "empty":
        ids = ids[:0]
    elif case == "all_masked":
        ids[:] = -1
    plan = build_plan(ids, E)
    _check_plan_invariants(ids, E, plan)


def test_plan_hand_case():
    # T=3, k=2, E=4: pairs p = t*k + j
    ids = np.array([[2, 0], [2, -1], [0, 2]])
    plan = build_plan(ids, 4)
    assert plan["expert_counts"].tolist() == [2, 0, 3, 0]
    assert plan["expert_start_indices"].tolist() == [0, 2, 2, 5, 5]
    assert plan["src_info"].tolist() == [1, 4, 0, 2, 5]
    assert plan["pair_row"].tolist() == [2, 0, 3, -1, 1, 4]
    assert plan["expert_ids"].tolist() == [0, 2, -1, -1]
    assert plan["num_active"] == 2


def test_plan_exhaustive_tiny():
    # every routing of T=2 tokens, k=2 slots over E=3 experts (with masked slots)
    for combo in itertools.product([-1, 0, 1, 2], repeat=4):
        ids = np.array(combo).reshape(2, 2)
        _check_plan_invariants(ids, 3, build_plan(ids, 3))


def test_nan_logit_ranks_last_and_gets_weight_zero():
    # MoEActivationPack page, routing_input_mode FromLogits; the pages say nothing of
    # NaN logits.  Reading: a NaN logit is -inf, for the ranking and in the softmax.
    # Token 0 has two real logits and k = 3, so one NaN expert is selected (the lower
    # index among the tied -inf keys) and its weight is exp(-inf) / sum = 0.
    nan = np.float32("nan")
    lg = np.array([[nan, 1, 2, nan], [0.5, nan, -1, 3]], dtype=np.float32)
    e1, e2 = np.exp(1.0), np.exp(2.0)
    for fn in (route_from_logits, route_from_logits_fast):
        idx, w = fn(lg, 3)
        assert idx.tolist() == [[2, 1, 0], [3, 0, 2]]
        assert np.allclose(w[0], [e2 / (e1 + e2), e1 / (e1 + e2), 0.0], rtol=0, atol=1e-15)
        assert w[0, 2] == 0.0
        ex = np.exp(np.array([3.0, 0.5, -1.0]))
        assert np.allclose(w[1], ex / ex.sum(), rtol=0, atol=1e-15)


def test_nan_logit_with_bias_and_all_nan_row():
    nan = np.float32("nan")
    # a bias cannot lift a NaN logit: logit + bias is NaN, which ranks last
    lg = np.array([[nan, 0, 1]], dtype=np.float32)
    bias = np.array([100, 0, 0], dtype=np.float32)
    for fn in (route_from_logits, route_from_logits_fast):
        idx, w = fn(lg, 2, bias)
        assert idx.tolist() == [[2, 1]]
        assert np.allclose(w[0], [np.exp(1) / (np.exp(1) + 1), 1 / (np.exp(1) + 1)], rtol=0, atol=1e-15)
    # every selected logit -inf: ids by index, the softmax is 0/0 (NaN weights)
    for fn in (route_from_logits, route_from_logits_fast):
        idx, w = fn(np.full((1, 4), nan, np.float32), 2)
        assert idx.tolist() == [[0, 1]]
        assert np.isnan(w).all()
