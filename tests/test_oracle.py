"""Pins for the float64 CPU oracle.

Each test ties the oracle to something other than its own formula:
hand-derived values, closed forms of special cases, invariants of the
definition, central finite differences, and torch's float64 CPU attention
(independent library code). A dropped scale, a wrong sign, a transposed
operand, a wrong causal direction, a wrong head grouping or a missing max
subtraction each fails at least one of them (see test_oracle_mutations.py).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from workloads import draw, as_f64

HERE = os.path.dirname(os.path.abspath(__file__))
TIGHT = 1e-12


def rnd(B, H, Hkv, N, d, seed, gain=1.0, Nk=None):
    rng = np.random.default_rng(seed)
    Nk = N if Nk is None else Nk
    q = rng.standard_normal((B, N, H, d)) * gain
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, N, H, d))
    return q, k, v, do


def load_golden():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


# ---------------------------------------------------------------- hand-worked

@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_hand_worked_forward_backward(case):
    a = {k: np.array(case[k], np.float64) for k in ("q", "k", "v", "do", "o", "lse", "dq", "dk", "dv")}
    o, lse = oracle.forward(a["q"], a["k"], a["v"], case["causal"], case["scale"])
    np.testing.assert_allclose(o, a["o"], atol=1e-14)
    np.testing.assert_allclose(lse, a["lse"], atol=1e-14)
    dq, dk, dv = oracle.backward(a["q"], a["k"], a["v"], a["do"], case["causal"], case["scale"])
    np.testing.assert_allclose(dq, a["dq"], atol=1e-14)
    np.testing.assert_allclose(dk, a["dk"], atol=1e-14)
    np.testing.assert_allclose(dv, a["dv"], atol=1e-14)


# ---------------------------------------------------------------- forward invariants

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k, v, _ = rnd(1, 2, 2, 37, 8, 11)
    for h in range(2):
        p = oracle.probs(q, k, 0.3, causal, 0, h)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
        assert np.all(p >= 0)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)
            assert np.all(np.diag(p) > 0)


def test_causal_row0_returns_v0():
    q, k, v, _ = rnd(2, 4, 2, 19, 16, 12)
    scale = 1 / 4
    o, lse = oracle.forward(q, k, v, True, scale)
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(o[b, 0, h], v[b, 0, g])
            assert lse[b, h, 0] == pytest.approx(scale * np.dot(q[b, 0, h], k[b, 0, g]), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    q, k, v, do = rnd(1, 2, 1, 23, 8, 13)
    k[:] = k[:, :1]                      # every key row equal to row 0
    scale = 0.7
    o, lse = oracle.forward(q, k, v, causal, scale)
    N = q.shape[1]
    for h in range(2):
        for i in range(N):
            cnt = i + 1 if causal else N
            np.testing.assert_allclose(o[0, i, h], v[0, :cnt, 0].mean(axis=0), atol=1e-13)
            s = scale * np.dot(q[0, i, h], k[0, 0, 0])
            assert lse[0, h, i] == pytest.approx(s + math.log(cnt), abs=1e-13)
    # uniform rows do not depend on q: the query gradient vanishes
    dq, _, _ = oracle.backward(q, k, v, do, causal, scale)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform(causal):
    q, k, v, _ = rnd(1, 1, 1, 17, 4, 14)
    o, lse = oracle.forward(q, k, v, causal, 0.0)
    for i in range(17):
        cnt = i + 1 if causal else 17
        np.testing.assert_allclose(o[0, i, 0], v[0, :cnt, 0].mean(axis=0), atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(cnt), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_only_lse(causal):
    q, k, v, _ = rnd(1, 2, 2, 21, 8, 15)
    u = np.random.default_rng(1).standard_normal(8)
    scale = 0.35
    o1, l1 = oracle.forward(q, k, v, causal, scale)
    o2, l2 = oracle.forward(q, k + u, v, causal, scale)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    shift = scale * np.einsum("bnhd,d->bhn", q, u)
    np.testing.assert_allclose(l2, l1 + shift, atol=1e-12)


def test_noncausal_key_permutation_invariance():
    q, k, v, _ = rnd(1, 2, 2, 29, 8, 16)
    perm = np.random.default_rng(2).permutation(29)
    o1, l1 = oracle.forward(q, k, v, False, 0.4)
    o2, l2 = oracle.forward(q, k[:, perm], v[:, perm], False, 0.4)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


@pytest.mark.parametrize("gain", [1.0, 60.0, 1000.0])
@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_scipy_logsumexp(causal, gain):
    # gain 1000 makes scores of magnitude ~1e3-1e4: exp without max-subtraction overflows
    q, k, v, _ = rnd(1, 1, 1, 33, 16, 17, gain=gain)
    scale = 0.25
    _, lse = oracle.forward(q, k, v, causal, scale)
    s = scale * q[0, :, 0] @ k[0, :, 0].T
    for i in range(33):
        row = s[i, : i + 1] if causal else s[i]
        assert lse[0, 0, i] == pytest.approx(logsumexp(row), rel=1e-14, abs=1e-12)
    assert np.all(np.isfinite(lse))


def test_peaked_row_selects_one_value():
    # one key aligned with the query at a huge score: O is that key's value
    q, k, v, _ = rnd(1, 1, 1, 9, 4, 18)
    k[0, 5, 0] = q[0, 8, 0] * 1e3
    o, _ = oracle.forward(q, k, v, False, 1.0)
    np.testing.assert_allclose(o[0, 8, 0], v[0, 5, 0], atol=1e-12)


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2), (4, 1)])
def test_matches_torch_float64_attention(causal, H, Hkv):
    q, k, v, do = rnd(2, H, Hkv, 24, 8, 19)
    scale = 0.3
    o, lse = oracle.forward(q, k, v, causal, scale)
    dq, dk, dv = oracle.backward(q, k, v, do, causal, scale)

    G = H // Hkv
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_(True)
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    to = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(o, to.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    s = torch.matmul(tq.detach(), kk.detach().transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(24, 24, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.forward(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_backward_matches_finite_differences(causal, H, Hkv):
    q, k, v, do = rnd(1, H, Hkv, 7, 4, 20)
    scale = 0.45
    dq, dk, dv = oracle.backward(q, k, v, do, causal, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, k, v, do, causal, scale)
            x[idx] = old - eps
            fm = _loss(q, k, v, do, causal, scale)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    q, k, v, do = rnd(2, 4, 2, 31, 8, 21)
    scale = 0.3
    dq, dk, dv = oracle.backward(q, k, v, do, causal, scale)
    # rows of dS sum to zero, so the key gradients of a K/V head sum to zero
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # rows of P sum to one, so the value gradients sum to the group's dO
    grp = do.reshape(2, 31, 2, 2, 8).sum(axis=3)
    np.testing.assert_allclose(dv.sum(axis=1), grp.sum(axis=1), atol=1e-12)
    if causal:
        # the first query sees one key only: its softmax is constant
        np.testing.assert_allclose(dq[:, 0], 0.0, atol=1e-14)
    # sum_j P_ij dP_ij equals dO_i . O_i
    o, _ = oracle.forward(q, k, v, causal, scale)
    for h in range(4):
        p = oracle.probs(q, k, scale, causal, 1, h)
        dp = do[1, :, h] @ v[1, :, h // 2].T
        np.testing.assert_allclose((p * dp).sum(axis=1), np.sum(do[1, :, h] * o[1, :, h], axis=1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_kv(causal):
    q, k, v, do = rnd(1, 6, 2, 13, 8, 22)
    G = 3
    kr = np.repeat(k, G, axis=2)          # head h -> kv head h // G
    vr = np.repeat(v, G, axis=2)
    o1, l1 = oracle.forward(q, k, v, causal, 0.5)
    o2, l2 = oracle.forward(q, kr, vr, causal, 0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    dq1, dk1, dv1 = oracle.backward(q, k, v, do, causal, 0.5)
    dq2, dk2, dv2 = oracle.backward(q, kr, vr, do, causal, 0.5)
    np.testing.assert_allclose(dq1, dq2, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(1, 13, 2, G, 8).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(1, 13, 2, G, 8).sum(axis=3), atol=1e-13)


# ---------------------------------------------------------------- merge

@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_two_key_chunks_equals_full(causal):
    q, k, v, _ = rnd(2, 2, 2, 40, 8, 23)
    scale = 0.33
    o, lse = oracle.forward(q, k, v, causal, scale)
    cut = 17
    # query rows [cut, 40) against keys [0, cut) and [cut, 40)
    qa = q[:, cut:]
    oa, la = oracle.forward(qa, k[:, :cut], v[:, :cut], causal, scale, q_offset=cut, k_offset=0)
    ob, lb = oracle.forward(qa, k[:, cut:], v[:, cut:], causal, scale, q_offset=cut, k_offset=cut)
    om, lm = oracle.merge(oa, la, ob, lb)
    np.testing.assert_allclose(om, o[:, cut:], atol=1e-13)
    np.testing.assert_allclose(lm, lse[:, :, cut:], atol=1e-13)
    # order independence
    om2, lm2 = oracle.merge(ob, lb, oa, la)
    np.testing.assert_allclose(om2, om, atol=1e-15)
    np.testing.assert_allclose(lm2, lm, atol=1e-15)


def test_merge_associative_and_identity():
    q, k, v, _ = rnd(1, 1, 1, 30, 4, 24)
    parts = [oracle.forward(q, k[:, a:b], v[:, a:b], False, 0.6)
             for a, b in ((0, 7), (7, 19), (19, 30))]
    (o0, l0), (o1, l1), (o2, l2) = parts
    left = oracle.merge(*oracle.merge(o0, l0, o1, l1), o2, l2)
    right = oracle.merge(o0, l0, *oracle.merge(o1, l1, o2, l2))
    full = oracle.forward(q, k, v, False, 0.6)
    for a, b in zip(left, right):
        np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(left[0], full[0], atol=1e-13)
    np.testing.assert_allclose(left[1], full[1], atol=1e-13)
    # the empty partial (o = 0, lse = -inf) is the identity; two empties stay empty
    zo = np.zeros_like(o0)
    zl = np.full_like(l0, -np.inf)
    om, lm = oracle.merge(o0, l0, zo, zl)
    np.testing.assert_array_equal(om, o0)
    np.testing.assert_array_equal(lm, l0)
    oe, le = oracle.merge(zo, zl, zo, zl)
    assert np.all(oe == 0) and np.all(le == -np.inf)


def test_chunk_pairs_merge_to_full_causal():
    # every causal chunk pair (i, j<=i) of P chunks, merged per query chunk
    q, k, v, _ = rnd(1, 2, 1, 48, 8, 25)
    P, R = 4, 12
    o, lse = oracle.forward(q, k, v, True, 0.4)
    for i in range(P):
        qi = q[:, i * R:(i + 1) * R]
        acc = None
        for j in range(i + 1):
            part = oracle.forward(qi, k[:, j * R:(j + 1) * R], v[:, j * R:(j + 1) * R],
                                  i == j, 0.4, q_offset=i * R, k_offset=j * R)
            acc = part if acc is None else oracle.merge(*acc, *part)
        np.testing.assert_allclose(acc[0], o[:, i * R:(i + 1) * R], atol=1e-13)
        np.testing.assert_allclose(acc[1], lse[:, :, i * R:(i + 1) * R], atol=1e-13)


# ---------------------------------------------------------------- tiled online softmax

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(16, 16), (8, 32), (32, 8), (13, 7), (64, 64)])
def test_tiled_online_softmax_equals_naive(causal, br, bc):
    q, k, v, _ = rnd(1, 2, 1, 45, 8, 26, gain=3.0)
    o1, l1 = oracle.forward(q, k, v, causal, 0.4)
    o2, l2 = oracle.tiled_forward(q, k, v, causal, 0.4, br, bc)
    np.testing.assert_allclose(o2, o1, atol=TIGHT)
    np.testing.assert_allclose(l2, l1, atol=TIGHT)


# ---------------------------------------------------------------- sampled-row helpers

@pytest.mark.parametrize("causal", [False, True])
def test_sampled_row_helpers_match_full(causal):
    q, k, v, do = rnd(2, 4, 2, 50, 8, 27)
    scale = 0.3
    o, lse = oracle.forward(q, k, v, causal, scale)
    dq, dk, dv = oracle.backward(q, k, v, do, causal, scale)
    rows = np.array([0, 1, 17, 49])
    for b, h in ((0, 0), (1, 3)):
        ro, rl = oracle.forward_rows(q, k, v, causal, scale, b, h, rows)
        np.testing.assert_allclose(ro, o[b, rows, h], atol=1e-13)
        np.testing.assert_allclose(rl, lse[b, h, rows], atol=1e-13)
        np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, do, causal, scale, b, h, rows),
                                   dq[b, rows, h], atol=1e-13)
    for b, g in ((0, 1), (1, 0)):
        rk, rv = oracle.backward_dkdv_rows(q, k, v, do, causal, scale, b, g, rows, row_block=16)
        np.testing.assert_allclose(rk, dk[b, rows, g], atol=1e-12)
        np.testing.assert_allclose(rv, dv[b, rows, g], atol=1e-12)


def test_workload_draws_are_seeded_and_rounded():
    a = draw(1, 2, 1, 8, 4, seed=3)
    b = draw(1, 2, 1, 8, 4, seed=3)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
        assert x.dtype == torch.bfloat16
    # the oracle consumes the rounded values exactly
    q = as_f64(a[0])
    assert np.array_equal(q, a[0].float().double().numpy())


# ---------------------------------------------------------------- key/value cache (decode, chunked prefill)

def _kvcache_by_loops(q, k, v, k_lens, causal, scale):
    """The cache case written out element by element with math.exp: batch b
    uses cache rows [0, L_b); query row i sits at position L_b - Nq + i."""
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = H // Hkv
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = Nk if k_lens is None else min(max(int(k_lens[b]), 0), Nk)
        for i in range(Nq):
            pos = L - Nq + i
            for h in range(H):
                g = h // G
                keys = [j for j in range(L) if not causal or j <= pos]
                if not keys:
                    continue
                sc = [scale * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                lse[b, h, i] = mx + math.log(tot)
                for c in range(d):
                    o[b, i, h, c] = sum(wj * float(v[b, j, g, c]) for wj, j in zip(w, keys)) / tot
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_matches_elementwise_loops(causal):
    q, k, v, _ = draw(2, 4, 2, 7, 3, seed=71, dtype=torch.float64)
    q = q[:, :3]                                   # Nq = 3 new rows, Nk = 7 cache rows
    lens = [7, 4]
    o, lse = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), lens, causal, 0.7)
    ro, rl = _kvcache_by_loops(q.numpy(), k.numpy(), v.numpy(), lens, causal, 0.7)
    assert np.max(np.abs(o - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_kvcache_square_case_is_causal_attention():
    q, k, v, _ = draw(1, 2, 1, 9, 4, seed=72, dtype=torch.float64)
    o, lse = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), None, True, 0.5)
    ro, rl = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, 0.5)
    assert np.max(np.abs(o - ro)) < 1e-13 and np.max(np.abs(lse - rl)) < 1e-13


def test_kvcache_single_new_row_sees_the_whole_cache():
    # the last position sees every valid cache row, so causal = non-causal
    q, k, v, _ = draw(3, 4, 2, 11, 8, seed=73, dtype=torch.float64)
    q = q[:, :1]
    lens = [11, 6, 1]
    a = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), lens, True, 0.3)
    b = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), lens, False, 0.3)
    assert np.max(np.abs(a[0] - b[0])) < 1e-14 and np.max(np.abs(a[1] - b[1])) < 1e-14
    # a single valid key returns its value exactly, with lse = its score
    assert np.max(np.abs(a[0][2, 0] - np.repeat(v.numpy()[2, 0], 2, axis=0))) < 1e-14
    s0 = 0.3 * np.einsum("hd,hd->h", q.numpy()[2, 0], np.repeat(k.numpy()[2, 0], 2, axis=0))
    assert np.max(np.abs(a[1][2, :, 0] - s0)) < 1e-13


def test_kvcache_ignores_rows_past_the_valid_length():
    q, k, v, _ = draw(2, 2, 2, 10, 4, seed=74, dtype=torch.float64)
    q = q[:, :2]
    lens = [6, 3]
    a = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), lens, True, 0.5)
    k2, v2 = k.numpy().copy(), v.numpy().copy()
    k2[0, 6:] = 100.0
    v2[1, 3:] = -50.0
    b = oracle.forward_kvcache(q.numpy(), k2, v2, lens, True, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_kvcache_rows_without_keys_are_the_merge_identity():
    # L = 2 cache rows and Nq = 4 new rows: rows 0 and 1 sit at positions -2, -1
    q, k, v, _ = draw(1, 2, 2, 4, 4, seed=75, dtype=torch.float64)
    o, lse = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), [2], True, 0.5)
    assert np.all(o[0, :2] == 0.0) and np.all(np.isneginf(lse[0, :, :2]))
    assert np.all(np.isfinite(lse[0, :, 2:]))


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_key_splits_merge_to_the_whole(causal):
    # the split-KV scheme: partials over [0, s) and [s, L) merged by LSE
    q, k, v, _ = draw(1, 4, 2, 13, 8, seed=76, dtype=torch.float64)
    q = q[:, :2]
    L, cut = 13, 5
    full = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), [L], causal, 0.4)
    qpos = L - 2 + np.arange(2)
    parts = []
    for lo, hi in ((0, cut), (cut, L)):
        parts.append(oracle.forward(q.numpy(), k.numpy()[:, lo:hi], v.numpy()[:, lo:hi], causal, 0.4,
                                    q_offset=int(qpos[0]), k_offset=lo))
    o, lse = oracle.merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    assert np.max(np.abs(o - full[0])) < 1e-13 and np.max(np.abs(lse - full[1])) < 1e-13


# ---------------------------------------------------------------- sliding window (local attention)

def _window_by_loops(q, k, v, scale, window):
    """Causal sliding-window attention element by element with math.exp:
    query i sees keys j with i - window < j <= i."""
    B, N, H, d = q.shape
    G = H // k.shape[2]
    o = np.zeros(q.shape)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(N):
                keys = range(max(0, i - window + 1), i + 1)
                sc = [scale * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                lse[b, h, i] = mx + math.log(tot)
                for c in range(d):
                    o[b, i, h, c] = sum(wj * float(v[b, j, g, c]) for wj, j in zip(w, keys)) / tot
    return o, lse


@pytest.mark.parametrize("window", [1, 3, 6])
def test_window_matches_elementwise_loops(window):
    q, k, v, _ = draw(1, 4, 2, 9, 3, seed=81, dtype=torch.float64)
    o, lse = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, 0.6, window=window)
    ro, rl = _window_by_loops(q.numpy(), k.numpy(), v.numpy(), 0.6, window)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12


def test_window_covering_the_sequence_is_causal():
    q, k, v, do = draw(1, 2, 1, 12, 4, seed=82, dtype=torch.float64)
    a = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, 0.5, window=12)
    b = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ga = oracle.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), True, 0.5, window=40)
    gb = oracle.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), True, 0.5)
    assert all(np.array_equal(x, y) for x, y in zip(ga, gb))


def test_window_of_one_key_is_the_identity_map():
    # each query sees only its own key: O = V, LSE = its score, dQ = dK = 0, dV = dO summed per group
    q, k, v, do = draw(2, 4, 2, 10, 8, seed=83, dtype=torch.float64)
    o, lse = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, 0.3, window=1)
    vr = np.repeat(v.numpy(), 2, axis=2)
    assert np.max(np.abs(o - vr)) < 1e-14
    s = 0.3 * np.einsum("bnhd,bnhd->bhn", q.numpy(), np.repeat(k.numpy(), 2, axis=2))
    assert np.max(np.abs(lse - s)) < 1e-13
    dq, dk, dv = oracle.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), True, 0.3, window=1)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    dvr = do.numpy().reshape(2, 10, 2, 2, 8).sum(axis=3)
    assert np.max(np.abs(dv - dvr)) < 1e-13


def test_window_backward_matches_finite_differences():
    q, k, v, do = draw(1, 2, 1, 7, 3, seed=84, dtype=torch.float64)
    q, k, v, do = (t.numpy() for t in (q, k, v, do))
    W, sc, eps = 3, 0.8, 1e-6
    f = lambda qq, kk, vv: float(np.sum(do * oracle.forward(qq, kk, vv, True, sc, window=W)[0]))
    dq, dk, dv = oracle.backward(q, k, v, do, True, sc, window=W)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - g)) < 1e-7


# ---------------------------------------------------------------- packed variable-length batches

def _varlen_by_loops(q, k, v, cu, causal, scale, window=0):
    """Packed-batch attention element by element with math.exp: token i of
    sequence s sees the tokens j of the same sequence (j <= i under causal,
    and i - window < j with a window)."""
    total, H, d = q.shape
    G = H // k.shape[1]
    seq_of = [None] * total
    for s in range(len(cu) - 1):
        for t in range(int(cu[s]), int(cu[s + 1])):
            seq_of[t] = s
    o = np.zeros(q.shape)
    lse = np.full((H, total), -np.inf)
    for h in range(H):
        g = h // G
        for i in range(total):
            keys = [j for j in range(total) if seq_of[j] == seq_of[i] and (not causal or j <= i)
                    and (window == 0 or i - j < window)]
            sc = [scale * sum(float(q[i, h, c]) * float(k[j, g, c]) for c in range(d)) for j in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            lse[h, i] = mx + math.log(tot)
            for c in range(d):
                o[i, h, c] = sum(wj * float(v[j, g, c]) for wj, j in zip(w, keys)) / tot
    return o, lse


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 2)])
def test_varlen_matches_elementwise_loops(causal, window):
    from workloads import draw_varlen
    q, k, v, _, cu = draw_varlen([3, 0, 5, 1, 4], 4, 2, 3, seed=91, dtype=torch.float64)
    o, lse = oracle.forward_varlen(q.numpy(), k.numpy(), v.numpy(), cu.numpy(), causal, 0.7, window)
    ro, rl = _varlen_by_loops(q.numpy(), k.numpy(), v.numpy(), cu.numpy(), causal, 0.7, window)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_varlen_matches_torch_block_diagonal_attention(causal, window):
    # the packed batch as one sequence under a block-diagonal mask, through
    # torch's float64 attention and autograd
    from workloads import draw_varlen
    lengths = [6, 1, 9, 4]
    q, k, v, do, cu = draw_varlen(lengths, 4, 2, 8, seed=92, dtype=torch.float64)
    scale = 0.35
    o, lse = oracle.forward_varlen(q.numpy(), k.numpy(), v.numpy(), cu.numpy(), causal, scale, window)
    dq, dk, dv = oracle.backward_varlen(q.numpy(), k.numpy(), v.numpy(), do.numpy(), cu.numpy(), causal,
                                        scale, window)
    seq = torch.repeat_interleave(torch.arange(len(lengths)), torch.tensor(lengths))
    pos = torch.arange(seq.numel())
    allow = seq[:, None] == seq[None, :]
    if causal:
        allow &= pos[None, :] <= pos[:, None]
    if window:
        allow &= pos[:, None] - pos[None, :] < window
    tq = q.permute(1, 0, 2).clone().requires_grad_(True)
    tk = k.permute(1, 0, 2).clone().requires_grad_(True)
    tv = v.permute(1, 0, 2).clone().requires_grad_(True)
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, dim=0), tv.repeat_interleave(2, dim=0), attn_mask=allow, scale=scale)
    to.backward(do.permute(1, 0, 2))
    np.testing.assert_allclose(o, to.detach().permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(1, 0, 2).numpy(), atol=1e-12)
    s = torch.matmul(q.permute(1, 0, 2), k.permute(1, 2, 0).repeat_interleave(2, dim=0)) * scale
    ref_lse = torch.logsumexp(s.masked_fill(~allow, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12)


def test_varlen_equal_lengths_is_batched_attention():
    from workloads import draw_varlen
    q, k, v, do, cu = draw_varlen([7, 7, 7], 2, 1, 4, seed=93, dtype=torch.float64)
    o, lse = oracle.forward_varlen(q.numpy(), k.numpy(), v.numpy(), cu.numpy(), True, 0.5)
    bo, bl = oracle.forward(q.numpy().reshape(3, 7, 2, 4), k.numpy().reshape(3, 7, 1, 4),
                            v.numpy().reshape(3, 7, 1, 4), True, 0.5)
    assert np.array_equal(o, bo.reshape(21, 2, 4))
    assert np.array_equal(lse, bl.transpose(1, 0, 2).reshape(2, 21))
    g = oracle.backward_varlen(q.numpy(), k.numpy(), v.numpy(), do.numpy(), cu.numpy(), True, 0.5)
    bg = oracle.backward(*(t.numpy().reshape(3, 7, t.shape[1], 4) for t in (q, k, v, do)), True, 0.5)
    assert all(np.array_equal(x, y.reshape(x.shape)) for x, y in zip(g, bg))


def test_varlen_sequences_do_not_see_each_other():
    from workloads import draw_varlen
    q, k, v, do, cu = draw_varlen([5, 8, 3], 2, 2, 4, seed=94, dtype=torch.float64)
    base = oracle.forward_varlen(q.numpy(), k.numpy(), v.numpy(), cu.numpy(), False, 0.5)
    gb = oracle.backward_varlen(q.numpy(), k.numpy(), v.numpy(), do.numpy(), cu.numpy(), False, 0.5)
    k2, v2 = k.numpy().copy(), v.numpy().copy()
    k2[5:13] += 3.0
    v2[5:13] -= 2.0
    pert = oracle.forward_varlen(q.numpy(), k2, v2, cu.numpy(), False, 0.5)
    gp = oracle.backward_varlen(q.numpy(), k2, v2, do.numpy(), cu.numpy(), False, 0.5)
    keep = np.r_[0:5, 13:16]
    assert np.array_equal(base[0][keep], pert[0][keep]) and np.array_equal(base[1][:, keep], pert[1][:, keep])
    assert all(np.array_equal(x[keep], y[keep]) for x, y in zip(gb, gp))
    assert not np.allclose(base[0][5:13], pert[0][5:13])


# ---------------------------------------------------------------- block-sparse attention

def _bs_mask(nbr, nbc, seed, density=0.5):
    return (np.random.default_rng(seed).random((nbr, nbc)) < density).astype(np.uint8)


def _blocksparse_by_loops(q, k, v, mask, causal, scale, bq, bk):
    """Block-sparse attention element by element with math.exp: query i sees
    key j iff mask[i // bq][j // bk] != 0 (and j <= i under causal); a row
    with no key gets o = 0, lse = -inf."""
    B, N, H, d = q.shape
    G = H // k.shape[2]
    o = np.zeros(q.shape)
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(N):
                keys = [j for j in range(N) if mask[i // bq][j // bk] and (not causal or j <= i)]
                if not keys:
                    continue
                sc = [scale * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                lse[b, h, i] = mx + math.log(tot)
                for c in range(d):
                    o[b, i, h, c] = sum(wj * float(v[b, j, g, c]) for wj, j in zip(w, keys)) / tot
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_matches_elementwise_loops(causal):
    q, k, v, _ = draw(1, 4, 2, 11, 3, seed=101, dtype=torch.float64)
    mask = np.array([[0, 1, 1, 1], [0, 1, 0, 1], [1, 1, 0, 0]], np.uint8)   # 4-row x 3-key blocks
    o, lse = oracle.forward_blocksparse(q.numpy(), k.numpy(), v.numpy(), mask, causal, 0.6, bq=4, bk=3)
    ro, rl = _blocksparse_by_loops(q.numpy(), k.numpy(), v.numpy(), mask, causal, 0.6, 4, 3)
    assert np.array_equal(np.isfinite(lse), np.isfinite(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(lse[fin] - rl[fin])) < 1e-12
    if causal:   # rows 0-2 see only key block 0, masked out for row block 0: empty
        assert np.all(lse[:, :, :3] == -np.inf) and np.all(o[:, :3] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_matches_torch_masked_attention(causal):
    # the expanded element mask through torch's float64 attention and autograd
    # (the mask keeps the diagonal blocks, so no row is empty)
    B, H, Hkv, N, d, bq, bk = 2, 4, 2, 20, 8, 4, 2
    q, k, v, do = rnd(B, H, Hkv, N, d, 102)
    mask = _bs_mask(5, 10, 7)
    for r in range(5):
        mask[r, 2 * r:2 * r + 2] = 1
    scale = 0.4
    o, lse = oracle.forward_blocksparse(q, k, v, mask, causal, scale, bq, bk)
    dq, dk, dv = oracle.backward_blocksparse(q, k, v, do, mask, causal, scale, bq, bk)
    allow = torch.tensor(mask[np.arange(N)[:, None] // bq, np.arange(N)[None, :] // bk] != 0)
    if causal:
        allow &= torch.ones(N, N, dtype=torch.bool).tril()
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_(True)
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1), attn_mask=allow, scale=scale)
    to.backward(torch.tensor(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(o, to.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    s = torch.matmul(tq.detach(), tk.detach().repeat_interleave(2, dim=1).transpose(-1, -2)) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s.masked_fill(~allow, float("-inf")), -1).numpy(),
                               atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_with_every_block_kept_is_dense_attention(causal):
    q, k, v, do = rnd(1, 2, 1, 13, 4, 103)
    ones = np.ones((4, 7), np.uint8)
    a = oracle.forward_blocksparse(q, k, v, ones, causal, 0.5, 4, 2)
    b = oracle.forward(q, k, v, causal, 0.5)
    assert np.max(np.abs(a[0] - b[0])) < 1e-14 and np.max(np.abs(a[1] - b[1])) < 1e-14
    ga = oracle.backward_blocksparse(q, k, v, do, ones, causal, 0.5, 4, 2)
    gb = oracle.backward(q, k, v, do, causal, 0.5)
    assert all(np.max(np.abs(x - y)) < 1e-14 for x, y in zip(ga, gb))


def test_blocksparse_equals_attention_over_the_kept_keys():
    # non-causal: each row block attends to exactly the keys of its kept
    # blocks, so deleting the other keys gives the same rows
    q, k, v, _ = rnd(1, 2, 2, 24, 4, 104)
    mask = np.array([[1, 0, 0, 1], [0, 1, 1, 0], [1, 1, 1, 0]], np.uint8)   # 8-row x 6-key blocks
    o, lse = oracle.forward_blocksparse(q, k, v, mask, False, 0.7, 8, 6)
    for r in range(3):
        keys = np.concatenate([np.arange(6 * c, 6 * c + 6) for c in range(4) if mask[r, c]])
        ro, rl = oracle.forward(q[:, 8 * r:8 * r + 8], k[:, keys], v[:, keys], False, 0.7)
        assert np.max(np.abs(o[:, 8 * r:8 * r + 8] - ro)) < 1e-13
        assert np.max(np.abs(lse[:, :, 8 * r:8 * r + 8] - rl)) < 1e-13


def test_blocksparse_empty_rows_have_no_gradient_path():
    q, k, v, do = rnd(1, 2, 2, 12, 4, 105)
    mask = np.array([[0, 1], [1, 1], [0, 0]], np.uint8)                    # 4-row x 6-key blocks
    o, lse = oracle.forward_blocksparse(q, k, v, mask, True, 0.5, 4, 6)
    assert np.all(lse[:, :, 0:4] == -np.inf) and np.all(lse[:, :, 8:12] == -np.inf)
    assert np.all(o[:, 0:4] == 0.0) and np.all(o[:, 8:12] == 0.0)
    dq, dk, dv = oracle.backward_blocksparse(q, k, v, do, mask, True, 0.5, 4, 6)
    assert np.all(dq[:, 0:4] == 0.0) and np.all(dq[:, 8:12] == 0.0)
    do2 = do.copy()
    do2[:, 0:4] += 5.0
    do2[:, 8:12] -= 3.0
    g2 = oracle.backward_blocksparse(q, k, v, do2, mask, True, 0.5, 4, 6)
    assert np.array_equal(g2[1], dk) and np.array_equal(g2[2], dv)


def test_blocksparse_backward_matches_finite_differences():
    q, k, v, do = rnd(1, 2, 1, 9, 3, 106)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)          # 3-row x 3-key blocks
    f = lambda qq, kk, vv: float(np.sum(do * oracle.forward_blocksparse(qq, kk, vv, mask, False, 0.8, 3, 3)[0]))
    grads = oracle.backward_blocksparse(q, k, v, do, mask, False, 0.8, 3, 3)
    eps = 1e-6
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = f(q, k, v)
            x[idx] = old - eps
            fm = f(q, k, v)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - g)) < 2e-8


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_row_and_column_helpers_match_full(causal):
    q, k, v, do = rnd(1, 4, 2, 40, 4, 107)
    mask = _bs_mask(5, 10, 8)
    o, lse = oracle.forward_blocksparse(q, k, v, mask, causal, 0.3, 8, 4)
    dq, dk, dv = oracle.backward_blocksparse(q, k, v, do, mask, causal, 0.3, 8, 4)
    rows = [0, 3, 9, 17, 31, 39]
    for h in range(4):
        ro, rl, rq = oracle.blocksparse_rows(q, k, v, do, mask, causal, 0.3, 0, h, rows, 8, 4)
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse[0, h, rows]))
        assert np.max(np.abs(ro - o[0, rows, h])) < 1e-13 and np.max(np.abs(rl[fin] - lse[0, h, rows][fin])) < 1e-13
        assert np.max(np.abs(rq - dq[0, rows, h])) < 1e-13
    for g in range(2):
        rk, rv = oracle.blocksparse_dkdv_cols(q, k, v, do, mask, causal, 0.3, 0, g, rows, 8, 4, row_block=16)
        assert np.max(np.abs(rk - dk[0, rows, g])) < 1e-13 and np.max(np.abs(rv - dv[0, rows, g])) < 1e-13
