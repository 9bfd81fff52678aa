"""GPU parity of the key/value-cache forward (attn_fwd_kvcache, split over
key ranges and merged by logsumexp) against the float64 oracle's
forward_kvcache on the same seeded inputs, element by element."""
import numpy as np
import pytest
import torch

import exact_attention_37_amd as mi
import oracle
from workloads import CACHE_WORKLOADS, draw_cache, draw_cache_workload, as_f64
from tests.helpers import check_bf16, check_abs, f64, BF16_LSE_ABS

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_case(q, k, v, lens, causal, scale, nsplit):
    print("case", tuple(q.shape), tuple(k.shape), None if lens is None else lens.tolist(),
          "causal", causal, "nsplit", nsplit, flush=True)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ld = None if lens is None else lens.to(DEV)
    o, lse = mi.fwd_kvcache(qd, kd, vd, ld, causal, scale, nsplit)
    torch.cuda.synchronize()
    ro, rl = oracle.forward_kvcache(as_f64(q), as_f64(k), as_f64(v),
                                    None if lens is None else lens.tolist(), causal, scale)
    eo = check_bf16("o", f64(o), ro)
    el = check_abs("lse", f64(lse), rl, BF16_LSE_ABS)
    print("errors o %.3g lse %.3g" % (eo, el), flush=True)
    return o, lse


# (B, H, Hkv, Nq, Nk, d, lens, causal, nsplit)
CASES = [
    (2, 8, 2, 1, 1000, 128, [1000, 517], True, 0),     # decode, GQA 4, ragged lengths
    (3, 4, 4, 3, 300, 64, [300, 45, 2], True, 3),      # 3 new rows; one cache shorter than them
    (1, 32, 8, 1, 4097, 128, None, False, 7),          # ragged cache end, several splits
    (2, 16, 1, 5, 777, 64, [777, 100], True, 1),       # MQA: 80 rows per group, one split
    (1, 4, 2, 17, 129, 128, [129], True, 0),           # chunked prefill, 34 rows per group
    (2, 4, 2, 1, 64, 64, [0, 64], True, 0),            # an empty cache: o = 0, lse = -inf
    (1, 8, 8, 2, 5000, 128, [4999], False, 40),        # many small splits
    (1, 4, 4, 3, 600, 64, [546], True, 19),            # last split (keys 544, 545) unseen by row 0
    (6, 8, 2, 1, 3000, 128, [3000, 0, 1, 33, 2999, 70], True, 0),   # skewed mix: ranges cross sequences
    (4, 8, 4, 2, 900, 64, [900, 5, 0, 64], True, 13),  # 13 ranges over 969 keys, two new rows
    (3, 4, 2, 1, 50, 128, [50, 1, 2], False, 64),      # more ranges than keys: some ranges empty
    (150, 4, 2, 1, 300, 64, "drawn", True, 0),        # 150 sequences, lengths 0..300: the length scans take three 64-wide steps
    (2, 8, 2, 1, 4000, 128, [4000, 10], False, 200),   # a sequence spanning about 200 ranges: merges past 64
    (5, 8, 2, 40, 2000, 64, [2000, 0, 41, 1500, 7], True, 0),   # 160 rows per group (4 waves); empty and short caches
    (3, 16, 2, 40, 1200, 128, [1200, 300, 77], True, 13),       # 320 rows per group (8 waves); ranges cross sequences
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_kvcache_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, lens, causal, nsplit = case
    q, k, v, drawn = draw_cache(B, H, Hkv, Nq, Nk, d, seed=100 + len(str(case)) + Nk,
                                min_len=0 if lens == "drawn" else None)
    lt = drawn if lens == "drawn" else (None if lens is None else torch.tensor(lens, dtype=torch.int32))
    run_case(q, k, v, lt, causal, d ** -0.5, nsplit)


def random_cache_cases(n=10, seed=2027):
    """(B, H, Hkv, Nq, Nk, d, lens, causal, nsplit): decode (Nq = 1) and
    chunked prefill, lengths 0..Nk, split counts from the default to 40."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 5))
        Nq = 1 if rng.random() < 0.5 else int(rng.integers(2, 41))
        Nk = int(rng.integers(1, 3000))
        lens = [int(x) for x in rng.integers(0, Nk + 1, size=B)]
        nsplit = int(rng.choice([0, 1, 3, 17, 40]))
        cases.append((B, H, Hkv, Nq, Nk, int(rng.choice([64, 128])), lens, bool(rng.integers(0, 2)), nsplit))
    return cases


@pytest.mark.parametrize("case", random_cache_cases(), ids=[str(i) for i in range(10)])
def test_random_kvcache_match_oracle(case):
    test_kvcache_matches_oracle(case)


def nan_past_lengths(t, lens, extra=256):
    """A device copy of cache t [B, Nk, Hkv, d] whose rows at or past each
    sequence's length hold NaN, inside a buffer that continues with NaN rows
    past the last sequence: caches hold stale or unwritten rows there, and any
    use of them (even times a zero weight) shows up as NaN in the output."""
    B, Nk = t.shape[:2]
    flat = torch.full((t.numel() + extra * t[0, 0].numel(),), float("nan"), dtype=t.dtype, device=DEV)
    view = flat[: t.numel()].view(t.shape)
    view.copy_(t.to(DEV))
    for b in range(B):
        view[b, int(lens[b]):] = float("nan")
    return view


@pytest.mark.parametrize("case", [
    (2, 8, 2, 1, 1000, 128, [1000, 517], True, 0),
    (3, 4, 4, 3, 300, 64, [300, 45, 2], True, 3),
    (4, 8, 4, 2, 900, 64, [900, 5, 0, 64], True, 13),
    (3, 16, 2, 40, 1200, 128, [1200, 300, 77], True, 13),
    (2, 8, 2, 1, 4000, 128, [4000, 10], False, 200),
    (1, 32, 8, 1, 4097, 128, [4097], False, 7),
], ids=lambda c: "B%dH%dKV%dNq%dNk%dd%d" % c[:6])
def test_kvcache_rows_past_each_length_are_not_used(case):
    B, H, Hkv, Nq, Nk, d, lens, causal, nsplit = case
    q, k, v, _ = draw_cache(B, H, Hkv, Nq, Nk, d, seed=300 + Nk)
    print("case", case, flush=True)
    kd, vd = nan_past_lengths(k, lens), nan_past_lengths(v, lens)
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = mi.fwd_kvcache(q.to(DEV), kd, vd, ld, causal, d ** -0.5, nsplit)
    torch.cuda.synchronize()
    ro, rl = oracle.forward_kvcache(as_f64(q), as_f64(k), as_f64(v), lens, causal, d ** -0.5)
    eo = check_bf16("o", f64(o), ro)
    el = check_abs("lse", f64(lse), rl, BF16_LSE_ABS)
    print("errors o %.3g lse %.3g" % (eo, el), flush=True)


def test_kvcache_split_count_changes_only_rounding():
    q, k, v, lens = draw_cache(2, 8, 2, 2, 3000, 128, seed=9, min_len=1500)
    qd, kd, vd, ld = (t.to(DEV) for t in (q, k, v, lens))
    o1, l1 = mi.fwd_kvcache(qd, kd, vd, ld, True, 128 ** -0.5, 1)
    o2, l2 = mi.fwd_kvcache(qd, kd, vd, ld, True, 128 ** -0.5, 16)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-4


def test_kvcache_negative_and_zero_scale():
    q, k, v, lens = draw_cache(1, 4, 2, 1, 200, 64, seed=10, min_len=100)
    for sc in (-0.125, 0.0):
        run_case(q, k, v, lens, True, sc, 0)


@pytest.mark.parametrize("name", sorted(CACHE_WORKLOADS))
def test_cache_workload_matches_oracle(name):
    w = CACHE_WORKLOADS[name]
    q, k, v, lens = draw_cache_workload(w)
    if w.Nq > 1:   # prefill: check the first two sequences in full
        q, k, v, lens = q[:2], k[:2], v[:2], lens[:2]
    run_case(q, k, v, lens, True, w.d ** -0.5, 0)


@pytest.mark.slow
def test_prefill16k_full_call_sampled_sequences():
    # the whole workload in one call, as bench.py times it; two of its
    # sequences (the shortest and the last) checked in full against the oracle
    w = CACHE_WORKLOADS["prefill16k"]
    q, k, v, lens = draw_cache_workload(w)
    qd, kd, vd, ld = (t.to(DEV) for t in (q, k, v, lens))
    o, lse = mi.fwd_kvcache(qd, kd, vd, ld, True, w.d ** -0.5, 0)
    torch.cuda.synchronize()
    for b in (1, 3):
        sl = slice(b, b + 1)
        ro, rl = oracle.forward_kvcache(as_f64(q[sl]), as_f64(k[sl]), as_f64(v[sl]), [int(lens[b])],
                                        True, w.d ** -0.5)
        check_bf16("o[b=%d]" % b, f64(o[sl]), ro)
        check_abs("lse[b=%d]" % b, f64(lse[sl]), rl, BF16_LSE_ABS)
        print("sequence", b, "length", int(lens[b]), "ok", flush=True)
