"""GPU parity of packed variable-length batches (attn_fwd_varlen /
attn_bwd_varlen) against the float64 oracle: every output element at small
sizes (ragged lengths, empty and one-row sequences, tails past a tile),
bitwise agreement with the batched entry points where the two describe the
same problem, and sampled rows of the full 16K-token packed workload."""
import numpy as np
import pytest
import torch

import exact_attention_37_amd as mi
import oracle
from workloads import draw_varlen, draw_varlen_workload, VARLEN_WORKLOADS, draw, as_f64
from tests.helpers import check_bf16, check_abs, check_rel, f64, BF16_LSE_ABS, default_scale

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (lengths, H, Hkv, d, causal, window, dtype)
CASES = [
    ([300, 0, 77, 513, 1, 256], 4, 2, 128, True, 0, torch.bfloat16),   # empty and one-row sequences
    ([300, 0, 77, 513, 1, 256], 4, 2, 128, False, 0, torch.bfloat16),
    ([129, 700, 31], 8, 2, 64, True, 0, torch.bfloat16),              # GQA 4, d = 64
    ([1000, 255, 257], 4, 1, 128, True, 100, torch.bfloat16),         # MQA with a sliding window
    ([64] * 9, 2, 2, 64, False, 0, torch.bfloat16),                   # many short sequences
    ([100, 3, 60], 2, 2, 64, True, 0, torch.float32),                 # float32 exactness path
    ([45, 130], 2, 1, 128, False, 0, torch.float32),
]


def run(q, k, v, do, cu, max_len, causal, window, scale):
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    o, lse = mi.fwd_varlen(qd, kd, vd, cud, max_len, causal, scale, window)
    dq, dk, dv = mi.bwd_varlen(qd, kd, vd, o, lse, dod, cud, max_len, causal, scale, window)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_varlen_matches_oracle(case):
    lengths, H, Hkv, d, causal, W, dt = case
    print("case", case, flush=True)
    q, k, v, do, cu = draw_varlen(lengths, H, Hkv, d, seed=300 + sum(lengths), dtype=dt)
    scale = default_scale(d)
    got = run(q, k, v, do, cu, max(lengths), causal, W, scale)
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    ro, rl = oracle.forward_varlen(qq, kk, vv, cu.numpy(), causal, scale, W)
    rg = oracle.backward_varlen(qq, kk, vv, dd, cu.numpy(), causal, scale, W)
    errs = {}
    for name, g, r in zip(("o", "lse", "dq", "dk", "dv"), got, (ro, rl) + rg):
        if dt == torch.float32:
            errs[name] = check_rel(name, f64(g), r)
        elif name == "lse":
            errs[name] = check_abs(name, f64(g), r, BF16_LSE_ABS)
        else:
            errs[name] = check_bf16(name, f64(g), r)
    print("errors", {k_: "%.3g" % v_ for k_, v_ in errs.items()}, flush=True)


def random_varlen_cases(n=10, seed=2026):
    """(lengths, H, Hkv, d, causal, window, dtype) with 1-7 sequences of
    0-450 rows each."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        lengths = [int(x) for x in rng.integers(0, 451, size=int(rng.integers(1, 8)))]
        if sum(lengths) == 0:
            lengths[0] = 1
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(1, 300)) if causal and rng.random() < 0.4 else 0
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        cases.append((lengths, H, Hkv, int(rng.choice([64, 128])), causal, window, dtype))
    return cases


@pytest.mark.parametrize("case", random_varlen_cases(), ids=[str(i) for i in range(10)])
def test_random_varlen_match_oracle(case):
    test_varlen_matches_oracle(case)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_equal_lengths_equal_the_batched_entry_points_bitwise(dt):
    # three sequences of 333 rows packed = a batch of three: the same tiles,
    # the same arithmetic, so the same bits
    B, N, H, Hkv, d = 3, 333, 4, 2, 128
    q, k, v, do = draw(B, H, Hkv, N, d, seed=41, dtype=dt)
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = mi.fwd(qd, kd, vd, True, 0.09)
    g = mi.bwd(qd, kd, vd, o, lse, dod, True, 0.09)
    pk = [t.reshape(B * N, t.shape[2], d) for t in (qd, kd, vd, dod)]
    po, plse = mi.fwd_varlen(pk[0], pk[1], pk[2], cu.to(DEV), N, True, 0.09)
    pg = mi.bwd_varlen(pk[0], pk[1], pk[2], po, plse, pk[3], cu.to(DEV), N, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(po.reshape(o.shape), o)
    assert torch.equal(plse.reshape(H, B, N).permute(1, 0, 2), lse)
    for x, y in zip(pg, g):
        assert torch.equal(x.reshape(y.shape), y)


def test_padding_rows_outside_every_sequence_are_untouched():
    # cu_seqlens ending before total: the trailing rows belong to no sequence
    q, k, v, do, _ = draw_varlen([200, 150], 2, 2, 64, seed=42)
    cu = torch.tensor([0, 120, 180], dtype=torch.int32)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o = torch.full_like(qd, 7.0)
    lse = torch.full((2, 350), 7.0, device=DEV)
    mi.fwd_varlen(qd, kd, vd, cu.to(DEV), 120, True, 0.125, out=o, out_lse=lse)
    dq, dk, dv = (torch.full_like(t, 5.0) for t in (qd, kd, vd))
    mi.bwd_varlen(qd, kd, vd, o, lse, dod, cu.to(DEV), 120, True, 0.125, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(o[180:] == 7.0) and torch.all(lse[:, 180:] == 7.0)
    for t in (dq, dk, dv):
        assert torch.all(t[180:] == 5.0)
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    ro, rl = oracle.forward_varlen(qq, kk, vv, cu.numpy(), True, 0.125)
    check_bf16("o", f64(o[:180]), ro[:180])
    check_abs("lse", f64(lse[:, :180]), rl[:, :180], BF16_LSE_ABS)
    rg = oracle.backward_varlen(qq, kk, vv, dd, cu.numpy(), True, 0.125)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        check_bf16(name, f64(g[:180]), r[:180])


@pytest.mark.parametrize("d", [64, 128])
def test_rows_outside_every_sequence_are_not_read(d):
    # the rows after the last sequence, and a buffer tail past the tensor,
    # hold NaN: a tile that reads any of them, even under a zero weight,
    # brings NaN into the outputs of the sequences
    lengths, cu = [200, 150], torch.tensor([0, 130, 197], dtype=torch.int32)
    q, k, v, do, _ = draw_varlen(lengths, 4, 2, d, seed=43 + d)
    dev = []
    for t in (q, k, v, do):
        flat = torch.full((t.numel() + 256 * t[0].numel(),), float("nan"), dtype=t.dtype, device=DEV)
        x = flat[: t.numel()].view(t.shape)
        x.copy_(t.to(DEV))
        x[197:] = float("nan")
        dev.append(x)
    qd, kd, vd, dod = dev
    o, lse = mi.fwd_varlen(qd, kd, vd, cu.to(DEV), 130, True, 0.1)
    dq, dk, dv = mi.bwd_varlen(qd, kd, vd, o, lse, dod, cu.to(DEV), 130, True, 0.1)
    torch.cuda.synchronize()
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    ro, rl = oracle.forward_varlen(qq, kk, vv, cu.numpy(), True, 0.1)
    check_bf16("o", f64(o[:197]), ro[:197])
    check_abs("lse", f64(lse[:, :197]), rl[:, :197], BF16_LSE_ABS)
    rg = oracle.backward_varlen(qq, kk, vv, dd, cu.numpy(), True, 0.1)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        check_bf16(name, f64(g[:197]), r[:197])


@pytest.mark.slow
def test_packed16k_sampled():
    w = VARLEN_WORKLOADS["packed16k"]
    q, k, v, do, cu = draw_varlen_workload(w)
    print("lengths", (cu[1:] - cu[:-1]).tolist(), flush=True)
    scale = default_scale(w.d)
    lengths = (cu[1:] - cu[:-1]).tolist()
    o, lse, dq, dk, dv = run(q, k, v, do, cu, max(lengths), True, 0, scale)
    G = w.H // w.Hkv
    sampled = {0, 1, len(lengths) - 1}          # the first two sequences and the last (ragged) one
    for s, (a, e) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
        L = e - a
        # any size: per sequence, dK of a head sums to zero and dV sums to the group's dO
        dks, dvs = dk[a:e].double(), dv[a:e].double()
        assert torch.all(dks.sum(0).abs() <= 2.0 ** -7 * dks.abs().sum(0))
        sdo = do[a:e].double().reshape(L, w.Hkv, G, w.d).sum(dim=(0, 2)).to(DEV)
        assert torch.all((dvs.sum(0) - sdo).abs() <= 2.0 ** -7 * dvs.abs().sum(0))
        if s not in sampled:
            continue
        sl = [as_f64(t[a:e])[None] for t in (q, k, v, do)]
        rows = sorted({0, 1, L // 3, L // 2 + 7, L - 2, L - 1})
        for h in (s % w.H, (5 * s + 17) % w.H):
            ro, rl = oracle.forward_rows(*sl[:3], True, scale, 0, h, rows)
            check_bf16("o[s=%d,h=%d]" % (s, h), f64(o[a:e][rows, h]), ro)
            check_abs("lse[s=%d,h=%d]" % (s, h), f64(lse[h, a:e][rows]), rl, BF16_LSE_ABS)
            rq = oracle.backward_dq_rows(*sl, True, scale, 0, h, rows)
            check_bf16("dq[s=%d,h=%d]" % (s, h), f64(dq[a:e][rows, h]), rq)
        gk = (3 * s) % w.Hkv
        rk, rv = oracle.backward_dkdv_rows(*sl, True, scale, 0, gk, rows)
        check_bf16("dk[s=%d,g=%d]" % (s, gk), f64(dk[a:e][rows, gk]), rk)
        check_bf16("dv[s=%d,g=%d]" % (s, gk), f64(dv[a:e][rows, gk]), rv)
        print("sequence", s, "rows", rows, "ok", flush=True)


def test_backward_accumulate_adds_into_float32_gradients():
    q, k, v, do, cu = draw_varlen([300, 77, 513], 4, 2, 128, seed=45)
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    o, lse = mi.fwd_varlen(qd, kd, vd, cud, 513, True, 0.1)
    g = mi.bwd_varlen(qd, kd, vd, o, lse, dod, cud, 513, True, 0.1)
    base = [torch.full(t.shape, 0.25, dtype=torch.float32, device=DEV) for t in (qd, kd, vd)]
    acc = mi.bwd_varlen(qd, kd, vd, o, lse, dod, cud, 513, True, 0.1, accumulate=True,
                        dq=base[0].clone(), dk=base[1].clone(), dv=base[2].clone())
    torch.cuda.synchronize()
    for a, b, x in zip(acc, g, base):
        # the bf16 gradients are the float32 sums rounded once
        check_bf16("accumulated", f64(a - x), f64(b))
