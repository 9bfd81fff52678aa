"""GPU parity of block-sparse attention (attn_fwd_blocksparse /
attn_bwd_blocksparse) against the float64 oracle under the same block mask:
every output element at small sizes (ragged N, GQA/MQA, causal and not,
rows left with no key), bitwise agreement with the dense entry points when
every block is kept, and sampled rows of the 16K workload."""
import numpy as np
import pytest
import torch

import exact_attention_37_amd as mi
import oracle
from workloads import draw, draw_block_mask, draw_workload, WORKLOADS, as_f64
from tests.helpers import check_bf16, check_abs, check_rel, f64, BF16_LSE_ABS, default_scale

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, H, Hkv, N, d, causal, density, keep the diagonal, dtype)
CASES = [
    (1, 4, 2, 700, 128, True, 0.5, True, torch.bfloat16),     # ragged N: tails in every tile size
    (1, 4, 2, 700, 128, False, 0.5, False, torch.bfloat16),
    (2, 8, 2, 1000, 64, True, 0.3, True, torch.bfloat16),     # GQA 4, d = 64
    (1, 4, 1, 1536, 128, True, 0.25, False, torch.bfloat16),  # MQA; rows with no key
    (1, 2, 2, 900, 64, False, 0.2, False, torch.bfloat16),    # non-causal, block rows with no key
    (1, 2, 2, 520, 64, False, 0.6, False, torch.float32),     # float32 exactness path
    (1, 2, 1, 300, 128, True, 0.5, False, torch.float32),
]


def run(q, k, v, do, mask, causal, scale):
    qd, kd, vd, dod, md = (t.to(DEV) for t in (q, k, v, do, mask))
    o, lse = mi.fwd_blocksparse(qd, kd, vd, md, causal, scale)
    dq, dk, dv = mi.bwd_blocksparse(qd, kd, vd, o, lse, dod, md, causal, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_blocksparse_matches_oracle(case):
    B, H, Hkv, N, d, causal, dens, diag, dt = case
    print("case", case, flush=True)
    q, k, v, do = draw(B, H, Hkv, N, d, seed=400 + N, dtype=dt)
    mask = draw_block_mask(N, dens, seed=N, diagonal=diag)
    scale = default_scale(d)
    got = run(q, k, v, do, mask, causal, scale)
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    ro, rl = oracle.forward_blocksparse(qq, kk, vv, mask.numpy(), causal, scale)
    rg = oracle.backward_blocksparse(qq, kk, vv, dd, mask.numpy(), causal, scale)
    print("rows with no key:", int(np.sum(~np.isfinite(rl))), flush=True)
    errs = {}
    for name, g, r in zip(("o", "lse", "dq", "dk", "dv"), got, (ro, rl) + rg):
        if name == "lse":
            errs[name] = check_abs(name, f64(g), r, 1e-5 if dt == torch.float32 else BF16_LSE_ABS)
        elif dt == torch.float32:
            errs[name] = check_rel(name, f64(g), r)
        else:
            errs[name] = check_bf16(name, f64(g), r)
    print("errors", {k_: "%.3g" % v_ for k_, v_ in errs.items()}, flush=True)


def random_block_cases(n=10, seed=2028):
    """(B, H, Hkv, N, d, causal, density, keep the diagonal, dtype)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        cases.append((int(rng.integers(1, 3)), H, Hkv, int(rng.integers(1, 1300)), int(rng.choice([64, 128])),
                      bool(rng.integers(0, 2)), float(rng.choice([0.1, 0.3, 0.6, 0.9])), bool(rng.integers(0, 2)),
                      torch.float32 if rng.random() < 0.25 else torch.bfloat16))
    return cases


@pytest.mark.parametrize("case", random_block_cases(), ids=[str(i) for i in range(10)])
def test_random_blocksparse_match_oracle(case):
    test_blocksparse_matches_oracle(case)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_every_block_kept_equals_dense_bitwise(causal, dt):
    B, H, Hkv, N, d = 1, 4, 2, 777, 128
    q, k, v, do = draw(B, H, Hkv, N, d, seed=43, dtype=dt)
    ones = torch.ones(mi.block_mask_shape(N), dtype=torch.uint8)
    a = run(q, k, v, do, ones, causal, 0.1)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = mi.fwd(qd, kd, vd, causal, 0.1)
    g = mi.bwd(qd, kd, vd, o, lse, dod, causal, 0.1)
    torch.cuda.synchronize()
    for x, y in zip(a, (o, lse) + g):
        assert torch.equal(x, y)


def test_empty_mask_gives_the_merge_identity_and_zero_gradients():
    q, k, v, do = draw(1, 2, 2, 600, 64, seed=44)
    zeros = torch.zeros(mi.block_mask_shape(600), dtype=torch.uint8)
    o, lse, dq, dk, dv = run(q, k, v, do, zeros, True, 0.125)
    assert torch.all(o == 0) and torch.all(lse == float("-inf"))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.slow
def test_llama16k_quarter_density_sampled():
    w = WORKLOADS["llama16k"]
    q, k, v, do = draw_workload(w)
    mask = draw_block_mask(w.N, 0.25, seed=9)
    scale = default_scale(w.d)
    o, lse, dq, dk, dv = run(q, k, v, do, mask, True, scale)
    print("kept blocks", int(mask.sum()), "of", mask.numel(), flush=True)
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    rows = [0, 1, 255, 256, 4097, 8191, 12000, w.N - 2, w.N - 1]
    for h in (0, 17):
        ro, rl, rq = oracle.blocksparse_rows(qq, kk, vv, dd, mask.numpy(), True, scale, 0, h, rows)
        check_bf16("o[h=%d]" % h, f64(o[0, rows, h]), ro)
        check_abs("lse[h=%d]" % h, f64(lse[0, h, rows]), rl, BF16_LSE_ABS)
        check_bf16("dq[h=%d]" % h, f64(dq[0, rows, h]), rq)
        print("head", h, "rows ok", flush=True)
    cols = [0, 127, 128, 5000, 9999, w.N - 1]
    rk, rv = oracle.blocksparse_dkdv_cols(qq, kk, vv, dd, mask.numpy(), True, scale, 0, 5, cols)
    check_bf16("dk[g=5]", f64(dk[0, cols, 5]), rk)
    check_bf16("dv[g=5]", f64(dv[0, cols, 5]), rv)
    # any size: the key gradients of a head sum to zero and the value
    # gradients to the summed dO of the rows that have keys
    dks, dvs = dk[0].double(), dv[0].double()
    assert torch.all(dks.sum(0).abs() <= 2.0 ** -7 * dks.abs().sum(0))
    has_key = torch.isfinite(lse[0]).T.unsqueeze(-1)                    # [N, H, 1]
    sdo = (do[0].double().to(DEV) * has_key).sum(0)
    assert torch.all((dvs.sum(0) - sdo).abs() <= 2.0 ** -7 * dvs.abs().sum(0))


def test_backward_accumulate_adds_into_float32_gradients():
    q, k, v, do = draw(1, 4, 2, 700, 128, seed=46)
    mask = draw_block_mask(700, 0.5, seed=5).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = mi.fwd_blocksparse(qd, kd, vd, mask, True, 0.1)
    g = mi.bwd_blocksparse(qd, kd, vd, o, lse, dod, mask, True, 0.1)
    base = [torch.full(t.shape, -0.5, dtype=torch.float32, device=DEV) for t in (qd, kd, vd)]
    acc = mi.bwd_blocksparse(qd, kd, vd, o, lse, dod, mask, True, 0.1, accumulate=True,
                             dq=base[0].clone(), dk=base[1].clone(), dv=base[2].clone())
    torch.cuda.synchronize()
    for a, b, x in zip(acc, g, base):
        check_bf16("accumulated", f64(a - x), f64(b))
