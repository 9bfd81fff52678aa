"""GPU parity of causal sliding-window attention (attn_fwd_window /
attn_bwd_window) against the float64 oracle with the same window, element by
element over O, LSE, dQ, dK, dV."""
import numpy as np
import pytest
import torch

import exact_attention_37_amd as mi
import oracle
from workloads import draw, as_f64
from tests.helpers import check_bf16, check_abs, check_rel, f64, BF16_LSE_ABS

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, H, Hkv, N, d, window, dtype)
CASES = [
    (1, 4, 2, 300, 64, 1, torch.bfloat16),        # each row sees only itself
    (1, 4, 4, 520, 128, 17, torch.bfloat16),      # window smaller than a tile
    (2, 8, 2, 1000, 128, 100, torch.bfloat16),    # GQA 4, window across tile edges
    (1, 2, 2, 700, 64, 256, torch.bfloat16),      # window = one workgroup of query rows
    (1, 4, 1, 777, 128, 255, torch.bfloat16),     # MQA, ragged N
    (1, 2, 2, 200, 64, 1000, torch.bfloat16),     # window past N = causal
    (1, 4, 2, 4096, 128, 1024, torch.bfloat16),   # long sequence, many skipped tiles
    (1, 2, 2, 128, 64, 33, torch.float32),        # float32 exactness path
    (1, 2, 1, 300, 128, 70, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_window_matches_oracle(case):
    B, H, Hkv, N, d, W, dt = case
    print("case", case, flush=True)
    q, k, v, do = draw(B, H, Hkv, N, d, seed=200 + N + W, dtype=dt)
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = mi.fwd(qd, kd, vd, True, scale, window=W)
    dq, dk, dv = mi.bwd(qd, kd, vd, o, lse, dod, True, scale, window=W)
    torch.cuda.synchronize()
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    ro, rl = oracle.forward(qq, kk, vv, True, scale, window=W)
    rdq, rdk, rdv = oracle.backward(qq, kk, vv, dd, True, scale, window=W)
    errs = {}
    for name, g, r in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), (ro, rl, rdq, rdk, rdv)):
        if dt == torch.float32:
            errs[name] = check_rel(name, f64(g), r)
        elif name == "lse":
            errs[name] = check_abs(name, f64(g), r, BF16_LSE_ABS)
        else:
            errs[name] = check_bf16(name, f64(g), r)
    print("errors", {k_: "%.3g" % v_ for k_, v_ in errs.items()}, flush=True)


def test_window_past_the_sequence_equals_causal_bitwise():
    q, k, v, do = draw(1, 4, 2, 600, 128, seed=31, dtype=torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    a = mi.fwd(qd, kd, vd, True, 0.1, window=600)
    b = mi.fwd(qd, kd, vd, True, 0.1)
    ga = mi.bwd(qd, kd, vd, a[0], a[1], dod, True, 0.1, window=5000)
    gb = mi.bwd(qd, kd, vd, b[0], b[1], dod, True, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)
