"""attn_bwd_noalloc (the backward for callers that cannot allocate) against
attn_bwd through the C ABI: the same kernels with the rowsum vector in the
library's fixed device array instead of its scratch buffer, so the gradients
must be bitwise equal. Two calls in a row on one device, the second smaller
(the array keeps the first call's contents), in bf16 and fp32."""
import pytest
import torch

import exact_attention_37_amd as mi
from workloads import draw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_pair(B, H, Hkv, N, d, causal, dtype, accumulate, seed):
    q, k, v, do = (t.to(DEV) for t in draw(B, H, Hkv, N, d, seed=seed, dtype=dtype))
    scale = d ** -0.5
    o, lse = mi.fwd(q, k, v, causal, scale)
    ref = mi.bwd(q, k, v, o, lse, do, causal, scale, accumulate=accumulate)
    gdt = torch.float32 if accumulate else dtype
    outs = [torch.full(t.shape, float("nan"), dtype=gdt, device=DEV) if not accumulate else
            torch.zeros(t.shape, dtype=gdt, device=DEV) for t in (q, k, v)]
    got = mi.bwd_noalloc(q, k, v, o, lse, do, causal, scale, *outs, accumulate=accumulate)
    torch.cuda.synchronize()
    print("noalloc B%dH%dKV%dN%dd%d causal=%d %s acc=%d" % (B, H, Hkv, N, d, causal, dtype, accumulate), flush=True)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_noalloc_backward_equals_attn_bwd_twice_second_smaller(dtype):
    run_pair(2, 8, 2, 1000, 128, True, dtype, False, seed=61)
    run_pair(1, 4, 4, 300, 64, False, dtype, False, seed=62)


def test_noalloc_backward_accumulate_and_full_size():
    run_pair(1, 32, 32, 16384, 128, True, torch.bfloat16, False, seed=63)    # 524288 rows of D
    run_pair(1, 4, 1, 520, 128, True, torch.bfloat16, True, seed=64)


def test_noalloc_refuses_oversized_rowsum():
    q = torch.zeros((1, 16, 64, 64), dtype=torch.bfloat16, device=DEV)   # B*H*N = 16 * 64 * ... below
    L = mi.lib()
    # 1 x 70000 rows x 64 heads: 4480000 > 4194304 rows; refused before any launch
    import ctypes
    vp = ctypes.c_void_p
    p = vp(q.data_ptr())
    st = L.attn_bwd_noalloc(p, p, p, p, p, 1, 64, 64, 70000, 64, 1, 0.125, None, p, p, p, p, 1, 0)
    assert st == 1 and b"exceeds the fixed scratch" in L.attn_last_error()
