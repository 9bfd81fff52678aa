"""Writes tests/golden/gqa64k_dkdv_cols.npz: the float64 oracle's dK and dV of
the gqa64k workload (B=1, H=32, Hkv=8, N=65536, d=128, bf16 inputs, causal,
seed 5) at sampled key rows of K/V heads 0 and 7.

The sampled keys sit in chunks 5, 6 and 7 of the workload's 8-chunk split,
so the chunked backward sums their gradients over 3, 2 and 1 chunk pairs
(DistFlashAttn reviews page, review 1 point 3 and review 4: the attention
work of a long sequence is cut into chunks whose partial results are
combined). A key row's gradient needs every query row at or after it, which
takes minutes of float64 work per K/V head, so the values are stored here
instead of being recomputed on every test run.

Only the oracle computes the values; the inputs come from the seeded
generator in workloads.py, and a SHA-1 of their bf16 bytes is stored beside
them so that the test can confirm it draws the same inputs.

    python tests/golden/make_gqa64k_dkdv.py      (about 5 minutes on 8 cores)
"""
import hashlib
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import WORKLOADS, draw_workload, as_f64  # noqa: E402

OUT = os.path.join(HERE, "gqa64k_dkdv_cols.npz")
KV_HEADS = (0, 7)


def sample_cols(N):
    # chunk 5 (3 pairs), chunk 6 (2 pairs), chunk 7 (1 pair), chunk rows 8192
    return np.array([N - 24576, N - 20481, N - 16385, N - 16384, N - 12289, N - 8193, N - 8192, N - 1])


def inputs_sha1(tensors):
    h = hashlib.sha1()
    for t in tensors:
        h.update(t.contiguous().view(-1).view(dtype=__import__("torch").int16).numpy().tobytes())
    return h.hexdigest()


def main():
    w = WORKLOADS["gqa64k"]
    t0 = time.time()
    q, k, v, do = draw_workload(w)
    sha = inputs_sha1((q, k, v, do))
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    del q, k, v, do
    scale = w.d ** -0.5
    cols = sample_cols(w.N)
    G = w.H // w.Hkv

    # one query head per task: the oracle on that head alone (its K/V head as
    # the only one) gives the head's share of the group's key gradients
    def head_share(task):
        g, h = task
        return oracle.backward_dkdv_rows(qq[:, :, h:h + 1], kk[:, :, g:g + 1], vv[:, :, g:g + 1],
                                         dd[:, :, h:h + 1], True, scale, 0, 0, cols)

    tasks = [(g, h) for g in KV_HEADS for h in range(g * G, (g + 1) * G)]
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=len(tasks)) as ex:
        shares = list(ex.map(head_share, tasks))
    dk = np.zeros((len(KV_HEADS), len(cols), w.d))
    dv = np.zeros_like(dk)
    for (g, _), (sk, sv) in zip(tasks, shares):
        dk[KV_HEADS.index(g)] += sk
        dv[KV_HEADS.index(g)] += sv
    np.savez(OUT, dk=dk, dv=dv, cols=cols, kv_heads=np.array(KV_HEADS), seed=np.array(w.seed),
             inputs_sha1=np.array(sha))
    print("wrote %s in %.0f s" % (OUT, time.time() - t0))


if __name__ == "__main__":
    main()
