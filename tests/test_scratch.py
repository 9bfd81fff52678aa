"""The scratch buffer the library keeps per stream: calls that reuse it (after
a larger call, a smaller one, or a call of another kind) give bit for bit
what the same calls give on freshly allocated scratch; calls on two streams
at once each keep their own; attn_release_scratch frees it and leaves the
next call working."""
import pytest
import torch

import exact_attention_37_amd as mi
from workloads import draw, draw_cache

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def calls():
    """Three calls with different scratch needs: a decode step (balanced key
    ranges and their prefix sums), a chunked prefill (per-sequence chunks)
    and a backward pass (the rowsum vector)."""
    dec = [t.to(DEV) for t in draw_cache(3, 8, 2, 1, 700, 128, seed=51, min_len=1)]
    pre = [t.to(DEV) for t in draw_cache(2, 8, 2, 96, 2000, 64, seed=52, min_len=96)]
    q, k, v, do = (t.to(DEV) for t in draw(1, 4, 2, 900, 128, seed=53))
    o, lse = mi.fwd(q, k, v, True, 0.1)
    return {
        "decode": lambda: mi.fwd_kvcache(*dec),
        "prefill": lambda: mi.fwd_kvcache(*pre),
        "bwd": lambda: mi.bwd(q, k, v, o, lse, do, True, 0.1),
    }


def fresh(fn):
    """fn's outputs with no kept buffer: every piece of scratch newly allocated."""
    mi.release_scratch()
    out = [t.clone() for t in fn()]
    mi.release_scratch()
    torch.cuda.synchronize()
    return out


def test_reused_scratch_gives_the_fresh_results_bitwise():
    c = calls()
    ref = {name: fresh(fn) for name, fn in c.items()}
    # grow, shrink and switch kinds on one stream without releasing
    for name in ("decode", "prefill", "decode", "bwd", "decode", "prefill", "bwd"):
        got = c[name]()
        torch.cuda.synchronize()
        for a, b in zip(got, ref[name]):
            assert torch.equal(a, b), name
        print(name, "ok", flush=True)
    mi.release_scratch()


def test_two_streams_keep_their_own_buffers():
    c = calls()
    ref = {name: fresh(fn) for name, fn in c.items()}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            outs.append(("prefill", [t.clone() for t in c["prefill"]()]))
        with torch.cuda.stream(s2):
            outs.append(("decode", [t.clone() for t in c["decode"]()]))
    torch.cuda.synchronize()
    for name, got in outs:
        for a, b in zip(got, ref[name]):
            assert torch.equal(a, b), name
    mi.release_scratch(s1)
    mi.release_scratch(s2)
    torch.cuda.synchronize()


def test_release_without_a_buffer_and_calls_after_release():
    mi.release_scratch()
    mi.release_scratch()            # nothing kept: not an error
    c = calls()
    a = [t.clone() for t in c["decode"]()]
    mi.release_scratch()
    b = c["decode"]()
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    mi.release_scratch()


def test_graph_replays_match_eager_and_survive_buffer_growth():
    # Captured calls take stream-ordered allocations that the graph owns, so
    # a later eager call that grows (and frees) the kept buffer cannot pull
    # memory out from under a replay. Every replay is checked against the
    # eager result, with eager work and synchronisations in between.
    c = calls()
    eager = {name: fresh(c[name]) for name in ("decode", "bwd")}
    mi.release_scratch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture's stream, outside the capture
        c["decode"](); c["bwd"]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec = c["decode"]()
        bw = c["bwd"]()
    for rep in range(4):
        c["prefill"]()                     # eager: grows this stream's kept buffer
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(dec, eager["decode"]):
            assert torch.equal(a, b), "decode, replay %d" % rep
        for a, b in zip(bw, eager["bwd"]):
            assert torch.equal(a, b), "bwd, replay %d" % rep
        print("replay", rep, "ok", flush=True)
    mi.release_scratch()
    mi.release_scratch(side)
    torch.cuda.synchronize()
