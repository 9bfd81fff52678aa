"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch them.

Each mutation swaps one oracle internal for a wrong variant; the pins of
test_oracle.py are then re-run and at least one must fail.
"""
import numpy as np
import pytest

import oracle.attention as A
import tests.test_oracle as T


def _pins():
    cases = T.load_golden()
    yield lambda: [T.test_hand_worked_forward_backward(c) for c in cases]
    yield lambda: T.test_causal_row0_returns_v0()
    yield lambda: T.test_matches_torch_float64_attention(True, 4, 2)
    yield lambda: T.test_matches_torch_float64_attention(False, 4, 2)
    yield lambda: T.test_lse_matches_scipy_logsumexp(False, 1000.0)
    yield lambda: T.test_backward_identities(True)
    yield lambda: T.test_merge_of_two_key_chunks_equals_full(True)
    yield lambda: T.test_tiled_online_softmax_equals_naive(True, 13, 7)
    yield lambda: T.test_kvcache_matches_elementwise_loops(True)
    yield lambda: T.test_kvcache_ignores_rows_past_the_valid_length()
    yield lambda: T.test_window_matches_elementwise_loops(3)
    yield lambda: T.test_varlen_matches_elementwise_loops(True, 0)
    yield lambda: T.test_varlen_matches_torch_block_diagonal_attention(True, 0)
    yield lambda: T.test_blocksparse_matches_elementwise_loops(True)
    yield lambda: T.test_blocksparse_matches_torch_masked_attention(False)
    yield lambda: T.test_blocksparse_equals_attention_over_the_kept_keys()


def _caught():
    for pin in _pins():
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            return True
    return False


def _no_scale(q_h, k_g, scale, causal, q_pos=None, k_pos=None, window=0):
    return _orig_scores(q_h, k_g, 1.0, causal, q_pos, k_pos, window)


def _flipped_causal(q_h, k_g, scale, causal, q_pos=None, k_pos=None, window=0):
    s = scale * (q_h @ k_g.T)
    if causal:
        q_pos = np.arange(q_h.shape[0]) if q_pos is None else q_pos
        k_pos = np.arange(k_g.shape[0]) if k_pos is None else k_pos
        s = np.where(k_pos[None, :] >= q_pos[:, None], s, -np.inf)
    return s


def _window_off_by_one(q_h, k_g, scale, causal, q_pos=None, k_pos=None, window=0):
    return _orig_scores(q_h, k_g, scale, causal, q_pos, k_pos, window + 1 if window > 0 else 0)


def _lse_without_max(s):
    p, lse = _orig_softmax(s)
    m = np.max(s, axis=1)
    return p, lse - np.where(np.isfinite(m), m, 0.0)


def _softmax_no_max_subtraction(s):
    e = np.exp(s)
    tot = e.sum(axis=1)
    return e / tot[:, None], np.log(tot)


def _merge_swapped_weights(o_a, lse_a, o_b, lse_b):
    return _orig_merge(o_b, lse_a, o_a, lse_b)


def _kvcache_top_left(q, k, v, k_lens, causal, scale):
    # new rows aligned to the start of the cache instead of its end
    q = np.asarray(q, np.float64)
    B, Nq = q.shape[:2]
    o = np.zeros(q.shape)
    lse = np.full((B, q.shape[2], Nq), -np.inf)
    for b in range(B):
        L = k.shape[1] if k_lens is None else int(k_lens[b])
        ob, lb = A.forward(q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L], causal, scale, q_offset=0)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def _kvcache_whole_cache(q, k, v, k_lens, causal, scale):
    # valid lengths ignored: every cache row attended to
    return _orig_kvcache(q, k, v, None, causal, scale)


def _varlen_one_sequence(q, k, v, cu_seqlens, causal, scale, window=0):
    # sequence boundaries ignored: the pack attended to as one sequence
    return _orig_varlen(q, k, v, [0, np.asarray(q).shape[0]], causal, scale, window)


def _varlen_backward_one_sequence(q, k, v, do, cu_seqlens, causal, scale, window=0):
    return _orig_varlen_bwd(q, k, v, do, [0, np.asarray(q).shape[0]], causal, scale, window)


def _varlen_offset_by_one(q, k, v, cu_seqlens, causal, scale, window=0):
    # each boundary taken one row late
    cu = [min(int(c) + 1, np.asarray(q).shape[0]) for c in cu_seqlens]
    cu[0] = 0
    return _orig_varlen(q, k, v, cu, causal, scale, window)


def _block_allowed_transposed(block_mask, Nq, Nk, bq=256, bk=128):
    # block mask indexed [key block, query block]
    bm = np.asarray(block_mask) != 0
    r = np.minimum(np.arange(Nq)[:, None] // bq, bm.shape[1] - 1)
    c = np.minimum(np.arange(Nk)[None, :] // bk, bm.shape[0] - 1)
    return bm[c, r]


def _block_allowed_sizes_swapped(block_mask, Nq, Nk, bq=256, bk=128):
    bm = np.asarray(block_mask) != 0
    r = np.minimum(np.arange(Nq)[:, None] // bk, bm.shape[0] - 1)
    c = np.minimum(np.arange(Nk)[None, :] // bq, bm.shape[1] - 1)
    return bm[r, c]


_orig_scores = A.scores
_orig_varlen = A.forward_varlen
_orig_varlen_bwd = A.backward_varlen
_orig_kvcache = A.forward_kvcache
_orig_softmax = A._softmax_rows
_orig_merge = A.merge

MUTATIONS = {
    "dropped_scale": ("scores", _no_scale),
    "causal_mask_reversed": ("scores", _flipped_causal),
    "lse_missing_max": ("_softmax_rows", _lse_without_max),
    "no_max_subtraction": ("_softmax_rows", _softmax_no_max_subtraction),
    "merge_weights_swapped": ("merge", _merge_swapped_weights),
    "kvcache_top_left_alignment": ("forward_kvcache", _kvcache_top_left),
    "window_off_by_one": ("scores", _window_off_by_one),
    "kvcache_lengths_ignored": ("forward_kvcache", _kvcache_whole_cache),
    "varlen_boundaries_ignored": ("forward_varlen", _varlen_one_sequence),
    "varlen_backward_boundaries_ignored": ("backward_varlen", _varlen_backward_one_sequence),
    "varlen_boundaries_off_by_one": ("forward_varlen", _varlen_offset_by_one),
    "block_mask_transposed": ("block_allowed", _block_allowed_transposed),
    "block_sizes_swapped": ("block_allowed", _block_allowed_sizes_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(A, attr, fn)
    if attr in ("merge", "forward_kvcache", "forward_varlen", "backward_varlen", "block_allowed"):
        # re-exported by the package
        import oracle
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(), "planted mistake %r passed every pin" % name


def _mutated_backward(kind):
    """A copy of the oracle's backward with one planted mistake."""
    def backward(q, k, v, do, causal, scale, row_block=512):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        do = np.asarray(do, np.float64)
        B, N, H, Hkv, d, Nk = A._check(q, k, v)
        G = H // Hkv
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                g = (h % Hkv) if kind == "head_map_modulo" else h // G
                s = A.scores(q[b, :, h], k[b, :, g], scale, causal)
                p, _ = A._softmax_rows(s)
                dv[b, :, g] += p.T @ do[b, :, h]
                dp = do[b, :, h] @ v[b, :, g].T
                rowdot = np.sum(p * dp, axis=1)
                ds = p * (dp + rowdot[:, None]) if kind == "ds_sign" else p * (dp - rowdot[:, None])
                kk = v[b, :, g] if kind == "dq_uses_v" else k[b, :, g]
                dq[b, :, h] = scale * (ds @ kk)
                sc = 1.0 if kind == "dk_missing_scale" else scale
                dk[b, :, g] += sc * (ds.T @ q[b, :, h])
        return dq, dk, dv
    return backward


@pytest.mark.parametrize("kind", ["ds_sign", "dq_uses_v", "dk_missing_scale", "head_map_modulo"])
def test_pins_catch_planted_backward_mistake(kind, monkeypatch):
    import oracle
    fn = _mutated_backward(kind)
    monkeypatch.setattr(A, "backward", fn)
    monkeypatch.setattr(oracle, "backward", fn)
    monkeypatch.setattr(T.oracle, "backward", fn)
    assert _caught(), "planted backward mistake %r passed every pin" % kind
