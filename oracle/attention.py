"""Plain, slow, float64 CPU oracle for exact attention -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this module. The GPU library never calls it, and it
shares no code with the GPU library: it takes numpy arrays and uses numpy
only (a matmul is the one library primitive it leans on).

What is computed (the pages state the operation, not its formulas; the
readings taken are listed next to each function):

* the result is exact attention softmax(Q K^T) V -- "FlashAttention" abstract
  page (exact, not approximate attention) and the DistFlashAttn reviews page,
  review 1 summary, which writes the operation out;
* the per-row logsumexp is the saved statistic -- FlashAttention-2 reviews
  page, reviewer 2 summary, point 2 (save logsumexp instead of max and sum);
* a causal mask halves the work -- DistFlashAttn reviews page, review 1
  summary, point 1; FlashAttention-2 reviews page, reviewer 4 (block skipping
  for causal masking, section 3.1);
* grouped-query attention shares one K/V head among several query heads --
  FlashAttention-2 reviews page, reviewer 1 (the MQA/GQA paragraph of the
  backward-pass section); DistFlashAttn reviews page, review 3 (GQA setting);
* partial results over key chunks are combined -- DistFlashAttn reviews page,
  reviews 1 and 4 (chunks of the attention computation spread over workers);
  BurstAttention rebuttal page (RingAttention vs. online softmax);
* local (sliding-window) attention is the same method with a banded mask --
  FlashAttention-2 reviews page, the authors' general response (local
  attention used to train Mistral-7B); BurstAttention rebuttal page (sparse
  attention only changes the attention mask);
* a batch may pack sequences of different lengths back to back --
  FlashAttention-2 reviews page, reviewer 2's questions (training batches
  whose tokens carry no explicit sequence dimension);
* block-sparse attention computes only the blocks a block mask keeps --
  FlashAttention abstract page (the extension to block-sparse attention, an
  approximation of dense attention); FlashAttention-2 reviews page, reviewer
  3's question on sparse block masks; BurstAttention rebuttal page (sparsity
  is a change of the attention mask).

Readings where the pages are silent (each also listed in the design notes):
scores are scale * Q K^T with a caller-given scale; causal keeps key position
<= query position (absolute positions, so a chunk pair can be masked by its
offsets); LSE is the natural-log logsumexp of the scaled, masked scores;
head h reads K/V head h // (H / Hkv); layouts are Q,O,dO [B, N, H, d],
K,V [B, N, Hkv, d], LSE [B, H, N]; the backward is the gradient of
sum(dO * O) with respect to Q, K, V.

Every function here is pinned in tests/test_oracle.py against things other
than its own formula: hand-worked values (tests/golden), closed forms,
invariants, finite differences and torch's float64 CPU attention.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores", "forward", "backward", "merge", "tiled_forward",
    "forward_rows", "backward_dq_rows", "backward_dkdv_rows", "probs",
    "forward_kvcache", "forward_varlen", "backward_varlen",
    "block_allowed", "forward_blocksparse", "backward_blocksparse",
    "blocksparse_rows", "blocksparse_dkdv_cols",
]


# ---------------------------------------------------------------------------
# the definition, one (batch, query head) at a time
# ---------------------------------------------------------------------------

def scores(q_h, k_g, scale, causal, q_pos=None, k_pos=None, window=0):
    """S[i, j] = scale * q_i . k_j, and -inf where a causal mask forbids j.

    q_h: [Nq, d], k_g: [Nk, d] float64. Positions default to 0..N-1; key j is
    allowed for query i iff k_pos[j] <= q_pos[i] under the causal mask, and,
    with a sliding window of ``window`` > 0 keys (local attention, causal
    only), also iff k_pos[j] > q_pos[i] - window.
    """
    s = scale * (q_h @ k_g.T)
    if causal:
        if q_pos is None:
            q_pos = np.arange(q_h.shape[0])
        if k_pos is None:
            k_pos = np.arange(k_g.shape[0])
        allowed = k_pos[None, :] <= q_pos[:, None]
        if window > 0:
            allowed &= k_pos[None, :] > q_pos[:, None] - window
        s = np.where(allowed, s, -np.inf)
    return s


def _softmax_rows(s):
    """Exact two-pass softmax of each row: returns (P, lse).

    lse = m + ln(sum_j exp(s_j - m)) with m the row max; P = exp(s - lse).
    A row with every entry -inf gets P = 0 and lse = -inf.
    """
    m = np.max(s, axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    tot = np.sum(e, axis=1)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(tot)
    lse = np.where(tot > 0, lse, -np.inf)
    p = np.where(tot[:, None] > 0, e / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return p, lse


def probs(q, k, scale, causal, b=0, h=0):
    """The full attention matrix P of one (batch, query head): [Nq, Nk]."""
    G = q.shape[2] // k.shape[2]
    s = scores(np.asarray(q[b, :, h], np.float64),
               np.asarray(k[b, :, h // G], np.float64), scale, causal)
    return _softmax_rows(s)[0]


def _check(q, k, v):
    B, N, H, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d or H % Hkv:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))
    return B, N, H, Hkv, d, Nk


def _row_blocks(n, blk):
    for r0 in range(0, n, blk):
        yield r0, min(n, r0 + blk)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def forward(q, k, v, causal, scale, q_offset=0, k_offset=0, row_block=512, window=0):
    """O and LSE of exact attention (``window`` > 0: causal sliding window of
    that many keys, see ``scores``).

    q: [B, Nq, H, d]; k, v: [B, Nk, Hkv, d] (any float dtype, used as float64).
    Returns o [B, Nq, H, d] float64 and lse [B, H, Nq] float64.

    Query rows are processed in blocks; each block's score rows are
    materialised at full key width and normalised exactly (max, then sum), so
    no online rescaling is involved. ``q_offset``/``k_offset`` are the absolute
    positions of row 0 of q and of k, used only by the causal mask.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, Hkv, d, Nk = _check(q, k, v)
    G = H // Hkv
    o = np.zeros((B, Nq, H, d))
    lse = np.zeros((B, H, Nq))
    k_pos = k_offset + np.arange(Nk)
    for b in range(B):
        for h in range(H):
            g = h // G
            for r0, r1 in _row_blocks(Nq, row_block):
                q_pos = q_offset + np.arange(r0, r1)
                s = scores(q[b, r0:r1, h], k[b, :, g], scale, causal, q_pos, k_pos, window)
                p, l = _softmax_rows(s)
                o[b, r0:r1, h] = p @ v[b, :, g]
                lse[b, h, r0:r1] = l
    return o, lse


def forward_kvcache(q, k, v, k_lens, causal, scale):
    """O and LSE of Nq new query rows against a key/value cache.

    Inference use of the method (FlashAttention-2 reviews page, reviewer 2,
    strengths; reviewer 3, point 3). q: [B, Nq, H, d]; k, v: [B, Nk, Hkv, d];
    k_lens: the number of valid cache rows of each batch entry (None: Nk),
    clamped to [0, Nk]. Batch entry b attends to cache rows [0, L_b) only.
    Reading where the pages are silent: the new rows are the last Nq
    positions of the sequence, so under the causal mask query row i sits at
    position L_b - Nq + i and sees cache rows j <= that position. A row that
    sees no key gets o = 0 and lse = -inf. Returns o [B, Nq, H, d] and
    lse [B, H, Nq], float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = Nk if k_lens is None else int(min(max(int(k_lens[b]), 0), Nk))
        if L == 0:
            continue
        ob, lb = forward(q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L], causal, scale, q_offset=L - Nq)
        o[b] = ob[0]
        lse[b] = lb[0]
    return o, lse


def _sequences(cu_seqlens, total):
    """(start, end) row ranges of a packed batch, each clamped to [0, total]."""
    cu = [int(x) for x in cu_seqlens]
    out = []
    for s in range(len(cu) - 1):
        e = min(max(cu[s + 1], 0), total)
        a = min(max(cu[s], 0), e)
        out.append((a, e))
    return out


def forward_varlen(q, k, v, cu_seqlens, causal, scale, window=0):
    """O and LSE of a packed batch of sequences of different lengths.

    q: [total, H, d]; k, v: [total, Hkv, d]; sequence s owns rows
    [cu_seqlens[s], cu_seqlens[s + 1]). Reading where the pages are silent
    (the reviewer asks what happens without sequence boundaries): the
    boundaries are given, and each sequence is its own attention problem --
    its queries see only its own keys, the causal mask and the window use
    positions counted from its first row. Rows outside every sequence are
    left at o = 0, lse = -inf. Returns o [total, H, d] and lse [H, total],
    float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    total, H, d = q.shape
    o = np.zeros((total, H, d))
    lse = np.full((H, total), -np.inf)
    for a, e in _sequences(cu_seqlens, total):
        if e == a:
            continue
        ob, lb = forward(q[None, a:e], k[None, a:e], v[None, a:e], causal, scale, window=window)
        o[a:e] = ob[0]
        lse[:, a:e] = lb[0]
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, causal, scale, window=0):
    """dQ, dK, dV of ``forward_varlen``: each sequence's gradients are those of
    its own attention problem (``backward``); rows outside every sequence get
    zero. Returns float64 arrays shaped like q, k, v."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, e in _sequences(cu_seqlens, q.shape[0]):
        if e == a:
            continue
        g = backward(q[None, a:e], k[None, a:e], v[None, a:e], do[None, a:e], causal, scale, window=window)
        dq[a:e], dk[a:e], dv[a:e] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# block-sparse attention
# ---------------------------------------------------------------------------
#
# Reading where the pages are silent: the block mask has one entry per block
# of bq query rows x bk keys (the library fixes bq = 256, bk = 128); a zero
# entry removes every (query, key) pair of its block, on top of the causal
# mask. The result is exact attention under that mask (and an approximation
# of dense attention, which is the pages' point). A query row left with no
# key gets o = 0 and lse = -inf (the merge identity) and zero gradients.

def block_allowed(block_mask, Nq, Nk, bq=256, bk=128):
    """allowed[i, j] = block_mask[i // bq, j // bk] != 0, for i < Nq, j < Nk."""
    bm = np.asarray(block_mask) != 0
    return bm[np.arange(Nq)[:, None] // bq, np.arange(Nk)[None, :] // bk]


def _masked_scores(q_h, k_g, scale, causal, allowed):
    return np.where(allowed, scores(q_h, k_g, scale, causal), -np.inf)


def forward_blocksparse(q, k, v, block_mask, causal, scale, bq=256, bk=128):
    """O [B, N, H, d] and LSE [B, H, N] (float64) of attention under a block
    mask (see above), one (batch, head) at a time."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, N, H, Hkv, d, Nk = _check(q, k, v)
    G = H // Hkv
    allowed = block_allowed(block_mask, N, Nk, bq, bk)
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            p, l = _softmax_rows(_masked_scores(q[b, :, h], k[b, :, h // G], scale, causal, allowed))
            o[b, :, h] = p @ v[b, :, h // G]
            lse[b, h] = l
    return o, lse


def backward_blocksparse(q, k, v, do, block_mask, causal, scale, bq=256, bk=128):
    """dQ, dK, dV of ``forward_blocksparse``: the gradient formulas of
    ``backward`` with P taken under the block mask (float64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, N, H, Hkv, d, Nk = _check(q, k, v)
    G = H // Hkv
    allowed = block_allowed(block_mask, N, Nk, bq, bk)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // G
            p, _ = _softmax_rows(_masked_scores(q[b, :, h], k[b, :, g], scale, causal, allowed))
            dv[b, :, g] += p.T @ do[b, :, h]
            dp = do[b, :, h] @ v[b, :, g].T
            ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
            dq[b, :, h] = scale * (ds @ k[b, :, g])
            dk[b, :, g] += scale * (ds.T @ q[b, :, h])
    return dq, dk, dv


def blocksparse_rows(q, k, v, do, block_mask, causal, scale, b, h, rows, bq=256, bk=128):
    """O, LSE and dQ of selected query rows of one (batch, head) under a block
    mask; every quantity of a query row depends on that row alone, so long
    sequences can be checked by sampling."""
    G = q.shape[2] // k.shape[2]
    kg = np.asarray(k[b, :, h // G], np.float64)
    vg = np.asarray(v[b, :, h // G], np.float64)
    rows = np.asarray(rows)
    qh = np.asarray(q[b, rows, h], np.float64)
    doh = np.asarray(do[b, rows, h], np.float64)
    bm = np.asarray(block_mask) != 0
    allowed = bm[rows[:, None] // bq, np.arange(kg.shape[0])[None, :] // bk]
    s = scale * (qh @ kg.T)
    if causal:
        allowed = allowed & (np.arange(kg.shape[0])[None, :] <= rows[:, None])
    p, lse = _softmax_rows(np.where(allowed, s, -np.inf))
    dp = doh @ vg.T
    ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
    return p @ vg, lse, scale * (ds @ kg)


def blocksparse_dkdv_cols(q, k, v, do, block_mask, causal, scale, b, g, cols, bq=256, bk=128, row_block=512):
    """dK and dV of selected key rows of K/V head g under a block mask, summed
    over the query heads of the group. Each query row's LSE is computed over
    all its keys (row blocks at a time); P and dS are then taken for the
    selected keys only."""
    H, Hkv = q.shape[2], k.shape[2]
    G = H // Hkv
    kg = np.asarray(k[b, :, g], np.float64)
    vg = np.asarray(v[b, :, g], np.float64)
    cols = np.asarray(cols)
    N, Nk = q.shape[1], kg.shape[0]
    bm = np.asarray(block_mask) != 0
    dk = np.zeros((len(cols), kg.shape[1]))
    dv = np.zeros((len(cols), kg.shape[1]))
    for h in range(g * G, (g + 1) * G):
        for r0, r1 in _row_blocks(N, row_block):
            ri = np.arange(r0, r1)
            qh = np.asarray(q[b, r0:r1, h], np.float64)
            doh = np.asarray(do[b, r0:r1, h], np.float64)
            allowed = bm[ri[:, None] // bq, np.arange(Nk)[None, :] // bk]
            if causal:
                allowed = allowed & (np.arange(Nk)[None, :] <= ri[:, None])
            p, _ = _softmax_rows(np.where(allowed, scale * (qh @ kg.T), -np.inf))
            dp = doh @ vg.T
            rowdot = np.sum(p * dp, axis=1)
            pc = p[:, cols]
            dsc = pc * (dp[:, cols] - rowdot[:, None])
            dv += pc.T @ doh
            dk += scale * (dsc.T @ qh)
    return dk, dv


def forward_rows(q, k, v, causal, scale, b, h, rows):
    """O[b, rows, h] and LSE[b, h, rows] for selected query rows only.

    The same definition as ``forward``, evaluated one row at a time so it can
    check sampled outputs of very long sequences.
    """
    G = q.shape[2] // k.shape[2]
    g = h // G
    kg = np.asarray(k[b, :, g], np.float64)
    vg = np.asarray(v[b, :, g], np.float64)
    rows = np.asarray(rows)
    out_o = np.zeros((len(rows), q.shape[3]))
    out_l = np.zeros(len(rows))
    for t, i in enumerate(rows):
        n_allowed = (i + 1) if causal else kg.shape[0]
        s = scale * (kg[:n_allowed] @ np.asarray(q[b, i, h], np.float64))
        p, l = _softmax_rows(s[None, :])
        out_o[t] = p[0] @ vg[:n_allowed]
        out_l[t] = l[0]
    return out_o, out_l


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def backward(q, k, v, do, causal, scale, row_block=512, window=0):
    """dQ, dK, dV: gradients of sum(dO * O) through exact attention
    (``window`` > 0: causal sliding window of that many keys).

    With P the softmax of the masked scaled scores (recomputed exactly here):
      dV_j  = sum_i P_ij dO_i
      dP_ij = dO_i . V_j
      dS_ij = P_ij (dP_ij - sum_l P_il dP_il)
      dQ_i  = scale * sum_j dS_ij K_j
      dK_j  = scale * sum_i dS_ij Q_i
    dK and dV of a K/V head are summed over the query heads that read it.
    Returns float64 arrays shaped like q, k, v.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, N, H, Hkv, d, Nk = _check(q, k, v)
    G = H // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // G
            for r0, r1 in _row_blocks(N, row_block):
                s = scores(q[b, r0:r1, h], k[b, :, g], scale, causal,
                           np.arange(r0, r1), np.arange(Nk), window)
                p, _ = _softmax_rows(s)
                dob = do[b, r0:r1, h]
                dv[b, :, g] += p.T @ dob
                dp = dob @ v[b, :, g].T
                rowdot = np.sum(p * dp, axis=1)
                ds = p * (dp - rowdot[:, None])
                dq[b, r0:r1, h] = scale * (ds @ k[b, :, g])
                dk[b, :, g] += scale * (ds.T @ q[b, r0:r1, h])
    return dq, dk, dv


def _lse_rows_from(qh, kg, scale, causal, row_lo, row_block=512):
    """Logsumexp of query rows [row_lo, Nq) (entries below row_lo are unused)."""
    n = qh.shape[0]
    out = np.zeros(n)
    for r0, r1 in _row_blocks(n - row_lo, row_block):
        r0, r1 = r0 + row_lo, r1 + row_lo
        hi = r1 if causal else kg.shape[0]
        s = scores(qh[r0:r1], kg[:hi], scale, causal, np.arange(r0, r1), np.arange(hi))
        out[r0:r1] = _softmax_rows(s)[1]
    return out


def backward_dq_rows(q, k, v, do, causal, scale, b, h, rows):
    """dQ[b, rows, h] for selected query rows (the same definition as
    ``backward``, one row at a time)."""
    G = q.shape[2] // k.shape[2]
    g = h // G
    kg = np.asarray(k[b, :, g], np.float64)
    vg = np.asarray(v[b, :, g], np.float64)
    out = np.zeros((len(rows), q.shape[3]))
    for t, i in enumerate(np.asarray(rows)):
        n_allowed = (i + 1) if causal else kg.shape[0]
        s = scale * (kg[:n_allowed] @ np.asarray(q[b, i, h], np.float64))
        p, _ = _softmax_rows(s[None, :])
        p = p[0]
        dp = vg[:n_allowed] @ np.asarray(do[b, i, h], np.float64)
        ds = p * (dp - np.dot(p, dp))
        out[t] = scale * (ds @ kg[:n_allowed])
    return out


def backward_dkdv_rows(q, k, v, do, causal, scale, b, g, cols, row_block=512):
    """dK[b, cols, g] and dV[b, cols, g] for selected key rows of K/V head g,
    summed over the query heads of its group.

    A key row's gradient needs P[i, j] for every query i that sees it, so each
    query head's row logsumexps are computed first (exactly, at full key
    width). Under the causal mask only queries i >= min(cols) see any of the
    selected keys; rows above that contribute exactly zero and are skipped."""
    H, Hkv = q.shape[2], k.shape[2]
    G = H // Hkv
    kg = np.asarray(k[b, :, g], np.float64)
    vg = np.asarray(v[b, :, g], np.float64)
    cols = np.asarray(cols)
    N = q.shape[1]
    dk = np.zeros((len(cols), q.shape[3]))
    dv = np.zeros((len(cols), q.shape[3]))
    row_lo = int(np.min(cols)) if causal else 0
    for h in range(g * G, (g + 1) * G):
        qh = np.asarray(q[b, :, h], np.float64)
        doh = np.asarray(do[b, :, h], np.float64)
        lse = _lse_rows_from(qh, kg, scale, causal, row_lo)
        for r0, r1 in _row_blocks(N - row_lo, row_block):
            r0, r1 = r0 + row_lo, r1 + row_lo
            # P[i, cols] and dP[i, cols] for this block of queries
            s = scores(qh[r0:r1], kg[cols], scale, causal, np.arange(r0, r1), cols)
            p = np.exp(s - lse[r0:r1, None])
            dp = doh[r0:r1] @ vg[cols].T
            # D_i = sum_j P_ij dP_ij over all keys of row i (full width)
            hi = r1 if causal else kg.shape[0]
            s_full = scores(qh[r0:r1], kg[:hi], scale, causal, np.arange(r0, r1), np.arange(hi))
            p_full = np.exp(s_full - lse[r0:r1, None])
            dp_full = doh[r0:r1] @ vg[:hi].T
            rowdot = np.sum(p_full * dp_full, axis=1)
            ds = p * (dp - rowdot[:, None])
            dv += p.T @ doh[r0:r1]
            dk += scale * (ds.T @ qh[r0:r1])
    return dk, dv


# ---------------------------------------------------------------------------
# merge of partial results over disjoint key sets
# ---------------------------------------------------------------------------

def merge(o_a, lse_a, o_b, lse_b):
    """Combine attention over key set A and over a disjoint key set B into
    attention over A u B.

    Softmax over a union: the new normaliser is e^{lse_a} + e^{lse_b}, so
      lse = M + ln(e^{lse_a - M} + e^{lse_b - M}),  M = max(lse_a, lse_b)
      o   = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b
    Rows where both sides are empty (lse = -inf) give lse = -inf, o = 0.
    o_*: [B, N, H, d]; lse_*: [B, H, N].
    """
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    tot = np.exp(lse_a - m_safe) + np.exp(lse_b - m_safe)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    lse_fin = np.where(np.isfinite(lse), lse, 0.0)
    wa = np.where(np.isfinite(lse), np.exp(lse_a - lse_fin), 0.0)
    wb = np.where(np.isfinite(lse), np.exp(lse_b - lse_fin), 0.0)
    # [B, H, N] weights -> [B, N, H, 1]
    wa = np.transpose(wa, (0, 2, 1))[..., None]
    wb = np.transpose(wb, (0, 2, 1))[..., None]
    return wa * o_a + wb * o_b, lse


# ---------------------------------------------------------------------------
# the tiled online-softmax algorithm (to pin that it equals the definition)
# ---------------------------------------------------------------------------

def tiled_forward(q, k, v, causal, scale, br, bc):
    """FlashAttention's tiled forward with online softmax, in float64.

    For each block of ``br`` query rows, keys are visited ``bc`` at a time
    with a running row max m, an un-normalised running sum l and an
    un-normalised accumulator; when the max grows both are rescaled by
    e^{m_old - m_new}, and the division by l happens once at the end
    (FlashAttention-2 reviews page, reviewer 2, point 1: deferred scaling;
    point 2: the saved statistic is m + ln l). Key tiles lying entirely
    above the diagonal are skipped under a causal mask.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, N, H, Hkv, d, Nk = _check(q, k, v)
    G = H // Hkv
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // G
            for r0, r1 in _row_blocks(N, br):
                m = np.full(r1 - r0, -np.inf)
                l = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, d))
                for c0, c1 in _row_blocks(Nk, bc):
                    if causal and c0 > r1 - 1:
                        break  # every key of this tile is after every query row
                    s = scores(q[b, r0:r1, h], k[b, c0:c1, g], scale, causal,
                               np.arange(r0, r1), np.arange(c0, c1))
                    m_new = np.maximum(m, np.max(s, axis=1))
                    m_use = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.exp(m - m_use)       # e^{-inf} = 0 on the first tile
                    p = np.exp(s - m_use[:, None])
                    l = alpha * l + np.sum(p, axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, c0:c1, g]
                    m = m_new
                o[b, r0:r1, h] = acc / l[:, None]
                lse[b, h, r0:r1] = m + np.log(l)
    return o, lse
