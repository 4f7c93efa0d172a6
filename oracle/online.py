"""The tiled online-softmax recurrence, in float64, in its two published forms.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the library.

Both functions walk the keys in blocks and, for every query row, carry what the
blocks seen so far give: the deferred form a running maximum m, a running sum l
of exponentials and an unnormalised output, rescaled by exp(m_old - m_new)
whenever the maximum grows; the normalised form the output itself with its
logsumexp (m + ln l as one number), merged with each block's own normalised
result. They are written from:

* the page "FlashAttention技术解析：优化Transformer注意力机制" (mhpq.cn),
  section 2.1 (tiled pseudo-code, code operators lost in extraction and
  restored by reading) and section 2.2 (online softmax: m_new = max(m, m_j),
  l <- e^(m - m_new) l + e^(m_j - m_new) l_j, history rescaled by e^(m - m_new));
* the page "FlashAttention v2相比于v1有哪些更新" (blogweb.cn), section 3,
  "Rescale操作": only the numerator is rescaled per block and the division by
  the sum happens once after the loop.

Reading of the garbled pseudo-code: S_ij = Q_i K_j^T * scale; per row of the
block, m_ij = max_j S_ij, p_ij = exp(S_ij - m_ij), l_ij = sum_j p_ij; the block
indices run i : i + block. One m and one l per query row.

The first block a row meets may be fully masked (causal), giving m_ij = -inf;
such a block contributes nothing, and exp(-inf - (-inf)) is taken as 0.
"""
from __future__ import annotations

import numpy as np

__all__ = ["online_fwd_normalise_each_block", "online_fwd_deferred"]


def _block_stats(q_rows, k_blk, scale, causal, row_ids, key_ids):
    s = scale * (q_rows @ k_blk.T)
    if causal:
        s = np.where(key_ids[None, :] > row_ids[:, None], -np.inf, s)
    m_blk = s.max(axis=1)
    finite = np.isfinite(m_blk)
    p = np.where(finite[:, None], np.exp(s - np.where(finite, m_blk, 0.0)[:, None]), 0.0)
    return m_blk, p, p.sum(axis=1)


def _safe_exp_diff(a, b):
    """exp(a - b) with exp(-inf - (-inf)) defined as 0 (both sides still empty)."""
    both_empty = np.isneginf(a) & np.isneginf(b)
    return np.where(both_empty, 0.0, np.exp(np.where(both_empty, 0.0, a - b)))


def _heads(q, k, v):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    for b in range(B):
        for h in range(Hq):
            yield b, h, q[b, h], k[b, h // G], v[b, h // G]


def _block_softmax(q_rows, k_blk, v_blk, scale, causal, row_ids, key_ids):
    """One key block on its own: its normalised output softmax_blk(s) V_blk and its logsumexp.

    A row with no visible key in the block gets output 0 and logsumexp -inf.
    """
    m_blk, p, l_blk = _block_stats(q_rows, k_blk, scale, causal, row_ids, key_ids)
    seen = l_blk > 0
    o_blk = np.where(seen[:, None], (p @ v_blk) / np.where(seen, l_blk, 1.0)[:, None], 0.0)
    return o_blk, np.where(seen, m_blk + np.log(np.where(seen, l_blk, 1.0)), -np.inf)


def online_fwd_normalise_each_block(q, k, v, causal, scale, block_q, block_k):
    """First form: the running output stays normalised after every key block.

    Written as a merge of normalised partial results. With lse = m + ln l the
    running maximum and sum of section 2.2 become one number per row, and the
    update O <- (l / l_new) e^(m - m_new) O + (e^(m_blk - m_new) / l_new) p_blk V_blk
    is O <- e^(lse - lse_new) O + e^(lse_blk - lse_new) O_blk with
    lse_new = log(e^lse + e^lse_blk) and O_blk the block's own normalised output.
    Returns (O, lse) like ``attention_fwd``.
    """
    B, Hq, N, d = np.shape(q)
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for b, h, qh, kh, vh in _heads(q, k, v):
        for i0 in range(0, N, block_q):
            rows = np.arange(i0, min(i0 + block_q, N))
            run_o = np.zeros((len(rows), d))
            run_lse = np.full(len(rows), -np.inf)
            for j0 in range(0, N, block_k):
                keys = np.arange(j0, min(j0 + block_k, N))
                o_blk, lse_blk = _block_softmax(qh[rows], kh[keys], vh[keys], scale, causal, rows, keys)
                new_lse = np.logaddexp(run_lse, lse_blk)
                w_run = _safe_exp_diff(run_lse, new_lse)
                w_blk = _safe_exp_diff(lse_blk, new_lse)
                run_o = w_run[:, None] * run_o + w_blk[:, None] * o_blk
                run_lse = new_lse
            O[b, h, rows] = run_o
            lse[b, h, rows] = run_lse
    return O, lse


def online_fwd_deferred(q, k, v, causal, scale, block_q, block_k):
    """Second form: an unnormalised accumulator, divided by l once after the last block.

    acc <- e^(m - m_new) acc + e^(m_blk - m_new) (p_blk V_blk);  O = acc / l.
    Returns (O, lse) like ``attention_fwd``.
    """
    B, Hq, N, d = np.shape(q)
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for b, h, qh, kh, vh in _heads(q, k, v):
        for i0 in range(0, N, block_q):
            rows = np.arange(i0, min(i0 + block_q, N))
            q_rows = qh[rows]
            m = np.full(len(rows), -np.inf)
            l = np.zeros(len(rows))
            acc = np.zeros((len(rows), d))
            for j0 in range(0, N, block_k):
                keys = np.arange(j0, min(j0 + block_k, N))
                m_blk, p, l_blk = _block_stats(q_rows, kh[keys], scale, causal, rows, keys)
                m_new = np.maximum(m, m_blk)
                keep = _safe_exp_diff(m, m_new)
                gain = _safe_exp_diff(m_blk, m_new)
                acc = keep[:, None] * acc + gain[:, None] * (p @ vh[keys])
                l = keep * l + gain * l_blk
                m = m_new
            O[b, h, rows] = acc / l[:, None]
            lse[b, h, rows] = m + np.log(l)
    return O, lse
