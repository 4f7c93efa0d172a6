"""The tiled online-softmax recurrence, in float64, in its two published forms.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the library.

Both functions walk the keys in blocks, keeping for every query row a running
maximum m and a running sum l of exponentials, and rescale what was gathered so
far by exp(m_old - m_new) whenever the maximum grows. They are written from:

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


def online_fwd_normalise_each_block(q, k, v, causal, scale, block_q, block_k):
    """First form: the output is kept normalised after every key block.

    O <- (l / l_new) e^(m - m_new) O + (e^(m_blk - m_new) / l_new) (p_blk V_blk).
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
            o = np.zeros((len(rows), d))
            for j0 in range(0, N, block_k):
                keys = np.arange(j0, min(j0 + block_k, N))
                m_blk, p, l_blk = _block_stats(q_rows, kh[keys], scale, causal, rows, keys)
                m_new = np.maximum(m, m_blk)
                keep = _safe_exp_diff(m, m_new)
                gain = _safe_exp_diff(m_blk, m_new)
                l_new = keep * l + gain * l_blk
                seen = l_new > 0
                inv = np.where(seen, 1.0 / np.where(seen, l_new, 1.0), 0.0)
                o = (l * keep * inv)[:, None] * o + (gain * inv)[:, None] * (p @ vh[keys])
                m, l = m_new, l_new
            O[b, h, rows] = o
            lse[b, h, rows] = m + np.log(l)
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
