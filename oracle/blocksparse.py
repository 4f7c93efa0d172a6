"""Block-sparse attention in float64: the definition with a block mask.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the library.

Followed: "FlashAttention技术解析" (mhpq.cn), section 6.2 "稀疏注意力集成":
a boolean block mask of n_blk x n_blk entries says which (query block, key
block) pairs of the score matrix are computed at all; blocks that are off are
skipped. Readings where the page's sketch is silent or garbled:
* query block i takes ONE softmax over the keys of all its enabled key
  blocks (the sketch writes each block pair's result into the output rows of
  block i; read as the usual block-sparse attention, not as the last block
  overwriting the others);
* key j is visible to query i iff mask[i // block, j // block] is set, and,
  with ``causal``, j <= i as well (both masks apply);
* a query row with no visible key has an empty softmax: O = 0, lse = -inf;
* the mask may differ per (batch, query head): shape [B, Hq, n_blk, n_blk],
  or [n_blk, n_blk] shared by all of them; n_blk = ceil(N / block).
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_fwd_blockmask", "element_mask"]


def element_mask(block_mask, N, block, causal):
    """[N, N] boolean visibility of key j (column) to query i (row) from one [n_blk, n_blk] block mask."""
    bm = np.asarray(block_mask).astype(bool)
    n_blk = -(-N // block)
    if bm.shape != (n_blk, n_blk):
        raise ValueError(f"block mask {bm.shape} does not match N={N}, block={block}")
    idx = np.arange(N) // block
    vis = bm[idx[:, None], idx[None, :]]
    if causal:
        vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
    return vis


def attention_fwd_blockmask(q, k, v, block_mask, causal, scale, block=128):
    """(O [B, Hq, N, d], lse [B, Hq, N]) of softmax over the visible keys only, in float64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (query head h reads key/value head
    h // (Hq // Hkv)); block_mask: [n_blk, n_blk] or [B, Hq, n_blk, n_blk].
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    bm = np.asarray(block_mask)
    O = np.zeros((B, Hq, N, d))
    lse = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        for h in range(Hq):
            m_bh = bm if bm.ndim == 2 else bm[b, h]
            vis = element_mask(m_bh, N, block, causal)
            s = np.where(vis, scale * (q[b, h] @ k[b, h // G].T), -np.inf)
            live = vis.any(axis=1)
            if not live.any():
                continue
            sl = s[live]
            m = sl.max(axis=1)
            e = np.exp(sl - m[:, None])
            l = e.sum(axis=1)
            O[b, h, live] = (e / l[:, None]) @ v[b, h // G]
            lse[b, h, live] = m + np.log(l)
    return O, lse
