"""Materialised float64 attention: the plain definition and its gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the library.

Definition followed: the attention formula of the page "FlashAttention v2相比于v1
有哪些更新" (blogweb.cn), section 1 "FlashAttention v1":
    Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V,
with the softmax taken over keys (per query row). Here the factor 1/sqrt(d_k)
is an explicit ``scale`` argument, applied to q.k before the softmax.

Readings where the pages are silent:
* causal mask: key j is visible to query i iff j <= i (queries and keys share
  one index range, mask anchored top-left). Row i always sees key 0.
* the value kept for the backward pass is the row logsumexp of the scaled,
  masked scores in the natural log: lse_i = m_i + ln(l_i) (the page
  "4.3 FlashAttention-2与FlashAttention-3演进", FlashAttention-3 section 3
  "反向传播优化", says only the softmax normalisation factor is stored).
* grouped heads: query head h reads key/value head h // (Hq // Hkv).
* gradients: the pages give no formulas; these follow from differentiating
  the definition (softmax Jacobian), with D_i = sum_c dO_ic O_ic.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "attention_fwd",
    "attention_fwd_rows",
    "attention_probs",
    "attention_bwd",
    "attention_bwd_head",
    "causal_tile_count",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    return B, Hq, Hkv, N, d


def _masked_scores(q_rows, k_head, scale, causal, row_index):
    """Scaled scores scale * q_rows @ k_head^T, with -inf where key j > query i (causal)."""
    s = scale * (q_rows @ k_head.T)
    if causal:
        keys = np.arange(k_head.shape[0])
        s = np.where(keys[None, :] > np.asarray(row_index)[:, None], -np.inf, s)
    return s


def _softmax_parts(s):
    """Row max m, exponentials e = exp(s - m), row sum l (every row has a finite entry)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return m, e, l


def attention_probs(q, k, causal, scale):
    """Softmax probabilities P [B, Hq, N, N] (float64); the definition's softmax(...)."""
    q, k = _f64(q), _f64(k)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    P = np.zeros((B, Hq, N, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            s = _masked_scores(q[b, h], k[b, h // G], scale, causal, rows)
            _, e, l = _softmax_parts(s)
            P[b, h] = e / l[:, None]
    return P


def attention_fwd(q, k, v, causal, scale):
    """O = softmax(scale * q k^T [+ mask]) v and lse, per (batch, query head), in float64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]. Returns (O [B, Hq, N, d], lse [B, Hq, N]).
    The whole N x N score matrix of one head is materialised.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    G = Hq // Hkv
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    if N == 0:  # no queries: empty outputs
        return O, lse
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            s = _masked_scores(q[b, h], k[b, h // G], scale, causal, rows)
            m, e, l = _softmax_parts(s)
            O[b, h] = (e / l[:, None]) @ v[b, h // G]
            lse[b, h] = m + np.log(l)
    return O, lse


def attention_fwd_rows(q, k, v, causal, scale, b, h, rows):
    """The definition evaluated for selected query rows of one (batch, query head).

    Used to check full-size outputs on a sample of rows. Returns (O_rows [R, d], lse_rows [R]).
    """
    Hq, Hkv = np.shape(q)[1], np.shape(k)[1]
    G = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    q_rows = _f64(q[b, h][rows])
    k_head = _f64(k[b, h // G])
    v_head = _f64(v[b, h // G])
    s = _masked_scores(q_rows, k_head, scale, causal, rows)
    m, e, l = _softmax_parts(s)
    return (e / l[:, None]) @ v_head, m + np.log(l)


def attention_bwd(q, k, v, dO, causal, scale):
    """Gradients (dQ, dK, dV) of sum(dO * O) for O = attention_fwd(q, k, v, causal, scale)[0].

    Per (b, h), with P the softmax probabilities:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
        dS = P * (dP - D[:, None]),  dQ = scale * dS K,  dK = scale * dS^T Q.
    Grouped heads: the dK, dV of a key/value head sum over the query heads that read it.
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    if dO.shape != q.shape:
        raise ValueError("dO must have q's shape")
    G = Hq // Hkv
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    if N == 0:
        return dQ, dK, dV
    for b in range(B):
        for h in range(Hq):
            gq, gk, gv = attention_bwd_head(q[b, h], k[b, h // G], v[b, h // G], dO[b, h], causal, scale)
            dQ[b, h] = gq
            dK[b, h // G] += gk
            dV[b, h // G] += gv
    return dQ, dK, dV


def attention_bwd_head(q, k, v, dO, causal, scale):
    """Gradients for one head: q, dO [N, d] and k, v [N, d]; returns (dQ, dK, dV) in float64."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    N = q.shape[0]
    s = _masked_scores(q, k, scale, causal, np.arange(N))
    _, e, l = _softmax_parts(s)
    P = e / l[:, None]
    O = P @ v
    dV = P.T @ dO
    dP = dO @ v.T
    D = np.sum(dO * O, axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV


def causal_tile_count(N, BM, BN):
    """Number of (query tile, key tile) pairs of an N x N causal problem that hold a visible entry.

    A BM x BN tile (queries i0..i0+BM-1, keys j0..j0+BN-1) holds a visible entry iff
    j0 <= min(i0 + BM, N) - 1. Counted by brute force over tiles (the page
    "Flash Attention V3技术解析", section 2.1, says tiles entirely above the diagonal
    are skipped).
    """
    count = 0
    for i0 in range(0, N, BM):
        last_q = min(i0 + BM, N) - 1
        for j0 in range(0, N, BN):
            if j0 <= last_q:
                count += 1
    return count
