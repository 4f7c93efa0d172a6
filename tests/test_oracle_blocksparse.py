"""Pins of the block-sparse oracle (CPU only): dense limit, independent blocks,
brute force, empty rows, per-head masks. See oracle/blocksparse.py for the
passage followed ("FlashAttention技术解析" (mhpq.cn), section 6.2)."""
import math

import numpy as np
import pytest

from oracle import attention_fwd, attention_fwd_blockmask, element_mask


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,block", [(37, 8), (64, 16), (5, 128)])
def test_all_blocks_on_is_the_dense_definition(causal, N, block):
    q, k, v = _rand((2, 4, N, 8), 1), _rand((2, 2, N, 8), 2), _rand((2, 2, N, 8), 3)
    n_blk = -(-N // block)
    O, L = attention_fwd_blockmask(q, k, v, np.ones((n_blk, n_blk), bool), causal, 0.4, block)
    Od, Ld = attention_fwd(q, k, v, causal, 0.4)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Ld, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_independent_subsequences(causal):
    # query block i sees only key block i: each block is an attention problem of its own
    N, block, d = 45, 16, 6  # blocks of 16, 16 and a ragged 13
    q, k, v = _rand((1, 3, N, d), 4), _rand((1, 3, N, d), 5), _rand((1, 3, N, d), 6)
    n_blk = 3
    O, L = attention_fwd_blockmask(q, k, v, np.eye(n_blk, dtype=bool), causal, 0.3, block)
    for i in range(n_blk):
        r = slice(i * block, min(N, (i + 1) * block))
        Oi, Li = attention_fwd(q[:, :, r], k[:, :, r], v[:, :, r], causal, 0.3)
        np.testing.assert_allclose(O[:, :, r], Oi, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[:, :, r], Li, rtol=0, atol=1e-12)


def _brute(q, k, v, bm, causal, scale, block):
    """Pure-Python loops: for each query row, a softmax over the visible keys."""
    N, d = len(q), len(q[0])
    O = [[0.0] * d for _ in range(N)]
    lse = [-math.inf] * N
    for i in range(N):
        keys = [j for j in range(N) if bm[i // block][j // block] and (not causal or j <= i)]
        if not keys:
            continue
        s = {j: scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in keys}
        l = sum(w.values())
        for c in range(d):
            O[i][c] = sum(w[j] * v[j][c] for j in keys) / l
        lse[i] = m + math.log(l)
    return O, lse


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_with_an_asymmetric_mask_and_an_empty_row_block(causal):
    N, d, block = 7, 3, 2
    # row block 0 sees key blocks 1, 3 only; row block 2 sees nothing; not symmetric
    bm = np.array([[0, 1, 0, 1], [1, 1, 0, 0], [0, 0, 0, 0], [1, 0, 1, 1]], dtype=bool)
    q, k, v = _rand((N, d), 7), _rand((N, d), 8), _rand((N, d), 9)
    O, L = attention_fwd_blockmask(q[None, None], k[None, None], v[None, None], bm, causal, 0.7, block)
    Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), bm.tolist(), causal, 0.7, block)
    np.testing.assert_allclose(O[0, 0], np.array(Ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[0, 0], np.array(Lb), rtol=0, atol=1e-13)
    # rows 4, 5 (row block 2) see nothing: O = 0, lse = -inf
    assert np.all(O[0, 0, 4:6] == 0) and np.all(np.isneginf(L[0, 0, 4:6]))
    if causal:
        # rows 0, 1 see key blocks 1 and 3 only, all above the diagonal
        assert np.all(O[0, 0, 0:2] == 0) and np.all(np.isneginf(L[0, 0, 0:2]))


def test_visible_counts_closed_form():
    N, block = 50, 16  # block sizes 16, 16, 16, 2
    sizes = [16, 16, 16, 2]
    bm = np.array([[1, 0, 1, 1], [0, 1, 0, 0], [1, 1, 1, 0], [0, 0, 0, 1]], dtype=bool)
    vis = element_mask(bm, N, block, causal=False)
    assert vis.sum() == sum(sizes[i] * sizes[j] for i in range(4) for j in range(4) if bm[i, j])
    full = element_mask(np.ones((4, 4), bool), N, block, causal=True)
    assert full.sum() == N * (N + 1) // 2


def test_per_head_masks_equal_per_head_calls():
    B, Hq, Hkv, N, d, block = 2, 4, 2, 33, 5, 8
    n_blk = 5
    rng = np.random.default_rng(10)
    bm = rng.random((B, Hq, n_blk, n_blk)) < 0.5
    q, k, v = _rand((B, Hq, N, d), 11), _rand((B, Hkv, N, d), 12), _rand((B, Hkv, N, d), 13)
    O, L = attention_fwd_blockmask(q, k, v, bm, True, 0.5, block)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            Oh, Lh = attention_fwd_blockmask(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                                             v[b:b + 1, h // G:h // G + 1], bm[b, h], True, 0.5, block)
            np.testing.assert_array_equal(O[b, h], Oh[0, 0])
            np.testing.assert_array_equal(L[b, h], Lh[0, 0])
