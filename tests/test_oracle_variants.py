"""Pins of the oracle's attention variants (grouped/single KV heads, sliding
window, block mask), on the CPU.

The variants are those of "TileLang programming model and FlashMLA",
section 5.1. Each test ties
``oracle.attention_masked`` to something other than itself: closed forms on
identical keys, the plain ``oracle.attention`` (itself pinned against a
50-digit brute force and torch's float64 attention), and the exact
split/combine identity over key ranges (``attention_partial`` and
``combine_partials``, pinned in tests/test_oracle.py).
"""

import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, H, Hkv, Sq, Skv, D, seed):
    return _rand((B, H, Sq, D), seed), _rand((B, Hkv, Skv, D), seed + 1), _rand((B, Hkv, Skv, D), seed + 2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_no_window_no_mask_is_plain_attention(causal, Hkv):
    q, k, v = _qkv(2, 4, Hkv, 9, 13, 5, 10)
    o, l = oracle.attention_masked(q, k, v, 0.4, causal=causal)
    ro, rl = oracle.attention(q, k, v, 0.4, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_single_kv_head_is_every_head_reading_it():
    # multi-query: one KV head shared by all query heads
    q, k, v = _qkv(1, 3, 1, 6, 7, 4, 20)
    o, l = oracle.attention_masked(q, k, v, 0.5, causal=True, window=3)
    for h in range(3):
        oh, lh = oracle.attention_masked(q[:, h:h + 1], k, v, 0.5, causal=True, window=3)
        np.testing.assert_allclose(o[:, h:h + 1], oh, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l[:, h:h + 1], lh, rtol=0, atol=1e-14)


@pytest.mark.parametrize("Sq,Skv", [(8, 8), (5, 11)])
def test_window_two_closed_form(Sq, Skv):
    # identical keys: each visible key has the same score, so O is the mean of
    # the visible V rows and LSE = score + ln(count). With W = 2 row i sees
    # the keys pos - 2 .. pos + 1 (pos = i + Skv - Sq) that lie in [0, Skv);
    # causal drops pos + 1.
    D = 4
    q = _rand((1, 1, Sq, D), 30)
    k = np.tile(_rand((1, 1, 1, D), 31), (1, 1, Skv, 1))
    v = _rand((1, 1, Skv, D), 32)
    scale = 0.7
    for causal in (False, True):
        o, l = oracle.attention_masked(q, k, v, scale, causal=causal, window=2)
        for i in range(Sq):
            pos = i + Skv - Sq
            cand = (pos - 2, pos - 1, pos) if causal else (pos - 2, pos - 1, pos, pos + 1)
            keys = [j for j in cand if 0 <= j < Skv]
            sc = scale * float(q[0, 0, i] @ k[0, 0, 0])
            if not keys:
                assert np.all(o[0, 0, i] == 0) and l[0, 0, i] == -np.inf
                continue
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, keys].mean(axis=0), rtol=0, atol=1e-14)
            np.testing.assert_allclose(l[0, 0, i], sc + np.log(len(keys)), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [1, 3, 6])
def test_window_is_attention_over_the_window_range(causal, W):
    # row i's result equals the partial over the key range [pos - W, pos + W)
    Sq, Skv = 11, 14
    q, k, v = _qkv(1, 2, 1, Sq, Skv, 5, 40)
    o, l = oracle.attention_masked(q, k, v, 0.3, causal=causal, window=W)
    for i in range(Sq):
        pos = i + Skv - Sq
        lo, hi = max(0, pos - W), min(Skv, pos + W)
        po, pl = oracle.attention_partial(q, k, v, 0.3, lo, hi, causal=causal)
        np.testing.assert_allclose(o[:, :, i], po[:, :, i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[:, :, i], pl[:, :, i], rtol=0, atol=1e-13)


def test_window_wider_than_everything_is_dense():
    q, k, v = _qkv(1, 2, 2, 7, 9, 3, 50)
    for causal in (False, True):
        o, l = oracle.attention_masked(q, k, v, 0.6, causal=causal, window=100)
        ro, rl = oracle.attention(q, k, v, 0.6, causal=causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_block_mask_all_ones_and_all_zeros():
    q, k, v = _qkv(1, 2, 2, 10, 12, 3, 60)
    blk = 4
    ones = np.ones((1, 2, 3, 3), np.uint8)
    o, l = oracle.attention_masked(q, k, v, 0.5, block_mask=ones, block=blk)
    ro, rl = oracle.attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)
    o, l = oracle.attention_masked(q, k, v, 0.5, block_mask=0 * ones, block=blk)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_block_mask_one_block_per_row_is_that_range():
    # query block r computes only key block (2r + 1) % 4: a non-symmetric
    # pattern, so swapping the query and key block index would show
    Sq, Skv, blk = 12, 16, 4
    q, k, v = _qkv(1, 1, 1, Sq, Skv, 3, 70)
    mask = np.zeros((1, 1, 3, 4), np.uint8)
    for r in range(3):
        mask[0, 0, r, (2 * r + 1) % 4] = 1
    o, l = oracle.attention_masked(q, k, v, 0.8, block_mask=mask, block=blk)
    for i in range(Sq):
        kb = (2 * (i // blk) + 1) % 4
        po, pl = oracle.attention_partial(q, k, v, 0.8, kb * blk, (kb + 1) * blk)
        np.testing.assert_allclose(o[0, 0, i], po[0, 0, i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[0, 0, i], pl[0, 0, i], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_random_block_mask_is_combine_of_active_blocks(causal):
    # with window and causal rule on top: the merge of per-key-block
    # partials over the row's active blocks gives the row's result
    Sq, Skv, blk, W = 13, 17, 4, 5
    q, k, v = _qkv(1, 2, 1, Sq, Skv, 3, 80)
    rng = np.random.default_rng(81)
    nqb, nkb = -(-Sq // blk), -(-Skv // blk)
    mask = (rng.random((1, 2, nqb, nkb)) < 0.5).astype(np.uint8)
    o, l = oracle.attention_masked(q, k, v, 0.45, causal=causal, window=W, block_mask=mask, block=blk)
    for h in range(2):
        for i in range(Sq):
            pos = i + Skv - Sq
            parts_o, parts_l = [], []
            for kb in range(nkb):
                if not mask[0, h, i // blk, kb]:
                    continue
                lo, hi = max(kb * blk, pos - W), min((kb + 1) * blk, pos + W, Skv)
                if hi <= lo:
                    continue
                po, pl = oracle.attention_partial(q[:, h:h + 1], k, v, 0.45, lo, hi, causal=causal)
                parts_o.append(po[0, 0, i])
                parts_l.append(pl[0, 0, i])
            if not parts_o:
                assert np.all(o[0, h, i] == 0) and l[0, h, i] == -np.inf
                continue
            co, cl = oracle.combine_partials(np.stack(parts_o), np.stack(parts_l))
            np.testing.assert_allclose(o[0, h, i], co, rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[0, h, i], cl, rtol=0, atol=1e-13)
