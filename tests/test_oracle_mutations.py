"""Plant plausible mistakes in the CPU oracle and check that its pins catch them.

Runs on the CPU only. Each case patches one piece of the oracle (an
off-by-one causal bound, a base-2 log-sum-exp, a softmax without its row max,
a dropped rotary term, a transposed product) and asserts that at least one of
the listed pin tests then fails.
"""

import numpy as np
import pytest

import oracle
import oracle.core as oa
import tests.test_oracle as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_off_by_one_causal_is_caught(monkeypatch):
    real = oa._allowed_count
    monkeypatch.setattr(oa, "_allowed_count",
                        lambda i, Sq, Skv, causal: real(i, Sq, Skv, causal) - (1 if causal else 0))
    assert _fails(pins.test_causal_closed_form)
    assert _fails(pins.test_causal_row0_is_v0)


def test_base2_lse_is_caught(monkeypatch):
    def finish(p, m, l, v):
        o, lse = real(p, m, l, v)
        return o, m + np.log2(np.where(l == 0, 1.0, l))
    real = oa._finish
    monkeypatch.setattr(oa, "_finish", finish)
    assert _fails(pins.test_two_keys_closed_form)
    assert _fails(pins.test_identical_keys_give_mean_v)


def test_wrong_sign_in_exponent_is_caught(monkeypatch):
    def softmax_rows(s, counts):
        return real(-s, counts)
    real = oa._softmax_rows
    monkeypatch.setattr(oa, "_softmax_rows", softmax_rows)
    assert _fails(pins.test_two_keys_closed_form)
    assert _fails(pins.test_decimal_brute_force, False)


def test_dropped_rotary_term_is_caught(monkeypatch):
    real = oracle.mla_decode
    monkeypatch.setattr(oracle, "mla_decode",
                        lambda q, q_pe, kv, k_pe, indptr, scale, batches=None:
                        real(q, 0 * np.asarray(q_pe, dtype=np.float64), kv, k_pe, indptr, scale, batches))
    assert _fails(pins.test_mla_equals_mha_on_concatenated_keys)


def test_transposed_scores_are_caught(monkeypatch):
    # Softmax taken over the query axis (scores transposed) instead of the key axis.
    real = oracle.attention

    def attention(q, k, v, scale, causal=False, rows=None, row_group=1024):
        if np.shape(q)[2] == np.shape(k)[2]:
            q, k = k, q
        return real(q, k, v, scale, causal, rows, row_group)
    monkeypatch.setattr(oracle, "attention", attention)
    assert _fails(pins.test_against_torch_sdpa_float64, True, 40, 40)


@pytest.mark.parametrize("drop", [True])
def test_missing_rescale_in_online_is_caught(monkeypatch, drop):
    # An online recurrence that forgets to rescale the accumulator by
    # exp(m_prev - m_new) must disagree with the two-pass definition.
    real_exp = np.exp

    def online(q, k, v, scale, causal=False, block=64):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, Sq, _ = q.shape
        out = np.zeros((B, H, Sq, v.shape[3]))
        lse = np.zeros((B, H, Sq))
        for b in range(B):
            for h in range(H):
                m = np.full(Sq, -np.inf)
                l = np.zeros(Sq)
                acc = np.zeros((Sq, v.shape[3]))
                for j0 in range(0, k.shape[2], block):
                    s = scale * (q[b, h] @ k[b, h, j0:j0 + block].T)
                    m_new = np.maximum(m, s.max(axis=1))
                    p = real_exp(s - m_new[:, None])
                    l = l * real_exp(m - m_new) + p.sum(axis=1)
                    acc = acc + p @ v[b, h, j0:j0 + block]   # rescale forgotten
                    m = m_new
                out[b, h] = acc / l[:, None]
                lse[b, h] = m + np.log(l)
        return out, lse
    monkeypatch.setattr(oracle, "online_attention", online)
    assert _fails(pins.test_online_matches_two_pass, 7, False)


def _patch_visible(monkeypatch, fn):
    monkeypatch.setattr(oa, "visible_keys", fn)


def test_window_upper_bound_off_by_one_is_caught(monkeypatch):
    import tests.test_oracle_variants as vpins
    real = oa.visible_keys

    def vis(i, Sq, Skv, causal=False, window=0, block_row=None, block=64):
        out = real(i, Sq, Skv, causal, window, block_row, block)
        pos = i + Skv - Sq
        if window > 0 and not causal and 0 <= pos + window < Skv:
            out = out.copy()
            out[pos + window] = True   # j <= pos + W instead of j < pos + W
        return out
    _patch_visible(monkeypatch, vis)
    assert _fails(vpins.test_window_two_closed_form, 8, 8)


def test_window_lower_bound_off_by_one_is_caught(monkeypatch):
    import tests.test_oracle_variants as vpins
    real = oa.visible_keys

    def vis(i, Sq, Skv, causal=False, window=0, block_row=None, block=64):
        out = real(i, Sq, Skv, causal, window, block_row, block)
        pos = i + Skv - Sq
        if window > 0 and 0 <= pos - window < Skv:
            out = out.copy()
            out[pos - window] = False  # j > pos - W instead of j >= pos - W
        return out
    _patch_visible(monkeypatch, vis)
    assert _fails(vpins.test_window_is_attention_over_the_window_range, False, 3)


def test_block_mask_transposed_is_caught(monkeypatch):
    import tests.test_oracle_variants as vpins
    real = oracle.attention_masked

    def masked(q, k, v, scale, causal=False, window=0, block_mask=None, block=64, rows=None):
        bm = None if block_mask is None else np.ascontiguousarray(
            np.swapaxes(np.asarray(block_mask), 2, 3)[:, :, :block_mask.shape[2], :block_mask.shape[3]])
        if bm is not None and bm.shape != np.asarray(block_mask).shape:
            bm = np.resize(bm, np.asarray(block_mask).shape)
        return real(q, k, v, scale, causal, window, bm, block, rows)
    monkeypatch.setattr(oracle, "attention_masked", masked)
    assert _fails(vpins.test_block_mask_one_block_per_row_is_that_range)
