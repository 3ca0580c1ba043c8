"""Pins of the CPU oracle against facts fixed by the mathematics (no GPU).

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, a 50-digit decimal brute force on
tiny inputs, torch's float64 CPU attention routine, or an identity between
two oracle functions that share no arithmetic path. Together they fail on a
dropped term, a wrong sign, base or index, a transposed operand, an
off-by-one causal mask or a mis-weighted merge.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_12_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, mha_inputs


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _rand(rng, *shape):
    return _bf16(rng.standard_normal(shape))


# ---------------------------------------------------------------- closed forms

def test_two_keys_closed_form():
    # scores [1, 0]: P = [e/(1+e), 1/(1+e)], LSE = ln(1+e)
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    o, lse = oracle.attention(q, k, v, 1.0)
    e = math.e
    assert o[0, 0, 0] == pytest.approx([e / (1 + e), 1 / (1 + e)], abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(1 + e), abs=1e-15)


def test_log_weights_closed_form():
    # scores [0, ln 2, ln 3]: P = [1, 2, 3]/6; V = 6*I gives O = [1, 2, 3]; LSE = ln 6
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.0], [math.log(2.0)], [math.log(3.0)]]]])
    v = 6.0 * np.eye(3)[None, None]
    o, lse = oracle.attention(q, k, v, 1.0)
    assert o[0, 0, 0] == pytest.approx([1.0, 2.0, 3.0], abs=1e-14)
    assert lse[0, 0, 0] == pytest.approx(math.log(6.0), abs=1e-15)


def test_causal_closed_form():
    # Q = K = V = I(3), scale 1/2: row i sees keys 0..i; only key i scores 1/2.
    eye = np.eye(3)[None, None]
    o, lse = oracle.attention(eye, eye, eye, 0.5, causal=True)
    r = math.exp(0.5)
    assert o[0, 0, 0] == pytest.approx([1.0, 0.0, 0.0], abs=1e-15)
    assert o[0, 0, 1] == pytest.approx([1 / (1 + r), r / (1 + r), 0.0], abs=1e-15)
    assert o[0, 0, 2] == pytest.approx([1 / (2 + r), 1 / (2 + r), r / (2 + r)], abs=1e-15)
    assert lse[0, 0] == pytest.approx([0.5, math.log(1 + r), math.log(2 + r)], abs=1e-15)


def test_causal_bottom_right_alignment():
    # Sq = 2, Skv = 4: row 0 sees keys 0..2, row 1 sees keys 0..3.
    q = np.zeros((1, 1, 2, 1))
    k = np.zeros((1, 1, 4, 1))
    v = np.arange(4.0).reshape(1, 1, 4, 1)
    o, lse = oracle.attention(q, k, v, 1.0, causal=True)
    assert o[0, 0, :, 0] == pytest.approx([1.0, 1.5], abs=1e-15)
    assert lse[0, 0] == pytest.approx([math.log(3.0), math.log(4.0)], abs=1e-15)
    # Sq > Skv: the first rows see nothing -> O = 0, LSE = -inf
    q = np.ones((1, 1, 4, 1))
    k = np.ones((1, 1, 2, 1))
    v = np.ones((1, 1, 2, 1))
    o, lse = oracle.attention(q, k, v, 1.0, causal=True)
    assert np.all(o[0, 0, :2] == 0.0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert o[0, 0, 2:, 0] == pytest.approx([1.0, 1.0], abs=1e-15)
    assert lse[0, 0, 2:] == pytest.approx([1.0, 1.0 + math.log(2.0)], abs=1e-15)


# ---------------------------------------------------------------- invariants

def test_single_key_gives_v():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 2, 3, 5, 16), _rand(rng, 2, 3, 1, 16), _rand(rng, 2, 3, 1, 8)
    scale = 0.25
    o, lse = oracle.attention(q, k, v, scale)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-15, rtol=0)
    expect = scale * np.einsum("bhsd,bhd->bhs", q, k[:, :, 0])
    assert np.allclose(lse, expect, atol=1e-13, rtol=0)


def test_identical_keys_give_mean_v():
    rng = np.random.default_rng(2)
    skv = 37
    q = _rand(rng, 1, 2, 4, 8)
    k = np.broadcast_to(_rand(rng, 1, 2, 1, 8), (1, 2, skv, 8)).copy()
    v = _rand(rng, 1, 2, skv, 8)
    scale = 0.3
    o, lse = oracle.attention(q, k, v, scale)
    assert np.allclose(o, v.mean(axis=2, keepdims=True), atol=1e-14, rtol=0)
    expect = scale * np.einsum("bhsd,bhd->bhs", q, k[:, :, 0]) + math.log(skv)
    assert np.allclose(lse, expect, atol=1e-13, rtol=0)


def test_row_shift_leaves_o_and_moves_lse():
    # A constant key column of ones plus a per-row query entry c_i/scale adds c_i
    # to every score of row i.
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 11, 8), _rand(rng, 1, 1, 11, 4)
    scale = 0.5
    c = np.array([0.0, 1.0, -2.0, 7.5, 30.0, -40.0])
    q2 = np.concatenate([q, (c / scale).reshape(1, 1, 6, 1)], axis=3)
    k2 = np.concatenate([k, np.ones((1, 1, 11, 1))], axis=3)
    o1, lse1 = oracle.attention(q, k, v, scale)
    o2, lse2 = oracle.attention(q2, k2, v, scale)
    assert np.allclose(o1, o2, atol=1e-13, rtol=0)
    assert np.allclose(lse2 - lse1, c.reshape(1, 1, 6), atol=1e-12, rtol=0)


def test_causal_row0_is_v0():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 2, 9, 16), _rand(rng, 2, 2, 9, 16), _rand(rng, 2, 2, 9, 16)
    o, lse = oracle.attention(q, k, v, 0.7, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.allclose(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                       atol=1e-13, rtol=0)


def test_causal_ignores_future_keys():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 1, 12, 8), _rand(rng, 1, 1, 12, 8), _rand(rng, 1, 1, 12, 8)
    o1, l1 = oracle.attention(q, k, v, 0.4, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[..., 6:, :] += 3.0
    v2[..., 6:, :] -= 5.0
    o2, l2 = oracle.attention(q, k2, v2, 0.4, causal=True)
    assert np.array_equal(o1[..., :6, :], o2[..., :6, :])
    assert np.array_equal(l1[..., :6], l2[..., :6])
    assert not np.allclose(o1[..., 6:, :], o2[..., 6:, :])


def test_weights_sum_to_one_and_key_permutation():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 2, 5, 8), _rand(rng, 1, 2, 13, 8), _rand(rng, 1, 2, 13, 8)
    o, _ = oracle.attention(q, k, np.ones((1, 2, 13, 3)), 0.9)
    assert np.allclose(o, 1.0, atol=1e-14, rtol=0)
    perm = rng.permutation(13)
    o1, l1 = oracle.attention(q, k, v, 0.9)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.9)
    assert np.allclose(o1, o2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)


def test_gqa_matches_repeated_heads():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 1, 4, 6, 8), _rand(rng, 1, 2, 9, 8), _rand(rng, 1, 2, 9, 8)
    o1, l1 = oracle.attention(q, k, v, 0.5, causal=True)
    o2, l2 = oracle.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 0.5, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 2, 40, 8), _rand(rng, 1, 2, 40, 8), _rand(rng, 1, 2, 40, 8)
    o, l = oracle.attention(q, k, v, 0.3, causal=True, row_group=7)
    rows = np.array([0, 5, 17, 39])
    os_, ls = oracle.attention(q, k, v, 0.3, causal=True, rows=rows)
    assert np.allclose(o[:, :, rows], os_, atol=1e-15, rtol=0)
    assert np.allclose(l[:, :, rows], ls, atol=1e-15, rtol=0)


# ---------------------------------------------------------------- brute force in 50 digits

def _decimal_attention(q, k, v, scale, causal):
    getcontext().prec = 50
    Sq, Skv = q.shape[0], k.shape[0]
    sc = Decimal(float(scale))
    outs, lses = [], []
    for i in range(Sq):
        n = Skv if not causal else min(Skv, max(0, i + Skv - Sq + 1))
        s = [sc * sum(Decimal(float(q[i, d])) * Decimal(float(k[j, d])) for d in range(q.shape[1]))
             for j in range(n)]
        m = max(s)
        w = [(x - m).exp() for x in s]
        tot = sum(w)
        outs.append([float(sum(w[j] * Decimal(float(v[j, d])) for j in range(n)) / tot)
                     for d in range(v.shape[1])])
        lses.append(float(m + tot.ln()))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
def test_decimal_brute_force(causal):
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 4, 6) * 2, _rand(rng, 7, 6) * 2, _rand(rng, 7, 5)
    scale = float(np.float32(1 / math.sqrt(6)))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal=causal)
    o_ref, lse_ref = _decimal_attention(q, k, v, scale, causal)
    assert np.allclose(o[0, 0], o_ref, atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], lse_ref, atol=1e-14, rtol=0)


# ---------------------------------------------------------------- independent library routine

@pytest.mark.parametrize("causal,sq,skv", [(False, 33, 47), (True, 40, 40), (True, 17, 50)])
def test_against_torch_sdpa_float64(causal, sq, skv):
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 2, 3, sq, 16), _rand(rng, 2, 3, skv, 16), _rand(rng, 2, 3, skv, 16)
    scale = float(np.float32(0.25))
    o, lse = oracle.attention(q, k, v, scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = None
    if causal:
        i = torch.arange(sq)[:, None]
        j = torch.arange(skv)[None, :]
        mask = j <= i + (skv - sq)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    assert np.allclose(o, ref.numpy(), atol=1e-13, rtol=0)
    s = scale * (tq @ tk.transpose(-1, -2))
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-13, rtol=0)


# ---------------------------------------------------------------- online recurrence and splits

@pytest.mark.parametrize("block", [1, 7, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_matches_two_pass(block, causal):
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 2, 50, 16) * 3, _rand(rng, 1, 2, 50, 16), _rand(rng, 1, 2, 50, 8)
    o1, l1 = oracle.attention(q, k, v, 0.5, causal=causal)
    o2, l2 = oracle.online_attention(q, k, v, 0.5, causal=causal, block=block)
    assert np.allclose(o1, o2, atol=1e-13, rtol=0)
    assert np.allclose(l1, l2, atol=1e-13, rtol=0)


def test_online_exp2_form_equals_exp_form():
    # The FlashMLA walk-through exponentiates with base 2 after folding the scale:
    # exp2(s*c - m*c) with c = log2(e) is exp(s - m).
    s = np.linspace(-20.0, 0.0, 101)
    c = math.log2(math.e)
    assert np.allclose(np.exp2(s * c), np.exp(s), rtol=1e-14, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_split_combine_identity(causal):
    rng = np.random.default_rng(12)
    skv = 45
    q, k, v = _rand(rng, 1, 2, 45, 8), _rand(rng, 1, 2, skv, 8), _rand(rng, 1, 2, skv, 8)
    o_full, l_full = oracle.attention(q, k, v, 0.6, causal=causal)
    bounds = [0, 0, 3, 3, 20, 44, 45, 45]  # includes empty ranges
    parts = [oracle.attention_partial(q, k, v, 0.6, lo, hi, causal=causal)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    o, l = oracle.combine_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(o, o_full, atol=1e-14, rtol=0)
    assert np.allclose(l, l_full, atol=1e-13, rtol=0)


def test_combine_all_empty():
    o, l = oracle.combine_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------- MLA

def _mla_case(rng, B, H, lens, dl=32, dr=8):
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(indptr[-1])
    return (_rand(rng, B, H, dl) * 0.5, _rand(rng, B, H, dr) * 0.5,
            _rand(rng, n, dl) * 0.5, _rand(rng, n, dr) * 0.5, indptr)


def test_mla_equals_mha_on_concatenated_keys():
    rng = np.random.default_rng(13)
    lens = [5, 1, 17]
    q, q_pe, kv, k_pe, indptr = _mla_case(rng, 3, 4, lens)
    scale = 0.2
    o, lse = oracle.mla_decode(q, q_pe, kv, k_pe, indptr, scale)
    for b in range(3):
        lo, hi = indptr[b], indptr[b + 1]
        qc = np.concatenate([q[b], q_pe[b]], axis=1)[None, :, None, :]        # [1,H,1,Dl+Dr]
        kc = np.concatenate([kv[lo:hi], k_pe[lo:hi]], axis=1)[None, None]     # [1,1,n,Dl+Dr]
        om, lm = oracle.attention(qc, kc, kv[lo:hi][None, None], scale)      # one KV head, V = KV
        assert np.allclose(o[b], om[0, :, 0], atol=1e-14, rtol=0)
        assert np.allclose(lse[b], lm[0, :, 0], atol=1e-14, rtol=0)


def test_mla_rope_part_matters_and_rows_match():
    rng = np.random.default_rng(14)
    q, q_pe, kv, k_pe, indptr = _mla_case(rng, 2, 3, [9, 4])
    o1, l1 = oracle.mla_decode(q, q_pe, kv, k_pe, indptr, 0.3)
    o2, l2 = oracle.mla_decode(q, 0 * q_pe, kv, k_pe, indptr, 0.3)
    assert not np.allclose(l1, l2)
    pairs = [(0, 0), (1, 2), (0, 1)]
    orow, lrow = oracle.mla_decode_rows(q, q_pe, kv, k_pe, indptr, 0.3, pairs)
    for n, (b, h) in enumerate(pairs):
        assert np.allclose(orow[n], o1[b, h], atol=1e-15, rtol=0)
        assert lrow[n] == pytest.approx(l1[b, h], abs=1e-15)


def test_mla_single_and_identical_keys():
    rng = np.random.default_rng(15)
    q, q_pe, kv, k_pe, indptr = _mla_case(rng, 2, 3, [1, 6])
    kv[1:7] = kv[1]
    k_pe[1:7] = k_pe[1]
    o, lse = oracle.mla_decode(q, q_pe, kv, k_pe, indptr, 0.5)
    assert np.allclose(o[0], kv[0][None], atol=1e-15, rtol=0)
    assert np.allclose(o[1], kv[1][None], atol=1e-15, rtol=0)
    s1 = 0.5 * (q[1] @ kv[1] + q_pe[1] @ k_pe[1])
    assert np.allclose(lse[1], s1 + math.log(6), atol=1e-14, rtol=0)


def test_mla_empty_batch():
    rng = np.random.default_rng(16)
    q, q_pe, kv, k_pe, indptr = _mla_case(rng, 2, 2, [0, 3])
    o, lse = oracle.mla_decode(q, q_pe, kv, k_pe, indptr, 0.5)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- the input generator

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties -> 1+2^-6
    assert got[:5].tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5]
    assert abs(float(got[5]) - 3.0e38) / 3.0e38 < 2**-8


def test_inputs_are_seeded():
    a = mha_inputs(1, 2, 8, 8, 16, seed=5)
    b = mha_inputs(1, 2, 8, 8, 16, seed=5)
    c = mha_inputs(1, 2, 8, 8, 16, seed=6)
    assert all(np.array_equal(a[n], b[n]) for n in "qkv")
    assert not np.array_equal(a["q"], c["q"])
