"""Pins of the CPU state-space-scan oracle (no GPU), and planted mistakes.

The scan has no printed worked example on the source pages, so the oracle is
pinned by what the recurrence fixes mathematically: the one-step and
constant-input (geometric series) closed forms, the impulse response, the
no-decay case (causal linear attention written as one masked matrix
product), a 50-digit decimal evaluation of the unrolled sum on a tiny input,
linearity, continuation from a final state, the head-to-group mapping, and
the chunked form against the step-by-step one at several chunk lengths.
Every pin runs on both oracle forms. The second half plants plausible
mistakes in the oracle and checks that some pin fails.
"""

from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle.ssd as ssd
from tiled_attention_12_amd.inputs import bf16_bits_to_f32, ssd_inputs

IMPLS = {
    "recurrence": lambda x, dt, A, B, C, s0=None: ssd.ssd_recurrence(x, dt, A, B, C, s0),
    "chunked64": lambda x, dt, A, B, C, s0=None: ssd.ssd_chunked(x, dt, A, B, C, 64, s0),
    "chunked5": lambda x, dt, A, B, C, s0=None: ssd.ssd_chunked(x, dt, A, B, C, 5, s0),
}


def _rand_case(Bt, L, H, G, P, N, seed, init=False):
    d = ssd_inputs(Bt, L, H, G, P, N, seed, init_state=init)
    out = [bf16_bits_to_f32(d["x"]), d["dt"], d["A"], bf16_bits_to_f32(d["B"]), bf16_bits_to_f32(d["C"])]
    return [np.asarray(a, dtype=np.float64) for a in out] + ([d["init_state"].astype(np.float64)] if init else [])


# ------------------------------------------------------------------ the pins

def pin_single_step(impl):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 1, 1, 3))
    B = rng.standard_normal((1, 1, 1, 4))
    C = rng.standard_normal((1, 1, 1, 4))
    dt = np.array([[[0.37]]])
    A = np.array([-2.5])
    s0 = rng.standard_normal((1, 1, 3, 4))
    y, f = impl(x, dt, A, B, C, s0)
    want_f = np.exp(0.37 * -2.5) * s0[0, 0] + 0.37 * np.outer(x[0, 0, 0], B[0, 0, 0])
    np.testing.assert_allclose(f[0, 0], want_f, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y[0, 0, 0], want_f @ C[0, 0, 0], rtol=1e-13, atol=1e-14)


def pin_constant_input(impl):
    # x_t = x, B_t = B, C_t = C, dt_t = d: the state is a geometric series,
    # state_t = d (1 - r^(t+1)) / (1 - r) x (outer) B with r = exp(d a).
    L, d, a = 150, 0.05, -3.0
    rng = np.random.default_rng(2)
    xv, bv, cv = rng.standard_normal(5), rng.standard_normal(7), rng.standard_normal(7)
    x = np.broadcast_to(xv, (1, L, 1, 5)).copy()
    B = np.broadcast_to(bv, (1, L, 1, 7)).copy()
    C = np.broadcast_to(cv, (1, L, 1, 7)).copy()
    dt = np.full((1, L, 1), d)
    y, f = impl(x, dt, np.array([a]), B, C)
    r = np.exp(d * a)
    t = np.arange(L)
    g = d * (1 - r ** (t + 1)) / (1 - r)
    want = g[:, None] * (bv @ cv) * xv[None, :]
    np.testing.assert_allclose(y[0, :, 0], want, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(f[0, 0], g[-1] * np.outer(xv, bv), rtol=1e-11, atol=1e-13)


def pin_impulse(impl):
    # one nonzero input at step s0: y_t = 0 for t < s0 and
    # y_t = exp(a * sum_{u=s0+1..t} dt_u) dt_{s0} (C_t . B_{s0}) x_{s0} after.
    L, s0, P, N = 140, 37, 4, 6
    rng = np.random.default_rng(3)
    x = np.zeros((1, L, 1, P))
    x[0, s0, 0] = rng.standard_normal(P)
    B = rng.standard_normal((1, L, 1, N))
    C = rng.standard_normal((1, L, 1, N))
    dt = rng.uniform(0.01, 0.2, size=(1, L, 1))
    a = -1.7
    y, _ = impl(x, dt, np.array([a]), B, C)
    want = np.zeros((L, P))
    for t in range(s0, L):
        decay = np.exp(a * dt[0, s0 + 1:t + 1, 0].sum())
        want[t] = decay * dt[0, s0, 0] * (C[0, t, 0] @ B[0, s0, 0]) * x[0, s0, 0]
    np.testing.assert_allclose(y[0, :, 0], want, rtol=1e-11, atol=1e-13)


def pin_no_decay(impl):
    # A = 0: y = ((C B^T) masked causally, times dt of the key step) x, one
    # matrix product per (batch, head).
    x, dt, _, B, C = _rand_case(2, 90, 2, 1, 5, 6, seed=4)
    A = np.zeros(2)
    y, _ = impl(x, dt, A, B, C)
    for b in range(2):
        for h in range(2):
            cb = C[b, :, 0] @ B[b, :, 0].T
            m = np.tril(cb) * dt[b, None, :, h]
            np.testing.assert_allclose(y[b, :, h], m @ x[b, :, h], rtol=1e-11, atol=1e-12)


def pin_decimal_brute_force(impl):
    # the unrolled sum y_t = sum_{s<=t} exp(a sum_{u=s+1..t} dt_u) dt_s (C_t.B_s) x_s
    # plus the decayed initial state, in 50-digit decimal arithmetic
    getcontext().prec = 50
    L, P, N = 6, 2, 3
    rng = np.random.default_rng(5)
    x = np.round(rng.standard_normal((1, L, 1, P)), 3)
    B = np.round(rng.standard_normal((1, L, 1, N)), 3)
    C = np.round(rng.standard_normal((1, L, 1, N)), 3)
    dt = np.round(rng.uniform(0.05, 0.5, size=(1, L, 1)), 3)
    s0 = np.round(rng.standard_normal((1, 1, P, N)), 3)
    a = -2.25
    y, f = impl(x, dt, np.array([a]), B, C, s0)
    D = lambda v: Decimal(repr(float(v)))
    for t in range(L):
        for p in range(P):
            acc = Decimal(0)
            for s in range(t + 1):
                e = (D(a) * sum((D(dt[0, u, 0]) for u in range(s + 1, t + 1)), Decimal(0))).exp()
                cb = sum(D(C[0, t, 0, n]) * D(B[0, s, 0, n]) for n in range(N))
                acc += e * D(dt[0, s, 0]) * cb * D(x[0, s, 0, p])
            e0 = (D(a) * sum((D(dt[0, u, 0]) for u in range(t + 1)), Decimal(0))).exp()
            acc += e0 * sum(D(s0[0, 0, p, n]) * D(C[0, t, 0, n]) for n in range(N))
            assert abs(float(acc) - y[0, t, 0, p]) <= 1e-13 * max(1.0, abs(float(acc)))


def pin_linearity(impl):
    x1, dt, A, B, C = _rand_case(1, 70, 2, 1, 4, 5, seed=6)
    x2 = _rand_case(1, 70, 2, 1, 4, 5, seed=7)[0]
    y1, f1 = impl(x1, dt, A, B, C)
    y2, f2 = impl(x2, dt, A, B, C)
    y3, f3 = impl(2.0 * x1 - 3.0 * x2, dt, A, B, C)
    np.testing.assert_allclose(y3, 2.0 * y1 - 3.0 * y2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f3, 2.0 * f1 - 3.0 * f2, rtol=1e-10, atol=1e-12)


def pin_continuation(impl):
    # running [0, L1) and then [L1, L) from the first part's final state is
    # the same as one run over [0, L)
    x, dt, A, B, C, s0 = _rand_case(2, 160, 2, 2, 4, 6, seed=8, init=True)
    y, f = impl(x, dt, A, B, C, s0)
    L1 = 67
    ya, fa = impl(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], s0)
    yb, fb = impl(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], fa)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fb, f, rtol=1e-10, atol=1e-12)


def pin_groups(impl):
    # head h reads group h // (H / G) of B and C
    x, dt, A, B, C = _rand_case(1, 50, 4, 2, 3, 4, seed=9)
    y, _ = impl(x, dt, A, B, C)
    for h in range(4):
        g = h // 2
        yh, _ = impl(x[:, :, h:h + 1], dt[:, :, h:h + 1], A[h:h + 1], B[:, :, g:g + 1], C[:, :, g:g + 1])
        np.testing.assert_allclose(y[:, :, h], yh[:, :, 0], rtol=1e-12, atol=1e-13)


PINS = [pin_single_step, pin_constant_input, pin_impulse, pin_no_decay, pin_decimal_brute_force,
        pin_linearity, pin_continuation, pin_groups]


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin, impl):
    pin(IMPLS[impl])


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("chunk", [1, 7, 64])
def test_chunked_equals_recurrence(L, chunk):
    x, dt, A, B, C, s0 = _rand_case(2, L, 4, 2, 6, 5, seed=10 + L, init=True)
    y0, f0 = ssd.ssd_recurrence(x, dt, A, B, C, s0)
    y1, f1 = ssd.ssd_chunked(x, dt, A, B, C, chunk, s0)
    np.testing.assert_allclose(y1, y0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f1, f0, rtol=1e-10, atol=1e-12)


def test_empty_sequence():
    x, dt, A, B, C, s0 = _rand_case(2, 0, 2, 1, 3, 4, seed=11, init=True)
    for impl in IMPLS.values():
        y, f = impl(x, dt, A, B, C, s0)
        assert y.shape == (2, 0, 2, 3)
        np.testing.assert_array_equal(f, s0)


def test_rows_match_full():
    x, dt, A, B, C, s0 = _rand_case(2, 130, 4, 2, 4, 5, seed=12, init=True)
    y, f = ssd.ssd_chunked(x, dt, A, B, C, 64, s0)
    pairs = [(0, 3), (1, 0), (1, 2)]
    yr, fr = ssd.ssd_rows(x, dt, A, B, C, pairs, 64, s0)
    for i, (b, h) in enumerate(pairs):
        np.testing.assert_allclose(yr[i], y[b, :, h], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(fr[i], f[b, h], rtol=1e-13, atol=1e-14)


def test_generator_ranges():
    d = ssd_inputs(2, 300, 8, 1, 4, 4, seed=13)
    assert d["dt"].dtype == np.float32 and d["A"].dtype == np.float32
    assert (d["dt"] >= 1e-3 * 0.999).all() and (d["dt"] <= 1e-1 * 1.001).all()
    assert (d["A"] <= -1.0).all() and (d["A"] >= -16.0).all()
    assert d["x"].dtype == np.uint16 and d["x"].shape == (2, 300, 8, 4)


# ------------------------------------------------------- planted mistakes

def _caught(impl):
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            return True
    return False


def test_exclusive_chunk_cumsum_is_caught(monkeypatch):
    real = ssd._chunk_cumsum
    monkeypatch.setattr(ssd, "_chunk_cumsum", lambda dt, A, lo, hi: real(dt, A, lo, hi) - dt[:, lo:hi] * A)
    assert _caught(IMPLS["chunked64"]) and _caught(IMPLS["chunked5"])


def test_chunk_cumsum_without_a_is_caught(monkeypatch):
    monkeypatch.setattr(ssd, "_chunk_cumsum", lambda dt, A, lo, hi: np.cumsum(dt[:, lo:hi], axis=1))
    assert _caught(IMPLS["chunked64"]) and _caught(IMPLS["chunked5"])


def test_state_passing_without_decay_is_caught(monkeypatch):
    real = ssd.state_passing
    monkeypatch.setattr(ssd, "state_passing", lambda S, tot, s0=None: real(S, np.zeros_like(tot), s0))
    assert _caught(IMPLS["chunked5"])


def test_step_without_dt_on_input_is_caught(monkeypatch):
    monkeypatch.setattr(ssd, "_step", lambda st, d, a, x, b: np.exp(d * a) * st + np.outer(x, b))
    assert _caught(IMPLS["recurrence"])


def test_step_with_positive_exponent_is_caught(monkeypatch):
    monkeypatch.setattr(ssd, "_step", lambda st, d, a, x, b: np.exp(-d * a) * st + d * np.outer(x, b))
    assert _caught(IMPLS["recurrence"])


def test_step_decaying_the_new_input_is_caught(monkeypatch):
    monkeypatch.setattr(ssd, "_step", lambda st, d, a, x, b: np.exp(d * a) * (st + d * np.outer(x, b)))
    assert _caught(IMPLS["recurrence"])


def test_swapped_b_and_c_is_caught():
    assert _caught(lambda x, dt, A, B, C, s0=None: ssd.ssd_chunked(x, dt, A, C, B, 64, s0))


def test_step_size_of_the_previous_step_is_caught():
    def shifted(x, dt, A, B, C, s0=None):
        d = np.concatenate([dt[:, :1], dt[:, :-1]], axis=1) if dt.shape[1] else dt
        return ssd.ssd_recurrence(x, d, A, B, C, s0)
    assert _caught(shifted)
