"""GPU parity of ssd_scan (the Mamba-2 state-space scan) against the CPU
float64 oracle (needs gfx950).

Element by element against the step-by-step definition
(``oracle.ssd.ssd_recurrence``) at sizes it finishes quickly (several 64-step
chunks and ragged tails, both workgroup shapes: two heads per workgroup when
heads per group is even, one when it is odd), with and without initial and
final states; on sampled whole heads, again by the recurrence, at the full
benchmark workload.

Tolerance (tests/ssd_bounds.py, pinned on the CPU by tests/test_ssd_bounds.py):
derived term by term from where the kernel rounds to bf16 (the decay-weighted
scores G inside a chunk, the state where it meets C, the decay-weighted B of
the state update, and y itself) and from its fp32 arithmetic. Per element,
|dy| <= 6 u sqrt(sum of the squared rounded terms) + half a bf16 ulp of y +
the worst-case fp32 terms (u = 2^-8), and the mean of |dy| over a head stays
under its expected size; the fp32 final state, which sees only the rounding
of B, is bounded the same way.
"""

import os

import numpy as np
import pytest

import oracle.ssd as ossd
from tests.helpers import to_dev, to_np
from tests.ssd_bounds import check_head, head_scales
from tiled_attention_12_amd import inputs
from tiled_attention_12_amd.workloads import WORKLOADS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ta(lib_path):
    import tiled_attention_12_amd as ta
    return ta


def _ref_inputs(d):
    return (inputs.stored_values(d["x"]), d["dt"], d["A"], inputs.stored_values(d["B"]),
            inputs.stored_values(d["C"]))


def _recurrence_heads(d, pairs):
    """(y [n, L, P], final state [n, P, N]) of the selected (batch, head)
    pairs by the step-by-step recurrence, one head at a time."""
    x, dt, A, B, C = _ref_inputs(d)
    H, G = x.shape[2], B.shape[2]
    ys, fs = [], []
    for b, h in pairs:
        g = h // (H // G)
        s0 = d["init_state"][b:b + 1, h:h + 1] if "init_state" in d else None
        y, f = ossd.ssd_recurrence(x[b:b + 1, :, h:h + 1], dt[b:b + 1, :, h:h + 1], A[h:h + 1],
                                   B[b:b + 1, :, g:g + 1], C[b:b + 1, :, g:g + 1], s0)
        ys.append(y[0, :, 0])
        fs.append(f[0, 0])
    return np.stack(ys), np.stack(fs)


def _run(ta, dev, d, final=False):
    x, B, C = (to_dev(d[n], dev) for n in ("x", "B", "C"))
    dt, A = to_dev(d["dt"], dev), to_dev(d["A"], dev)
    s0 = to_dev(d["init_state"], dev) if "init_state" in d else None
    # outputs start as NaN, so an element the kernel does not write fails
    Bt, L, H, P = x.shape
    y = torch.full((Bt, L, H, P), float("nan"), dtype=torch.bfloat16, device=dev)
    fs = torch.full((Bt, H, P, B.shape[3]), float("nan"), dtype=torch.float32, device=dev) if final else False
    r = ta.ssd_scan(x, dt, A, B, C, init_state=s0, final_state=fs, out=y)
    torch.cuda.synchronize()
    if final:
        return to_np(r[0]), to_np(r[1])
    return to_np(r), None


def _scales(d, refs, b, h):
    x, dt, A, B, C = refs
    g = h // (x.shape[2] // B.shape[2])
    s0 = d["init_state"][b, h].astype(np.float64) if "init_state" in d else None
    return head_scales(x[b, :, h], dt[b, :, h].astype(np.float64), A[h], B[b, :, g], C[b, :, g], s0)


def _check(d, pairs, y, ry, what, f=None, rf=None):
    """Per (batch, head) pair i: y [Bt, L, H, P] against ry[i] [L, P] and, when
    given, the final states f [Bt, H, P, N] against rf[i] [P, N]."""
    refs = _ref_inputs(d)
    for i, (b, h) in enumerate(pairs):
        check_head(y[b, :, h], ry[i], _scales(d, refs, b, h), f"{what} b={b} h={h}",
                   None if f is None else f[b, h], None if rf is None else rf[i])


def _check_all(d, y, ry, what, f=None, rf=None):
    """Every head of a batched run against the batched recurrence outputs."""
    Bt, _, H, _ = d["x"].shape
    pairs = [(b, h) for b in range(Bt) for h in range(H)]
    _check(d, pairs, y, [ry[b, :, h] for b, h in pairs], what, f,
           None if rf is None else [rf[b, h] for b, h in pairs])


CASES = [
    # Bt, L, H, G, init, final
    (2, 200, 4, 1, True, True),      # two heads per workgroup, ragged tail, states in and out
    (2, 130, 6, 2, True, True),      # three heads per group: one head per workgroup
    (1, 64, 8, 4, False, True),      # exactly one chunk, four groups
    (3, 65, 2, 1, False, False),     # 3 workgroups (no XCD order), one step in the last chunk
    (1, 1, 2, 2, True, True),        # a single step; one head per group
    (2, 63, 2, 1, True, True),
    (4, 700, 16, 2, False, True),    # 32 workgroups, 11 chunks
]


def _random_case(i):
    rng = np.random.default_rng(11000 + i)
    G = int(rng.choice([1, 2, 4]))
    return (int(rng.integers(1, 5)), int(rng.integers(1, 601)), G * int(rng.integers(1, 5)), G,
            bool(rng.integers(0, 2)), bool(rng.integers(0, 2)))


_N_RANDOM = 16 * max(1, int(os.environ.get("TATTN_RANDOM_SCALE", "1")))  # more for a longer sweep


@pytest.mark.parametrize("Bt,L,H,G,init,final", CASES + [_random_case(i) for i in range(_N_RANDOM)])
def test_ssd_against_oracle(ta, dev, Bt, L, H, G, init, final):
    d = inputs.ssd_inputs(Bt, L, H, G, 64, 128, seed=7000 + L + H, init_state=init)
    print(f"ssd Bt={Bt} L={L} H={H} G={G} init={init} final={final}", flush=True)
    y, f = _run(ta, dev, d, final)
    ry, rf = ossd.ssd_recurrence(*_ref_inputs(d), d.get("init_state"))
    _check_all(d, y, ry, "ssd", f, rf if final else None)


def test_ssd_empty_sequence_copies_the_state(ta, dev):
    d = inputs.ssd_inputs(2, 0, 4, 1, 64, 128, seed=7100, init_state=True)
    y, f = _run(ta, dev, d, final=True)
    assert y.shape == (2, 0, 4, 64)
    np.testing.assert_array_equal(f, d["init_state"].astype(np.float64))
    d.pop("init_state")
    _, f = _run(ta, dev, d, final=True)
    assert not f.any()


def test_ssd_extreme_decay_rates(ta, dev):
    # fastest decay of the Mamba-2 range (dt = 0.1, A = -16: the state forgets
    # within a step or two and exp underflows inside a chunk) next to almost
    # no decay over a long sequence (dt = 1e-3, A = -1)
    d = inputs.ssd_inputs(1, 1000, 4, 1, 64, 128, seed=7200, init_state=True)
    d["dt"][:, :, :2] = 0.1
    d["dt"][:, :, 2:] = 1e-3
    d["A"][:2] = -16.0
    d["A"][2:] = -1.0
    y, f = _run(ta, dev, d, final=True)
    ry, rf = ossd.ssd_recurrence(*_ref_inputs(d), d["init_state"])
    _check_all(d, y, ry, "extreme decays", f, rf)


def test_ssd_full_workload_sampled_heads(ta, dev):
    w = WORKLOADS["ssd_scan_bf16"]
    d = inputs.ssd_inputs(w["Bt"], w["L"], w["H"], w["G"], w["P"], w["N"], seed=w["seed"])
    print(f"ssd full workload {w}", flush=True)
    y, f = _run(ta, dev, d, final=True)
    rng = np.random.default_rng(5)
    pairs = [(0, 0), (w["Bt"] - 1, w["H"] - 1)] + [(int(rng.integers(w["Bt"])), int(rng.integers(w["H"])))
                                                    for _ in range(6)]
    ry, rf = _recurrence_heads(d, pairs)
    _check(d, pairs, y, ry, "full workload", f, rf)


def test_ssd_more_heads_than_one_pass_of_the_chip(ta, dev):
    # 16 x 80 heads (a 2.7B-class layer): 640 workgroups of two heads
    d = inputs.ssd_inputs(16, 256, 80, 1, 64, 128, seed=7300)
    y, _ = _run(ta, dev, d)
    pairs = [(0, 0), (15, 79), (7, 40), (3, 1), (12, 63)]
    ry, _ = _recurrence_heads(d, pairs)
    _check(d, pairs, y, ry, "640 workgroups")


def test_ssd_continuation_matches_one_pass(ta, dev):
    # a sequence scanned in two calls, the first call's final state fed to the
    # second as its initial state: each call, and the one-pass scan, match the
    # recurrence on their own inputs (the recurrence continues exactly, so the
    # second call's outputs are the one-pass ones up to both calls' bounds)
    d = inputs.ssd_inputs(2, 320, 4, 1, 64, 128, seed=7400, init_state=True)
    y, f = _run(ta, dev, d, final=True)
    ry, rf = ossd.ssd_recurrence(*_ref_inputs(d), d["init_state"])
    _check_all(d, y, ry, "one pass", f, rf)
    L1 = 192
    first = {k: (v[:, :L1] if k in ("x", "B", "C", "dt") else v) for k, v in d.items()}
    y1, f1 = _run(ta, dev, first, final=True)
    ry1, rf1 = ossd.ssd_recurrence(*_ref_inputs(first), first["init_state"])
    _check_all(first, y1, ry1, "first half", f1, rf1)
    second = {k: (v[:, L1:] if k in ("x", "B", "C", "dt") else v) for k, v in d.items()}
    second["init_state"] = f1.astype(np.float32)
    y2, f2 = _run(ta, dev, second, final=True)
    ry2, rf2 = ossd.ssd_recurrence(*_ref_inputs(second), second["init_state"])
    _check_all(second, y2, ry2, "second half", f2, rf2)


_N_LARGER = 4 * max(1, int(os.environ.get("TATTN_RANDOM_SCALE", "1")))


@pytest.mark.parametrize("i", range(_N_LARGER))
def test_ssd_random_larger_launch(ta, dev, i):
    # larger seeded launches, often with more workgroups than compute units:
    # every output written (NaN-prefilled), three heads against the recurrence
    rng = np.random.default_rng(16000 + i)
    G = int(rng.choice([1, 2, 4]))
    Bt, L, H = int(rng.integers(1, 9)), int(rng.integers(500, 3001)), G * int(rng.integers(4, 25))
    init, final = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    print(f"larger scan case {i}: Bt={Bt} L={L} H={H} G={G} init={init} final={final}", flush=True)
    d = inputs.ssd_inputs(Bt, L, H, G, 64, 128, seed=16500 + i, init_state=init)
    x, B, C = (to_dev(d[n], dev) for n in ("x", "B", "C"))
    dt, A = to_dev(d["dt"], dev), to_dev(d["A"], dev)
    s0 = to_dev(d["init_state"], dev) if init else None
    y = torch.full((Bt, L, H, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    fs = torch.full((Bt, H, 64, 128), float("nan"), dtype=torch.float32, device=dev) if final else False
    r = ta.ssd_scan(x, dt, A, B, C, init_state=s0, final_state=fs, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item() and (not final or not torch.isnan(fs).any().item())
    pairs = [(0, 0), (Bt - 1, H - 1), (int(rng.integers(Bt)), int(rng.integers(H)))]
    ry, rf = _recurrence_heads(d, pairs)
    _check(d, pairs, to_np(y), ry, f"larger scan case {i}", to_np(r[1]) if final else None, rf if final else None)
