"""Seeded random configurations of the prefill (bf16 and fp32) and decode
entry points, every element compared with the float64 oracle (needs gfx950).

Each case draws its own shape and options from a fixed seed: batch, query and
KV head counts (grouped or not), ragged query and key lengths, head width,
causal mask, sliding window, block-mask density, input magnitude, scale and
the dense prefill's workgroup shape (automatic or forced), or, for the
decode, the batch count, head count and per-batch key counts (empty batches
included). Outputs start as NaN so an unwritten element fails.

Gates. Inputs drawn with standard deviation sigma (a power of two) give
outputs sigma times as large, so O is compared after dividing both sides by
sigma (exact). The mean, LSE and relative-L2 gates are those of the other
edge tests. The per-element gate is the error bound of a bf16-P kernel:
with P rounded to bf16 for the P*V product (8 significant bits: relative
error <= 2^-8 per term) and the row sum l kept in fp32,
|dO| <= 2^-8 * sum_j p_j |v_j| / l <= 2^-8 * max |v_j|, plus the half-ulp of
rounding O itself to bf16, plus the fp32 accumulation of the P*V sums (at
most Skv 2^-24 max|v|). Very peaked rows (large sigma and scale) come close
to it: the steps exponentiate against a running max that may sit below the
row's true max (tile 0's max on the dense path, a max raised only by more
than 2^8 on the exact step), so even a row's dominant term 2^d (0 <= d <= 8)
is rounded, where with the exact row max it would be 1. For unit-variance
inputs (max|v| ~ 4.5) the bound is ~0.018 plus the half-ulp; the errors
measured there stay under 1e-2, and the configuration tests hold them to it.
"""

import os

import numpy as np
import pytest

import oracle
from tests.helpers import (BF16_MAX_ABS_LSE, BF16_REL_L2_O, assert_bf16_parity, assert_f32_parity,
                           bf16_half_ulp, bf16_mean_o_bound, parity_stats, to_dev, to_np)
from tiled_attention_12_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# how many seeded cases of each kind run; TATTN_RANDOM_SCALE multiplies the
# defaults for a longer sweep (the seeds of the default cases stay the same)
_SCALE = max(1, int(os.environ.get("TATTN_RANDOM_SCALE", "1")))
N_PREFILL, N_FP32, N_DECODE, N_MANY = 60 * _SCALE, 12 * _SCALE, 20 * _SCALE, 8 * _SCALE
N_BIG_DECODE = 4 * _SCALE


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ta(lib_path):
    import tiled_attention_12_amd as ta
    return ta


def _prefill_case(i):
    rng = np.random.default_rng(5000 + i)
    hkv = int(rng.choice([1, 2, 4]))
    c = {"B": int(rng.integers(1, 4)), "Hkv": hkv, "H": hkv * int(rng.choice([1, 2, 4])),
         "Sq": int(rng.integers(1, 520)), "Skv": int(rng.integers(1, 520)), "D": int(rng.choice([64, 128])),
         "causal": bool(rng.integers(0, 2)),
         "window": int(rng.integers(1, 400)) if rng.random() < 0.35 else 0,
         "density": float(rng.uniform(0.15, 0.9)) if rng.random() < 0.3 else None,
         "sigma": float(rng.choice([0.5, 1.0, 2.0])),
         "waves": str(rng.choice(["auto", "4", "8"]))}
    c["scale"] = float(np.float32(c["D"] ** -0.5 if rng.random() < 0.6 else rng.uniform(0.05, 0.3)))
    c["plain"] = c["H"] == c["Hkv"] and c["window"] == 0 and c["density"] is None and rng.random() < 0.5
    return c


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill_configuration(ta, dev, i, monkeypatch):
    c = _prefill_case(i)
    if c["waves"] == "auto":
        monkeypatch.delenv("TATTN_MHA_WAVES", raising=False)
    else:
        monkeypatch.setenv("TATTN_MHA_WAVES", c["waves"])
    B, H, Sq, Skv, D = c["B"], c["H"], c["Sq"], c["Skv"], c["D"]
    x = inputs.mha_inputs(B, H, Sq, Skv, D, seed=6000 + i, sigma=c["sigma"], Hkv=c["Hkv"])
    mask = None if c["density"] is None else inputs.block_mask(B, H, Sq, Skv, c["density"], seed=7000 + i)
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    if c["plain"]:
        ta.attn_fwd(q, k, v, causal=c["causal"], scale=c["scale"], out=o, lse=lse)
    else:
        m = None if mask is None else torch.from_numpy(mask).to(dev)
        ta.attn_fwd_ex(q, k, v, causal=c["causal"], scale=c["scale"], window=c["window"], block_mask=m,
                       out=o, lse=lse)
    torch.cuda.synchronize()
    vals = [inputs.stored_values(x[n]) for n in "qkv"]
    ro, rl = oracle.attention_masked(*vals, c["scale"], causal=c["causal"], window=c["window"], block_mask=mask)
    sg = c["sigma"]
    got, ref = to_np(o) / sg, ro / sg
    st = parity_stats(got, to_np(lse), ref, rl)
    msg = f"random prefill case {i} {c}: {st}"
    # per (batch, query head): 2^-8 max|v| of its KV head, plus O's half-ulp
    vmax = np.abs(vals[2]).max(axis=(2, 3)) / sg  # [B, Hkv]
    vmax = np.repeat(vmax, H // c["Hkv"], axis=1)[:, :, None, None]
    # (+ the fp32 accumulation of sum_j p_j v_j over Skv terms, <= Skv 2^-24 max|v| after the 1/l, doubled)
    bound = 2.0 ** -8 * vmax + bf16_half_ulp(ref) + Skv * 2.0 ** -23 * vmax + 1e-5
    assert np.all(np.abs(got - ref) <= bound), msg + f" (worst excess {(np.abs(got - ref) - bound).max():.3g})"
    assert st["mean_o"] <= bf16_mean_o_bound(ref), msg
    assert st["max_lse"] <= BF16_MAX_ABS_LSE, msg
    assert st["rel_l2"] <= BF16_REL_L2_O, msg


def _many_items_case(i):
    rng = np.random.default_rng(12000 + i)
    hkv = int(rng.choice([2, 4, 8, 16]))
    c = {"B": int(rng.integers(1, 5)), "Hkv": hkv, "H": hkv * int(rng.choice([1, 2, 4, 8])),
         "Sq": int(rng.integers(600, 3001)), "D": int(rng.choice([64, 128])), "causal": bool(rng.integers(0, 2)),
         "window": int(rng.integers(1, 1200)) if rng.random() < 0.3 else 0,
         "density": float(rng.uniform(0.2, 0.9)) if rng.random() < 0.25 else None,
         "waves": str(rng.choice(["auto", "4", "8"]))}
    c["Skv"] = c["Sq"] if rng.random() < 0.5 else int(rng.integers(600, 3001))
    c["H"] = min(c["H"], 64)
    return c


@pytest.mark.parametrize("i", range(N_MANY))
def test_random_prefill_with_many_work_items(ta, dev, i, monkeypatch):
    # larger launches, most with more work items than compute units (the
    # persistent workgroups loop over several items, in the XCD and causal
    # orders):
    # every output written (NaN-prefilled), three sampled heads against the
    # oracle under the same bounds as the configuration tests above
    c = _many_items_case(i)
    if c["waves"] == "auto":
        monkeypatch.delenv("TATTN_MHA_WAVES", raising=False)
    else:
        monkeypatch.setenv("TATTN_MHA_WAVES", c["waves"])
    B, H, Hkv, Sq, Skv, D = c["B"], c["H"], c["Hkv"], c["Sq"], c["Skv"], c["D"]
    print(f"many items case {i}: {c}", flush=True)
    x = inputs.mha_inputs(B, H, Sq, Skv, D, seed=12500 + i, Hkv=Hkv)
    mask = None if c["density"] is None else inputs.block_mask(B, H, Sq, Skv, c["density"], seed=13000 + i)
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(D ** -0.5))
    m = None if mask is None else torch.from_numpy(mask).to(dev)
    ta.attn_fwd_ex(q, k, v, causal=c["causal"], scale=scale, window=c["window"], block_mask=m, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), f"case {i}: unwritten outputs"
    rng = np.random.default_rng(14000 + i)
    picks = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in picks:
        kh = h // (H // Hkv)
        mk = None if mask is None else mask[b:b + 1, h:h + 1]
        qh = inputs.stored_values(x["q"][b:b + 1, h:h + 1])
        kk, vv = (inputs.stored_values(x[n][b:b + 1, kh:kh + 1]) for n in "kv")
        ro, rl = oracle.attention_masked(qh, kk, vv, scale, causal=c["causal"], window=c["window"], block_mask=mk)
        got, got_l = to_np(o[b:b + 1, h:h + 1]), to_np(lse[b:b + 1, h:h + 1])
        st = parity_stats(got, got_l, ro, rl)
        msg = f"many items case {i} {c} head ({b}, {h}): {st}"
        vmax = np.abs(vv).max()
        bound = 2.0 ** -8 * vmax + bf16_half_ulp(ro) + Skv * 2.0 ** -23 * vmax + 1e-5
        assert np.all(np.abs(got - ro) <= bound), msg
        assert st["mean_o"] <= bf16_mean_o_bound(ro), msg
        assert st["max_lse"] <= BF16_MAX_ABS_LSE, msg
        assert st["rel_l2"] <= BF16_REL_L2_O, msg


@pytest.mark.parametrize("i", range(N_FP32))
def test_random_fp32_prefill_configuration(ta, dev, i):
    # the fp32 path (no rounding of P or O): the plain fp32 gates
    rng = np.random.default_rng(10000 + i)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    Sq, Skv, D = int(rng.integers(1, 400)), int(rng.integers(1, 400)), int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    scale = float(np.float32(D ** -0.5 if rng.random() < 0.6 else rng.uniform(0.05, 0.3)))
    x = inputs.mha_inputs(B, H, Sq, Skv, D, seed=10500 + i, dtype="f32")
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    ta.attn_fwd_f32(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], scale, causal=causal)
    assert_f32_parity(to_np(o), to_np(lse), ro, rl, f"random fp32 case {i} B={B} H={H} {Sq}x{Skv} D={D} "
                                                    f"causal={causal} scale={scale}")


def _decode_case(i):
    rng = np.random.default_rng(8000 + i)
    B = int(rng.integers(1, 41))
    H = int(rng.integers(1, 129))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.15] = 0
    return B, H, lens.astype(np.int64)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_configuration(ta, dev, i):
    B, H, lens = _decode_case(i)
    rng = np.random.default_rng(9000 + i)
    sig = np.float32(0.3)
    n = int(lens.sum())
    m = {"q": inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 512), dtype=np.float32) * sig),
         "q_pe": inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32) * sig),
         "kv": inputs.f32_to_bf16_bits(rng.standard_normal((n, 512), dtype=np.float32) * sig),
         "k_pe": inputs.f32_to_bf16_bits(rng.standard_normal((n, 64), dtype=np.float32) * sig),
         "indptr": np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)}
    scale = float(np.float32(576 ** -0.5))
    args = [to_dev(m[k], dev) for k in ("q", "q_pe", "kv", "k_pe")]
    o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    ta.mla_decode(*args, to_dev(m["indptr"], dev), scale, out=o, lse=lse)
    torch.cuda.synchronize()
    vals = [inputs.stored_values(m[k]) for k in ("q", "q_pe", "kv", "k_pe")]
    ro, rl = oracle.mla_decode(*vals, m["indptr"], scale)
    assert_bf16_parity(to_np(o), to_np(lse), ro, rl, f"random decode case {i} B={B} H={H} keys={n}")
    empty = lens == 0
    assert np.all(to_np(o)[empty] == 0) and np.all(np.isneginf(to_np(lse)[empty]))


@pytest.mark.parametrize("i", range(N_BIG_DECODE))
def test_random_decode_with_many_batches(ta, dev, i):
    # 900-1300 batches: both sides of the batch count at which the split plan
    # moves from the split workgroups into a kernel of its own; every output
    # written (NaN-prefilled), empty batches exact, eight batches against the
    # oracle one at a time
    rng = np.random.default_rng(15000 + i)
    B, H = int(rng.integers(900, 1301)), int(rng.integers(1, 129))
    lens = rng.integers(0, 400, size=B)
    lens[rng.random(B) < 0.15] = 0
    n = int(lens.sum())
    print(f"many-batch decode case {i}: B={B} H={H} keys={n}", flush=True)
    sig = np.float32(0.3)
    m = {"q": inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 512), dtype=np.float32) * sig),
         "q_pe": inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32) * sig),
         "kv": inputs.f32_to_bf16_bits(rng.standard_normal((n, 512), dtype=np.float32) * sig),
         "k_pe": inputs.f32_to_bf16_bits(rng.standard_normal((n, 64), dtype=np.float32) * sig)}
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = float(np.float32(576 ** -0.5))
    o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    ta.mla_decode(*(to_dev(m[k], dev) for k in ("q", "q_pe", "kv", "k_pe")), to_dev(indptr, dev), scale,
                  out=o, lse=lse)
    torch.cuda.synchronize()
    on, ln = to_np(o), to_np(lse)
    assert not np.isnan(on).any() and not np.isnan(ln).any(), f"case {i}: unwritten outputs"
    empty = lens == 0
    assert np.all(on[empty] == 0) and np.all(np.isneginf(ln[empty]))
    picks = sorted({0, B - 1, *(int(b) for b in rng.integers(0, B, size=6))})
    for b in picks:
        lo, hi = indptr[b], indptr[b + 1]
        ro, rl = oracle.mla_decode(*(inputs.stored_values(m[k][b:b + 1]) for k in ("q", "q_pe")),
                                   *(inputs.stored_values(m[k][lo:hi]) for k in ("kv", "k_pe")),
                                   np.array([0, hi - lo], np.int32), scale)
        assert_bf16_parity(on[b:b + 1], ln[b:b + 1], ro, rl, f"many-batch decode case {i} batch {b} ({hi - lo} keys)")


N_STREAMS_CASES = 2 * _SCALE


@pytest.mark.parametrize("i", range(N_STREAMS_CASES))
def test_random_decode_calls_over_many_streams(ta, dev, i):
    # 40 decode calls of random sizes spread over 10 streams (more than the
    # library's 8 workspace slots, so slots pass between streams and grow):
    # every result equals the same call made alone on the current stream, bit
    # for bit (the split depends only on the device, not on the stream)
    rng = np.random.default_rng(17000 + i)
    sig = np.float32(0.3)
    shapes = []
    for _ in range(6):
        B, H = int(rng.integers(1, 300)), int(rng.integers(1, 129))
        lens = rng.integers(0, 800, size=B)
        n = int(lens.sum())
        m = {"q": rng.standard_normal((B, H, 512), dtype=np.float32) * sig,
             "q_pe": rng.standard_normal((B, H, 64), dtype=np.float32) * sig,
             "kv": rng.standard_normal((n, 512), dtype=np.float32) * sig,
             "k_pe": rng.standard_normal((n, 64), dtype=np.float32) * sig}
        args = [to_dev(inputs.f32_to_bf16_bits(m[k]), dev) for k in ("q", "q_pe", "kv", "k_pe")]
        args.append(to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), dev))
        shapes.append((B, H, args))
    scale = float(np.float32(576 ** -0.5))
    refs = []
    for B, H, args in shapes:
        refs.append(ta.mla_decode(*args, scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(10)]
    calls = [(int(rng.integers(len(shapes))), int(rng.integers(len(streams)))) for _ in range(40)]
    outs = [(torch.empty((shapes[k][0], shapes[k][1], 512), dtype=torch.bfloat16, device=dev),
             torch.empty((shapes[k][0], shapes[k][1]), dtype=torch.float32, device=dev)) for k, _ in calls]
    torch.cuda.synchronize()
    for (k, s), (o, lse) in zip(calls, outs):
        ta.mla_decode(*shapes[k][2], scale, out=o, lse=lse, stream=streams[s])
    torch.cuda.synchronize()
    for j, ((k, s), (o, lse)) in enumerate(zip(calls, outs)):
        assert torch.equal(o, refs[k][0]) and torch.equal(lse, refs[k][1]), f"case {i} call {j} (shape {k}, stream {s})"
