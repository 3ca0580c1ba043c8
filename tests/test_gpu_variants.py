"""GPU parity of attn_fwd_ex (grouped/single KV heads, sliding window, block
mask) against the CPU float64 oracle (needs gfx950).

Element by element at sizes the oracle finishes quickly (several 256-row
query tiles, several 64-key tiles and ragged tails), and on sampled rows at
the full variant workloads the benchmark times.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import assert_bf16_parity, to_dev, to_np
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


@pytest.fixture(params=[4, 8], ids=["waves4", "waves8"])
def dense_waves(request, monkeypatch):
    """Forces the dense prefill's workgroup shape (grouped heads without a
    window or mask take the dense path)."""
    monkeypatch.setenv("TATTN_MHA_WAVES", str(request.param))
    return request.param


def _vals(x, names):
    return [inputs.stored_values(x[n]) for n in names]


def _run(ta, dev, x, causal, scale, window=0, mask=None):
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    m = None if mask is None else torch.from_numpy(mask).to(dev)
    o, lse = ta.attn_fwd_ex(q, k, v, causal=causal, scale=scale, window=window, block_mask=m)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hkv", [1, 2, 4, 8])
@pytest.mark.parametrize("sq,skv", [(130, 130), (65, 300), (300, 65)])
def test_grouped_kv_heads(ta, dev, D, causal, Hkv, sq, skv, dense_waves):
    x = inputs.mha_inputs(2, 8, sq, skv, D, seed=900 + Hkv + sq + D, Hkv=Hkv)
    scale = float(np.float32(D ** -0.5))
    o, lse = _run(ta, dev, x, causal, scale)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), scale, causal=causal)
    assert_bf16_parity(o, lse, ro, rl, f"gqa Hkv={Hkv} D={D} causal={causal} {sq}x{skv}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [1, 31, 64, 100, 300])
@pytest.mark.parametrize("sq,skv", [(300, 300), (200, 457), (457, 200)])
def test_sliding_window(ta, dev, D, causal, W, sq, skv):
    x = inputs.mha_inputs(1, 3, sq, skv, D, seed=950 + W + sq + D + int(causal))
    scale = float(np.float32(D ** -0.5))
    o, lse = _run(ta, dev, x, causal, scale, window=W)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), scale, causal=causal, window=W)
    assert_bf16_parity(o, lse, ro, rl, f"window W={W} D={D} causal={causal} {sq}x{skv}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [385, 900])
def test_wide_sliding_window(ta, dev, D, causal, W):
    # wider than 768 visible keys per row (non-causal 2W, causal W + 1) or
    # not: both workgroup shapes of the window walk, with ragged tails
    x = inputs.mha_inputs(1, 3, 1300, 1250, D, seed=960 + W + D + int(causal))
    scale = float(np.float32(D ** -0.5))
    o, lse = _run(ta, dev, x, causal, scale, window=W)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), scale, causal=causal, window=W)
    assert_bf16_parity(o, lse, ro, rl, f"wide window W={W} D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_narrow_window_more_items_than_workgroup_slots(ta, dev, D, causal):
    # 4*16 heads of eighteen 128-row query tiles (the last one ragged): 1152
    # work items, more than the persistent grid has workgroups (four per
    # compute unit at head width 64, three at 128), in the XCD order. Outputs
    # are prefilled with NaN so an item that no workgroup wrote fails; every
    # element is checked.
    x = inputs.mha_inputs(4, 16, 2200, 2200, D, seed=995 + D + int(causal))
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(D ** -0.5))
    ta.attn_fwd_ex(q, k, v, causal=causal, scale=scale, window=100, out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = to_np(out), to_np(lse)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), scale, causal=causal, window=100)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    assert_bf16_parity(o, l, ro, rl, f"narrow window many items D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.3, 0.7])
@pytest.mark.parametrize("sq,skv", [(257, 300), (600, 600), (100, 700)])
def test_block_mask(ta, dev, D, causal, density, sq, skv):
    x = inputs.mha_inputs(2, 2, sq, skv, D, seed=980 + sq + int(10 * density))
    mask = inputs.block_mask(2, 2, sq, skv, density, seed=981 + sq)
    o, lse = _run(ta, dev, x, causal, 0.088, mask=mask)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), 0.088, causal=causal, block_mask=mask)
    # rows whose every visible key block is masked: O = 0, LSE = -inf on both sides
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    assert np.all(o[np.isneginf(rl)] == 0)
    assert_bf16_parity(o, lse, ro, rl, f"block mask d={density} causal={causal} {sq}x{skv}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_grouped_heads_and_more_items_than_one_pass(ta, dev, D, causal):
    # 4*16 heads of eighteen 128-row query tiles each (the last one ragged):
    # 1152 work items, more than the persistent grid has workgroups (three or
    # four per compute unit), in the XCD order (heads a multiple of 8), 4
    # query heads per KV head
    x = inputs.mha_inputs(4, 16, 2200, 1000, D, seed=985 + D, Hkv=4)
    mask = inputs.block_mask(4, 16, 2200, 1000, 0.4, seed=986)
    o, lse = _run(ta, dev, x, causal, 0.088, mask=mask)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), 0.088, causal=causal, block_mask=mask)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    assert_bf16_parity(o, lse, ro, rl, f"block mask gqa many items causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [150, 800])
def test_all_variants_together(ta, dev, causal, W):
    x = inputs.mha_inputs(2, 6, 520, 610, 128, seed=990, Hkv=2)
    mask = inputs.block_mask(2, 6, 520, 610, 0.6, seed=991)
    o, lse = _run(ta, dev, x, causal, 0.09, window=W, mask=mask)
    ro, rl = oracle.attention_masked(*_vals(x, "qkv"), 0.09, causal=causal, window=W, block_mask=mask)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    assert_bf16_parity(o, lse, ro, rl, f"gqa+window W={W}+mask causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("jump", [24.0, 200.0, -200.0])
def test_window_and_mask_score_jumps(ta, dev, D, jump):
    # the window/mask walk takes the exact step on every tile (tile max,
    # raise past the threshold, O rescale): from key 640 on one query/key
    # dimension adds `jump` base-2 units to every score, under a window and
    # under a block mask
    B, H, S = 1, 2, 1000
    x = inputs.mha_inputs(B, H, S, S, D, seed=46)
    q = inputs.stored_values(x["q"]).copy()
    k = inputs.stored_values(x["k"]).copy()
    scale = float(np.float32(D ** -0.5))
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[..., 640:, 0] = jump * np.log(2.0) / scale
    y = dict(x, q=inputs.f32_to_bf16_bits(q), k=inputs.f32_to_bf16_bits(k))
    mask = inputs.block_mask(B, H, S, S, 0.7, seed=47)
    for causal in (False, True):
        for window, m in ((300, None), (0, mask)):
            o, lse = _run(ta, dev, y, causal, scale, window=window, mask=m)
            ro, rl = oracle.attention_masked(*_vals(y, "qkv"), scale, causal=causal, window=window,
                                             block_mask=m)
            assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
            assert_bf16_parity(o, lse, ro, rl, f"jump {jump} D={D} causal={causal} W={window} mask={m is not None}")


def test_masked_out_everything(ta, dev):
    x = inputs.mha_inputs(1, 2, 130, 200, 64, seed=992)
    mask = np.zeros((1, 2, 3, 4), np.uint8)
    o, lse = _run(ta, dev, x, False, 0.125, mask=mask)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_plain_call_is_bitwise_attn_fwd(ta, dev):
    # Hkv == H, no window, no mask: the same kernel path as attn_fwd
    x = inputs.mha_inputs(2, 4, 333, 333, 128, seed=993)
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    for causal in (False, True):
        o1, l1 = ta.attn_fwd(q, k, v, causal=causal, scale=0.09)
        o2, l2 = ta.attn_fwd_ex(q, k, v, causal=causal, scale=0.09)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_grouped_heads_are_bitwise_repeated_heads(ta, dev):
    # a KV head shared by a group gives exactly what attn_fwd gives on the
    # KV head repeated for every query head of the group
    x = inputs.mha_inputs(2, 8, 300, 300, 128, seed=994, Hkv=2)
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o1, l1 = ta.attn_fwd_ex(q, k, v, causal=True, scale=0.09)
    o2, l2 = ta.attn_fwd(q, kr, vr, causal=True, scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _sampled(ta, dev, name, causal, window=0, density=None, n_rows=48):
    w = WORKLOADS[name]
    x = inputs.mha_inputs(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], seed=w["seed"], sigma=w["sigma"],
                          Hkv=w.get("Hkv"))
    mask = None
    if density is not None:
        mask = inputs.block_mask(w["B"], w["H"], w["Sq"], w["Skv"], density, seed=w["seed"] + 100)
    o, lse = _run(ta, dev, x, causal, w["scale"], window=window, mask=mask)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w["Sq"] - 1], rng.integers(0, w["Sq"], n_rows)]))
    q, k, v = _vals(x, "qkv")
    for b in range(w["B"]):
        hs = [0, w["H"] - 1]
        for h in hs:
            kv_h = h // (w["H"] // w.get("Hkv", w["H"]))
            bm = None if mask is None else mask[b:b + 1, h:h + 1]
            ro, rl = oracle.attention_masked(q[b:b + 1, h:h + 1], k[b:b + 1, kv_h:kv_h + 1], v[b:b + 1, kv_h:kv_h + 1],
                                             w["scale"], causal=causal, window=window, block_mask=bm, rows=rows)
            assert_bf16_parity(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], ro, rl,
                               f"{name} b={b} h={h}")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_workload_sampled(ta, dev, causal):
    _sampled(ta, dev, "mha_gqa_bf16", causal)


def test_window_workload_sampled(ta, dev):
    w = WORKLOADS["mha_window_bf16"]
    _sampled(ta, dev, "mha_window_bf16", True, window=w["window"])


def test_blocksparse_workload_sampled(ta, dev):
    w = WORKLOADS["mha_blocksparse_bf16"]
    _sampled(ta, dev, "mha_blocksparse_bf16", False, density=w["density"])
