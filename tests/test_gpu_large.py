"""Tensors past 4 GiB: the prefill's K/V, its Q/O, the decode's latent key
rows and the scan's x/y each span more than 2^32 bytes, so byte offsets past
2^31 and 2^32 are exercised (needs gfx950 and ~20 GB of device memory).

Only a few heads carry seeded random data (the first, a middle and the last,
whose data sits past 4 GiB); the others are zero, which gives outputs with a
closed form (uniform softmax: O = the mean of V, LSE = ln(keys); zero keys
and values: O = 0; a zero scan input: y = 0). Outputs start as NaN, so an element no workgroup wrote fails.
The random heads are compared with the float64 oracle.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.ssd as ossd
from tests.helpers import assert_bf16_parity, to_np
from tests.ssd_bounds import check_head, head_scales
from tiled_attention_12_amd import inputs

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


def _bf16(rng, shape):
    """Seeded standard normals as bf16 bits (uint16) and their exact values."""
    bits = inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return bits, inputs.stored_values(bits)


def _put(t, index, bits):
    t[index] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(t.device)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_keys_and_values_past_4_gib(ta, dev, causal):
    # K and V of 128 heads x 2^18 keys x 128: 8 GiB each; the last head's rows
    # start 7.9 GiB in
    B, H, Sq, Skv, D = 1, 128, 32, 1 << 18, 128
    print(f"large K/V: B={B} H={H} Sq={Sq} Skv={Skv} D={D} causal={causal}", flush=True)
    rng = np.random.default_rng(9100)
    qb, qv = _bf16(rng, (B, H, Sq, D))
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.zeros((B, H, Skv, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    heads = [0, 77, H - 1]
    kv = {}
    for h in heads:
        kb, kvals = _bf16(rng, (Skv, D))
        vb, vvals = _bf16(rng, (Skv, D))
        _put(k, (0, h), kb)
        _put(v, (0, h), vb)
        kv[h] = (kvals, vvals)
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(D ** -0.5))
    ta.attn_fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    on, ln = to_np(o), to_np(lse)
    for h in heads:
        ro, rl = oracle.attention(qv[:, h:h + 1], kv[h][0][None, None], kv[h][1][None, None], scale, causal=causal)
        assert_bf16_parity(on[:, h:h + 1], ln[:, h:h + 1], ro, rl, f"large K/V head {h}")
    # zero heads: a uniform softmax over the keys each row sees, V = 0
    zero = [h for h in range(H) if h not in heads]
    visible = np.arange(Sq) + Skv - Sq + 1 if causal else np.full(Sq, Skv)  # bottom-right aligned
    assert np.all(on[:, zero] == 0.0)
    np.testing.assert_allclose(ln[:, zero], np.broadcast_to(np.log(visible), ln[:, zero].shape), atol=1e-5)
    del k, v, o
    torch.cuda.empty_cache()


def test_prefill_queries_and_outputs_past_4_gib(ta, dev):
    # Q and O of 128 heads x 2^18 rows x 128: 8 GiB each, 96 keys per head
    # (a full tile and a ragged one); rows sampled at both ends and between
    B, H, Sq, Skv, D = 1, 128, 1 << 18, 96, 128
    print(f"large Q/O: B={B} H={H} Sq={Sq} Skv={Skv} D={D}", flush=True)
    rng = np.random.default_rng(9200)
    q = torch.zeros((B, H, Sq, D), dtype=torch.bfloat16, device=dev)
    kb, kvals = _bf16(rng, (B, H, Skv, D))
    vb, vvals = _bf16(rng, (B, H, Skv, D))
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    v = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(dev)
    heads = [0, 50, H - 1]
    rows = np.concatenate([np.arange(64), np.sort(rng.choice(Sq - 128, 64, replace=False)) + 64,
                           np.arange(Sq - 64, Sq)])
    qvals = {}
    for h in heads:
        qb_h, qv_h = _bf16(rng, (Sq, D))
        _put(q, (0, h), qb_h)
        qvals[h] = qv_h[rows]
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(D ** -0.5))
    ta.attn_fwd(q, k, v, causal=False, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    ridx = torch.from_numpy(rows).to(dev)
    for h in heads:
        got_o, got_l = to_np(o[0, h].index_select(0, ridx)), to_np(lse[0, h].index_select(0, ridx))
        ro, rl = oracle.attention(qvals[h][None, None], kvals[:, h:h + 1], vvals[:, h:h + 1], scale)
        assert_bf16_parity(got_o[None, None], got_l[None, None], ro, rl, f"large Q/O head {h}")
    # zero queries: O = the mean of the head's V rows, LSE = ln(Skv)
    for h in (1, 64, H - 2):
        got_o, got_l = to_np(o[0, h].index_select(0, ridx)), to_np(lse[0, h].index_select(0, ridx))
        mean_v = vvals[0, h].mean(axis=0)
        assert np.abs(got_o - mean_v[None]).max() <= 1e-2, h
        assert np.abs(got_l - math.log(Skv)).max() <= 1e-5, h
    del q, o
    torch.cuda.empty_cache()


def test_scan_inputs_and_outputs_past_4_gib(ta, dev):
    # x and y of one batch x 2^16 steps x 512 heads x 64: 4 GiB each; the last
    # head's elements end at the last byte
    Bt, L, H, G, P, N = 1, 1 << 16, 512, 1, 64, 128
    print(f"large scan: Bt={Bt} L={L} H={H} G={G}", flush=True)
    d = inputs.ssd_inputs(Bt, L, 2, G, P, N, seed=9301)   # B, C, dt and two heads' x and A
    x = torch.zeros((Bt, L, H, P), dtype=torch.bfloat16, device=dev)
    heads = [0, H - 1]
    for i, h in enumerate(heads):
        _put(x, (0, slice(None), h), d["x"][0, :, i])
    dt = torch.from_numpy(np.ascontiguousarray(
        np.broadcast_to(d["dt"][:, :, :1], (Bt, L, H)))).to(dev)
    dt[0, :, H - 1] = torch.from_numpy(d["dt"][0, :, 1]).to(dev)
    A = torch.full((H,), float(d["A"][0]), dtype=torch.float32, device=dev)
    A[H - 1] = float(d["A"][1])
    Bm = torch.from_numpy(d["B"].view(np.int16)).view(torch.bfloat16).to(dev)
    Cm = torch.from_numpy(d["C"].view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.full((Bt, L, H, P), float("nan"), dtype=torch.bfloat16, device=dev)
    ta.ssd_scan(x, dt, A, Bm, Cm, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item()
    xs, Bs, Cs = (inputs.stored_values(d[n]) for n in ("x", "B", "C"))
    for i, h in enumerate(heads):
        ry, _ = ossd.ssd_recurrence(xs[:, :, i:i + 1], d["dt"][:, :, i:i + 1], d["A"][i:i + 1], Bs, Cs)
        sc = head_scales(xs[0, :, i], d["dt"][0, :, i].astype(np.float64), d["A"][i], Bs[0, :, 0], Cs[0, :, 0])
        check_head(to_np(y[0, :, h]), ry[0, :, 0], sc, f"large scan head {h}")
    # zero inputs give zero outputs
    assert not torch.count_nonzero(y[0, :, 1:H - 1]).item()
    del x, y
    torch.cuda.empty_cache()


def test_mla_key_rows_past_4_gib(ta, dev):
    # 80 batches x 65,536 keys: 5.4 GB of latent rows (the last batch's start
    # 5.0 GiB in) and 0.7 GB of rotary rows; batches 0, 41 and 79 random, the
    # rest zero (O = 0, LSE = ln(keys))
    B, H, n = 80, 128, 1 << 16
    print(f"large MLA: B={B} H={H} keys per batch={n}", flush=True)
    rng = np.random.default_rng(9400)
    sig = np.float32(0.3)
    qb = inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 512), dtype=np.float32) * sig)
    qpb = inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32) * sig)
    kv = torch.zeros((B * n, 512), dtype=torch.bfloat16, device=dev)
    kpe = torch.zeros((B * n, 64), dtype=torch.bfloat16, device=dev)
    rows = {}
    for b in (0, 41, B - 1):
        kvb = inputs.f32_to_bf16_bits(rng.standard_normal((n, 512), dtype=np.float32) * sig)
        kpb = inputs.f32_to_bf16_bits(rng.standard_normal((n, 64), dtype=np.float32) * sig)
        _put(kv, slice(b * n, (b + 1) * n), kvb)
        _put(kpe, slice(b * n, (b + 1) * n), kpb)
        rows[b] = (inputs.stored_values(kvb), inputs.stored_values(kpb))
    indptr = torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=dev)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
    qpe = torch.from_numpy(qpb.view(np.int16)).view(torch.bfloat16).to(dev)
    o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    scale = float(np.float32(576 ** -0.5))
    ta.mla_decode(q, qpe, kv, kpe, indptr, scale, out=o, lse=lse)
    torch.cuda.synchronize()
    on, ln = to_np(o), to_np(lse)
    assert not np.isnan(on).any() and not np.isnan(ln).any()
    qv, qpv = inputs.stored_values(qb), inputs.stored_values(qpb)
    for b, (kvv, kpv) in rows.items():
        ro, rl = oracle.mla_decode(qv[b:b + 1], qpv[b:b + 1], kvv, kpv, np.array([0, n], np.int32), scale)
        assert_bf16_parity(on[b:b + 1], ln[b:b + 1], ro, rl, f"large MLA batch {b}")
    zero = [b for b in range(B) if b not in rows]
    assert np.all(on[zero] == 0.0)
    assert np.abs(ln[zero] - math.log(n)).max() <= 1e-5
    del kv, kpe
    torch.cuda.empty_cache()
