"""The five benchmark configurations against the CPU float64 oracle, every
output element, under the plain limits (needs gfx950).

Outputs are NaN-filled device buffers before each call, so a work item the
persistent grid skipped leaves NaN behind and fails. Limits: bf16
max|dO| <= 1e-2, mean|dO| <= 1e-3, max|dLSE| <= 1e-3 (plus a relative-L2
gate of 1e-2 on O); fp32 max|dO| <= 1e-5, max|dLSE| <= 1e-5. The launch
configuration is the one the benchmark times (same entry points, shapes and
seeds).
"""

import numpy as np
import pytest

import oracle
from tests.helpers import assert_config_parity, nan_like, to_dev, to_np
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


def _mha(ta, dev, w, causal, fp32=False):
    x = inputs.mha_inputs(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], seed=w["seed"], sigma=w["sigma"],
                          dtype="f32" if fp32 else "bf16")
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    out = nan_like(tuple(q.shape), q.dtype, dev)
    lse = nan_like((w["B"], w["H"], w["Sq"]), torch.float32, dev)
    fn = ta.attn_fwd_f32 if fp32 else ta.attn_fwd
    fn(q, k, v, causal=causal, scale=w["scale"], out=out, lse=lse)
    torch.cuda.synchronize()
    return x, to_np(out), to_np(lse)


def test_config1_tiny_fp32(ta, dev):
    w = WORKLOADS["mha_tiny_f32"]
    print(f"config 1 {w}", flush=True)
    x, o, lse = _mha(ta, dev, w, False, fp32=True)
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], w["scale"])
    print("config 1", assert_config_parity(o, lse, ro, rl, "config 1", fp32=True))


@pytest.mark.parametrize("causal", [False, True])
def test_config2_prefill_every_element(ta, dev, causal):
    w = WORKLOADS["mha_prefill_bf16"]
    print(f"config 2 causal={causal}", flush=True)
    x, o, lse = _mha(ta, dev, w, causal)
    ro, rl = oracle.attention(*(inputs.stored_values(x[n]) for n in "qkv"), w["scale"], causal=causal)
    print("config 2", causal, assert_config_parity(o, lse, ro, rl, f"config 2 causal={causal}"))


def test_config3_long_causal_eight_full_heads(ta, dev):
    # every output of every head must be written (finite); eight whole heads
    # (first, last and six drawn) are compared element by element
    w = WORKLOADS["mha_long_causal_bf16"]
    print("config 3", flush=True)
    x, o, lse = _mha(ta, dev, w, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(31)
    heads = sorted({0, w["H"] - 1, *(int(h) for h in rng.choice(np.arange(1, w["H"] - 1), 6, replace=False))})
    assert len(heads) == 8
    for h in heads:
        sl = lambda n: inputs.stored_values(x[n][:, h:h + 1])
        ro, rl = oracle.attention(sl("q"), sl("k"), sl("v"), w["scale"], causal=True)
        st = assert_config_parity(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"config 3 head {h}")
        print("config 3 head", h, st, flush=True)


def _mla(ta, dev, name):
    w = WORKLOADS[name]
    kw = {"kv_len": w["kv_len"]} if "kv_len" in w else {"kv_len_range": w["kv_len_range"]}
    m = inputs.mla_inputs(w["B"], w["H"], seed=w["seed"], sigma=w["sigma"], **kw)
    args = [to_dev(m[n], dev) for n in ("q", "q_pe", "kv", "k_pe")]
    out = nan_like((w["B"], w["H"], 512), torch.bfloat16, dev)
    lse = nan_like((w["B"], w["H"]), torch.float32, dev)
    ta.mla_decode(*args, to_dev(m["indptr"], dev), w["scale"], out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(*(inputs.stored_values(m[n]) for n in ("q", "q_pe", "kv", "k_pe")),
                               m["indptr"], w["scale"])
    return to_np(out), to_np(lse), ro, rl


def test_config4_mla_decode_every_element(ta, dev):
    print("config 4", flush=True)
    o, lse, ro, rl = _mla(ta, dev, "mla_decode_bf16")
    print("config 4", assert_config_parity(o, lse, ro, rl, "config 4"))


def test_config5_ragged_mla_decode_every_element(ta, dev):
    print("config 5", flush=True)
    o, lse, ro, rl = _mla(ta, dev, "mla_decode_ragged_bf16")
    print("config 5", assert_config_parity(o, lse, ro, rl, "config 5"))
