"""HIP graph capture of the attention entry points that allocate nothing
(attn_fwd, attn_fwd_ex, mla_decode_noalloc), on gfx950.

The graph is replayed several times with eager work and synchronisations in
between, on new inputs copied into the captured buffers, and every replay
must equal the eager call bit for bit.
"""

import os

import numpy as np
import pytest

from tests.helpers import to_dev
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


def _capture_and_replay(dev, call, bufs, new_inputs):
    """call(bufs) -> (o, lse) writes into preallocated outputs; new_inputs is a
    list of input dicts copied into bufs before each replay."""
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call(bufs)  # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call(bufs)
    for x in new_inputs:
        for k, v in x.items():
            bufs[k].copy_(v)
        g.replay()
        torch.cuda.synchronize()
        got = tuple(t.clone() for t in out)
        # eager reference on separate buffers, with other work in between
        junk = torch.randn(1 << 20, device=dev).sum()
        ref = call({k: v.clone() for k, v in bufs.items()}, fresh=True)
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


@pytest.mark.parametrize("causal", [False, True])
def test_attn_fwd_in_a_graph(ta, dev, causal):
    B, H, S, D = 2, 8, 300, 128
    xs = [inputs.mha_inputs(B, H, S, S, D, seed=1200 + i) for i in range(3)]
    bufs = {n: to_dev(xs[0][n], dev) for n in "qkv"}
    o = torch.empty_like(bufs["q"])
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)

    def call(b, fresh=False):
        if fresh:
            return ta.attn_fwd(b["q"], b["k"], b["v"], causal=causal, scale=0.09)
        return ta.attn_fwd(b["q"], b["k"], b["v"], causal=causal, scale=0.09, out=o, lse=lse)

    _capture_and_replay(dev, call, bufs, [{n: to_dev(x[n], dev) for n in "qkv"} for x in xs[1:] + xs[:1]])


def test_attn_fwd_ex_in_a_graph(ta, dev):
    B, H, Hkv, S, D = 1, 8, 2, 700, 128
    xs = [inputs.mha_inputs(B, H, S, S, D, seed=1300 + i, Hkv=Hkv) for i in range(3)]
    mask = torch.from_numpy(inputs.block_mask(B, H, S, S, 0.6, seed=1310)).to(dev)
    bufs = {n: to_dev(xs[0][n], dev) for n in "qkv"}
    o = torch.empty_like(bufs["q"])
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)

    def call(b, fresh=False):
        kw = dict(causal=True, scale=0.09, window=200, block_mask=mask)
        if fresh:
            return ta.attn_fwd_ex(b["q"], b["k"], b["v"], **kw)
        return ta.attn_fwd_ex(b["q"], b["k"], b["v"], out=o, lse=lse, **kw)

    _capture_and_replay(dev, call, bufs, [{n: to_dev(x[n], dev) for n in "qkv"} for x in xs[1:] + xs[:1]])


def test_mla_decode_noalloc_in_a_graph(ta, dev):
    # the decode without allocations (its workspace is the library's static
    # array) captured once and replayed on new inputs of the same shapes; the
    # eager reference is mla_decode with its own workspace, same kernels
    lens = [700, 33, 0, 2500]
    B, H = len(lens), 128
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(indptr[-1])
    xs = []
    for i in range(3):
        m = inputs.mla_inputs(B, H, seed=1400 + i, kv_len=1)
        g = np.random.default_rng(1410 + i)
        m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
        m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
        xs.append({k: to_dev(m[k], dev) for k in ("q", "q_pe", "kv", "k_pe")})
    ind = to_dev(indptr, dev)
    bufs = {k: v.clone() for k, v in xs[0].items()}
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    scale = float(np.float32(576 ** -0.5))

    def call(b, fresh=False):
        if fresh:
            return ta.mla_decode(b["q"], b["q_pe"], b["kv"], b["k_pe"], ind, scale)
        return ta.mla_decode_noalloc(b["q"], b["q_pe"], b["kv"], b["k_pe"], ind, scale, out=o, lse=lse)

    _capture_and_replay(dev, call, bufs, xs[1:] + xs[:1])


_N_RANDOM = 6 * max(1, int(os.environ.get("TATTN_RANDOM_SCALE", "1")))


@pytest.mark.parametrize("i", range(_N_RANDOM))
def test_random_entry_point_in_a_graph(ta, dev, i):
    # a seeded random entry point and shape, captured and replayed as above
    rng = np.random.default_rng(18000 + i)
    kind = ("attn_fwd", "attn_fwd_ex", "mla_decode_noalloc")[i % 3]
    if kind == "mla_decode_noalloc":
        B, H = int(rng.integers(1, 60)), int(rng.integers(1, 129))
        lens = rng.integers(0, 1500, size=B)
        indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        n = int(indptr[-1])
        xs = []
        for r in range(3):
            g = np.random.default_rng(18500 + 10 * i + r)
            xs.append({k: to_dev(inputs.f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(0.3)),
                                 dev)
                       for k, shape in (("q", (B, H, 512)), ("q_pe", (B, H, 64)), ("kv", (n, 512)),
                                        ("k_pe", (n, 64)))})
        ind = to_dev(indptr, dev)
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        scale = float(np.float32(576 ** -0.5))

        def call(b, fresh=False):
            if fresh:
                return ta.mla_decode(b["q"], b["q_pe"], b["kv"], b["k_pe"], ind, scale)
            return ta.mla_decode_noalloc(b["q"], b["q_pe"], b["kv"], b["k_pe"], ind, scale, out=o, lse=lse)
    else:
        hkv = int(rng.choice([1, 2, 4]))
        B, H = int(rng.integers(1, 4)), hkv * int(rng.choice([1, 2, 4]))
        Sq, Skv, D = int(rng.integers(1, 900)), int(rng.integers(1, 900)), int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        if kind == "attn_fwd":
            hkv = H
        window = int(rng.integers(1, 500)) if kind == "attn_fwd_ex" and rng.random() < 0.5 else 0
        mask = (torch.from_numpy(inputs.block_mask(B, H, Sq, Skv, 0.6, seed=18600 + i)).to(dev)
                if kind == "attn_fwd_ex" and rng.random() < 0.5 else None)
        xs = [{n: to_dev(inputs.mha_inputs(B, H, Sq, Skv, D, seed=18700 + 10 * i + r, Hkv=hkv)[n], dev)
               for n in "qkv"} for r in range(3)]
        o = torch.empty_like(xs[0]["q"])
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        kw = dict(causal=causal, scale=0.09)
        if kind == "attn_fwd_ex":
            kw.update(window=window, block_mask=mask)
        fn = getattr(ta, kind)

        def call(b, fresh=False):
            if fresh:
                return fn(b["q"], b["k"], b["v"], **kw)
            return fn(b["q"], b["k"], b["v"], out=o, lse=lse, **kw)
    print(f"graph case {i}: {kind}", flush=True)
    bufs = {k: v.clone() for k, v in xs[0].items()}
    _capture_and_replay(dev, call, bufs, xs[1:] + xs[:1])
