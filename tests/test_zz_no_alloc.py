"""mla_decode_noalloc (the entry point with the library's static workspace)
against mla_decode on the GPU, through the C ABI.

Two calls in a row, the second with a smaller input, each compared bit for
bit with mla_decode on the same inputs (same kernels, so the results must be
identical) and with the CPU oracle under the bf16 limits; a request whose
workspace exceeds the static array is refused before any launch and leaves
the output untouched.
"""

import ctypes

import numpy as np
import pytest

import oracle
from tests.helpers import assert_bf16_parity, to_dev, to_np
from tiled_attention_12_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCALE = float(np.float32(576 ** -0.5))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def L(lib_path):
    from tiled_attention_12_amd import _binding
    return _binding.lib()


def _call(L, fn, args, o, lse, B, H):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in args]
    return getattr(L, fn)(*ptrs[:4], ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), B, H,
                          ptrs[4], ctypes.c_float(SCALE), stream)


def _case(dev, B, H, seed, **kw):
    m = inputs.mla_inputs(B, H, seed=seed, **kw)
    args = [to_dev(m[n], dev) for n in ("q", "q_pe", "kv", "k_pe", "indptr")]
    return m, args


def test_noalloc_matches_mla_decode_on_two_calls(L, dev):
    for B, H, seed, kw in ((64, 128, 501, {"kv_len": 4096}), (3, 64, 502, {"kv_len_range": (1, 700)})):
        print(f"noalloc B={B} H={H} {kw}", flush=True)
        m, args = _case(dev, B, H, seed, **kw)
        o_ref = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        l_ref = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        assert _call(L, "mla_decode", args, o_ref, l_ref, B, H) == 0
        assert _call(L, "mla_decode_noalloc", args, o, lse, B, H) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        ro, rl = oracle.mla_decode(*(inputs.stored_values(m[n]) for n in ("q", "q_pe", "kv", "k_pe")),
                                   m["indptr"], SCALE)
        assert_bf16_parity(to_np(o), to_np(lse), ro, rl, f"noalloc B={B} H={H}")


def test_noalloc_refuses_a_workspace_above_its_array(L, dev):
    # (CUs + B) * 128 * 1028 bytes above 64 MiB: about 250 batches at H = 128
    B, H = 1000, 128
    m, args = _case(dev, B, H, 503, kv_len=1)
    o = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=dev)
    assert _call(L, "mla_decode_noalloc", args, o, lse, B, H) == -6
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0)) and bool(torch.all(lse == 7.0))
