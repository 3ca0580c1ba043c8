"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol the header declares, and rejects bad arguments before touching a
device. Without a GPU, a valid request returns TATTN_ERR_HIP."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tattn.h")


def _header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _header_symbols() == ["attn_fwd", "attn_fwd_ex", "attn_fwd_f32", "mla_decode", "mla_decode_noalloc",
                                 "ssd_scan", "tattn_status_str"]


def test_library_exports_every_declared_symbol(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    for sym in _header_symbols():
        assert sym in exported, sym
    lib = ctypes.CDLL(lib_path)
    for sym in _header_symbols():
        assert hasattr(lib, sym)


@pytest.fixture(scope="module")
def L(lib_path):
    from tiled_attention_12_amd import _binding
    return _binding.lib()


F = ctypes.c_float
OK, INVALID, UNSUP, ALIGN, OOM, HIP, SCRATCH = 0, -1, -2, -3, -4, -5, -6


def _mha(L, fn, q=16, k=16, v=16, o=16, lse=16, B=1, H=1, Sq=8, Skv=8, D=128, causal=0, scale=0.1):
    return getattr(L, fn)(q, k, v, o, lse, B, H, Sq, Skv, D, causal, F(scale), None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_mha_argument_validation(L, fn):
    assert _mha(L, fn, q=None) == INVALID
    assert _mha(L, fn, o=None) == INVALID
    assert _mha(L, fn, lse=None) == INVALID
    assert _mha(L, fn, k=None) == INVALID
    assert _mha(L, fn, B=-1) == INVALID
    assert _mha(L, fn, Skv=-3) == INVALID
    assert _mha(L, fn, causal=2) == INVALID
    assert _mha(L, fn, scale=float("nan")) == INVALID
    assert _mha(L, fn, scale=float("inf")) == INVALID
    assert _mha(L, fn, scale=0.0) == INVALID
    assert _mha(L, fn, scale=-0.5) == INVALID
    assert _mha(L, fn, D=96) == UNSUP
    assert _mha(L, fn, D=256) == UNSUP
    assert _mha(L, fn, q=24) == ALIGN
    assert _mha(L, fn, o=8) == ALIGN
    assert _mha(L, fn, lse=18) == ALIGN
    assert _mha(L, fn, Sq=(1 << 30) + 1) == UNSUP
    # nothing to do: OK without looking at pointers or the device
    assert _mha(L, fn, q=None, k=None, v=None, o=None, lse=None, B=0) == OK
    assert _mha(L, fn, q=None, k=None, v=None, o=None, lse=None, Sq=0) == OK
    # no keys: k and v may be null (the kernel writes O = 0, LSE = -inf)
    st = _mha(L, fn, k=None, v=None, Skv=0)
    assert st in (OK, HIP)


def test_mha_ex_argument_validation(L):
    def call(q=16, k=16, v=16, o=16, lse=16, B=1, H=4, Hkv=2, Sq=8, Skv=8, D=128, causal=0, window=0,
             mask=None, scale=0.1):
        return L.attn_fwd_ex(q, k, v, o, lse, B, H, Hkv, Sq, Skv, D, causal, window, mask, F(scale), None)
    assert call(Hkv=0) == INVALID
    assert call(Hkv=-1) == INVALID
    assert call(Hkv=3) == INVALID          # 4 query heads do not split into groups of 3 KV heads
    assert call(window=-1) == INVALID
    assert call(window=(1 << 30) + 1) == UNSUP
    assert call(q=None) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(D=80) == UNSUP
    assert call(k=40) == ALIGN
    assert call(B=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert call(H=0, Hkv=0, q=None) == OK


@pytest.mark.parametrize("fn", ["mla_decode", "mla_decode_noalloc"])
def test_mla_argument_validation(L, fn):
    def call(q=16, qpe=16, kv=16, kpe=16, o=16, lse=16, B=2, H=128, ind=16, scale=0.05):
        return getattr(L, fn)(q, qpe, kv, kpe, o, lse, B, H, ind, F(scale), None)
    assert call(q=None) == INVALID
    assert call(ind=None) == INVALID
    assert call(B=-1) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(H=0) == UNSUP
    assert call(H=129) == UNSUP
    assert call(kv=40) == ALIGN
    assert call(ind=2) == ALIGN
    assert call(B=0, q=None) == OK
    # no keys in any batch: kv and k_pe may be null (validation passes; on a
    # machine without a GPU the call then reports the missing device)
    assert call(kv=None, kpe=None) in (OK, HIP)


def test_ssd_argument_validation(L):
    def call(x=16, dt=4, A=4, B=16, C=16, y=16, s0=None, s1=None, Bt=2, Ls=100, H=8, G=1, P=64, N=128):
        return L.ssd_scan(x, dt, A, B, C, y, s0, s1, Bt, Ls, H, G, P, N, None)
    assert call(x=None) == INVALID
    assert call(A=None) == INVALID
    assert call(y=None) == INVALID
    assert call(Bt=-1) == INVALID
    assert call(Ls=-1) == INVALID
    assert call(G=0) == INVALID
    assert call(G=3) == INVALID            # 8 heads do not split into 3 groups
    assert call(P=128) == UNSUP
    assert call(N=64) == UNSUP
    assert call(x=24) == ALIGN
    assert call(B=8) == ALIGN
    assert call(dt=2) == ALIGN
    assert call(s0=32, s1=40) == ALIGN
    # final state overlapping the initial state
    assert call(s0=4096, s1=4096 + 64 * 128 * 4) == INVALID
    assert call(Bt=0, x=None, dt=None, A=None, B=None, C=None, y=None) == OK
    assert call(H=0, G=0, x=None) == OK
    # no steps and no final state: nothing to do
    assert call(Ls=0, x=None, dt=None, B=None, C=None, y=None) == OK


def test_valid_request_without_gpu_is_a_hip_error(lib_path):
    """Run in a child process that hides every GPU, so the answer is the
    no-device path on any host."""
    code = (
        "import ctypes,sys;"
        f"L=ctypes.CDLL({lib_path!r});"
        "F=ctypes.c_float;"
        "r1=L.attn_fwd(16,16,16,16,16,1,1,8,8,128,0,F(0.1),None);"
        "r2=L.attn_fwd_f32(16,16,16,16,16,1,1,8,8,64,1,F(0.1),None);"
        "r3=L.mla_decode(16,16,16,16,16,16,2,128,16,F(0.1),None);"
        "r4=L.attn_fwd_ex(16,16,16,16,16,1,4,1,8,8,128,1,3,None,F(0.1),None);"
        "r5=L.ssd_scan(16,16,16,16,16,16,None,None,1,64,2,1,64,128,None);"
        "r6=L.mla_decode_noalloc(16,16,16,16,16,16,2,128,16,F(0.1),None);"
        "print(r1,r2,r3,r4,r5,r6)"
    )
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == [str(HIP)] * 6


def test_status_strings_cover_every_code(L):
    from tiled_attention_12_amd import _binding
    seen = set()
    for code in (OK, INVALID, UNSUP, ALIGN, OOM, HIP, SCRATCH):
        s = _binding.status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert _binding.status_str(7) == "unknown status"


def test_binding_rejects_host_tensors(lib_path):
    import torch
    import tiled_attention_12_amd as ta
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ta.attn_fwd(x, x, x)


def test_binding_rejects_wrong_output_shapes_before_any_launch(lib_path):
    # an undersized out or lse would let the kernels write past the buffer:
    # the binding refuses it before it looks at devices or calls the library
    import torch
    import tiled_attention_12_amd as ta
    B, H, N = 2, 128, 10
    bf = torch.bfloat16
    q, qpe = torch.zeros(B, H, 512, dtype=bf), torch.zeros(B, H, 64, dtype=bf)
    kv, kpe = torch.zeros(N, 512, dtype=bf), torch.zeros(N, 64, dtype=bf)
    ind = torch.tensor([0, 4, N], dtype=torch.int32)
    for out, lse in ((torch.zeros(B, H - 1, 512, dtype=bf), None),
                     (torch.zeros(B, H, 256, dtype=bf), None),
                     (None, torch.zeros(B, H - 1)),
                     (None, torch.zeros(B * H))):
        with pytest.raises(ValueError, match="out must be"):
            ta.mla_decode(q, qpe, kv, kpe, ind, 0.05, out=out, lse=lse)
    x = torch.zeros(1, 2, 8, 64, dtype=bf)
    for out, lse in ((torch.zeros(1, 2, 7, 64, dtype=bf), None), (None, torch.zeros(1, 2, 7))):
        with pytest.raises(ValueError):
            ta.attn_fwd(x, x, x, out=out, lse=lse)
