"""ctypes binding of libtattn.so: argument marshalling only.

Every function here checks dtypes, devices, shapes and contiguity of torch
tensors, allocates outputs with torch, and passes raw device pointers plus
the HIP stream (the caller's, else the device's current one) to the C ABI,
with the tensors' device made current for the call. All arithmetic runs in the library's
gfx950 kernels; if the library is missing, loading this module fails.
"""

import ctypes
import math
import os

from ._build import library_path

TATTN_OK = 0
TATTN_ERR_INVALID_ARG = -1
TATTN_ERR_UNSUPPORTED = -2
TATTN_ERR_ALIGN = -3
TATTN_ERR_OOM = -4
TATTN_ERR_HIP = -5
TATTN_ERR_SCRATCH = -6

EXPORTED = ("attn_fwd", "attn_fwd_ex", "attn_fwd_f32", "mla_decode", "mla_decode_noalloc", "ssd_scan",
            "tattn_status_str")


class TattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m tiled_attention_12_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    mha = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.attn_fwd.argtypes = mha
    lib.attn_fwd.restype = i32
    lib.attn_fwd_f32.argtypes = mha
    lib.attn_fwd_f32.restype = i32
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, f32, vp]
    lib.attn_fwd_ex.restype = i32
    for fn in (lib.mla_decode, lib.mla_decode_noalloc):
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, f32, vp]
        fn.restype = i32
    lib.ssd_scan.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.ssd_scan.restype = i32
    lib.tattn_status_str.argtypes = [i32]
    lib.tattn_status_str.restype = ctypes.c_char_p
    return lib


_LIB = _load()


def lib():
    """The loaded ctypes library (raw C ABI)."""
    return _LIB


def status_str(status):
    return _LIB.tattn_status_str(int(status)).decode()


def _torch():
    import torch
    return torch


def _launch(fn, device, stream, *args):
    """Calls fn(*args, stream handle) with the tensors' device current: the
    library launches on the current device, so tensors on another device
    than the current one are handled by switching to theirs for the call."""
    torch = _torch()
    if stream is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    with torch.cuda.device(device):
        s = torch.cuda.current_stream(device) if stream is None else stream
        return fn(*args, ctypes.c_void_p(s.cuda_stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _check_dev(name, t, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a ROCm device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mha(fn_name, q, k, v, causal, scale, out, lse, stream, dtype):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    _check_dev("out", out, dtype, dev)
    _check_dev("lse", lse, torch.float32, dev)
    if tuple(out.shape) != (B, H, Sq, D) or tuple(lse.shape) != (B, H, Sq):
        raise ValueError("out/lse have the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _launch(getattr(_LIB, fn_name), dev, stream, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq,
                 Skv, D, int(bool(causal)), ctypes.c_float(scale))
    if rc != TATTN_OK:
        raise TattnError(rc, fn_name)
    return out, lse


def attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """bf16 multi-head attention forward: returns (O bf16 [B,H,Sq,D], LSE fp32 [B,H,Sq])."""
    return _mha("attn_fwd", q, k, v, causal, scale, out, lse, stream, _torch().bfloat16)


def attn_fwd_ex(q, k, v, causal=False, scale=None, window=0, block_mask=None, out=None, lse=None,
                stream=None):
    """bf16 attention with grouped KV heads (k, v [B, Hkv, Skv, D]), an optional
    key window (0: none) and an optional uint8 block mask [B, H, ceil(Sq/64),
    ceil(Skv/64)] on the device. Returns (O bf16 [B,H,Sq,D], LSE fp32 [B,H,Sq])."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Skv, D) or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, torch.bfloat16, dev)
    if block_mask is not None:
        _check_dev("block_mask", block_mask, torch.uint8, dev)
        if tuple(block_mask.shape) != (B, H, -(-Sq // 64), -(-Skv // 64)):
            raise ValueError("block_mask must be uint8 [B, H, ceil(Sq/64), ceil(Skv/64)]")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.bfloat16, dev)
    _check_dev("lse", lse, torch.float32, dev)
    if tuple(out.shape) != (B, H, Sq, D) or tuple(lse.shape) != (B, H, Sq):
        raise ValueError("out/lse have the wrong shape")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _launch(_LIB.attn_fwd_ex, dev, stream, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Sq,
                 Skv, D, int(bool(causal)), int(window), _ptr(block_mask), ctypes.c_float(scale))
    if rc != TATTN_OK:
        raise TattnError(rc, "attn_fwd_ex")
    return out, lse


def attn_fwd_f32(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """fp32 multi-head attention forward: returns (O fp32 [B,H,Sq,D], LSE fp32 [B,H,Sq])."""
    return _mha("attn_fwd_f32", q, k, v, causal, scale, out, lse, stream, _torch().float32)


def _mla(fn_name, q, q_pe, kv, k_pe, kv_indptr, scale, out, lse, stream):
    torch = _torch()
    if q.dim() != 3 or q_pe.dim() != 3 or kv.dim() != 2 or k_pe.dim() != 2:
        raise ValueError("q [B,H,512], q_pe [B,H,64], kv [N,512], k_pe [N,64]")
    B, H, Dl = q.shape
    N = kv.shape[0]
    if Dl != 512 or tuple(q_pe.shape) != (B, H, 64) or kv.shape[1] != 512 or tuple(k_pe.shape) != (N, 64):
        raise ValueError("MLA widths must be 512 (latent) and 64 (rotary)")
    # the kernels write B*H rows of O and LSE: wrong-shaped buffers are
    # rejected before any device check or launch
    if (out is not None and tuple(out.shape) != (B, H, 512)) or (lse is not None and tuple(lse.shape) != (B, H)):
        raise ValueError("out must be [B, H, 512] and lse [B, H]")
    dev = q.device
    for n, t in (("q", q), ("q_pe", q_pe), ("kv", kv), ("k_pe", k_pe)):
        _check_dev(n, t, torch.bfloat16, dev)
    _check_dev("kv_indptr", kv_indptr, torch.int32, dev)
    if tuple(kv_indptr.shape) != (B + 1,):
        raise ValueError("kv_indptr must have B + 1 entries")
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.bfloat16, dev)
    _check_dev("lse", lse, torch.float32, dev)
    rc = _launch(getattr(_LIB, fn_name), dev, stream, _ptr(q), _ptr(q_pe), _ptr(kv), _ptr(k_pe), _ptr(out),
                 _ptr(lse), B, H, _ptr(kv_indptr), ctypes.c_float(float(scale)))
    if rc != TATTN_OK:
        raise TattnError(rc, fn_name)
    return out, lse


def mla_decode(q, q_pe, kv, k_pe, kv_indptr, scale, out=None, lse=None, stream=None):
    """MLA decode: q [B,H,512], q_pe [B,H,64], kv [N,512], k_pe [N,64] (bf16),
    kv_indptr int32 [B+1] on the device. Returns (O bf16 [B,H,512], LSE fp32 [B,H])."""
    return _mla("mla_decode", q, q_pe, kv, k_pe, kv_indptr, scale, out, lse, stream)


def mla_decode_noalloc(q, q_pe, kv, k_pe, kv_indptr, scale, out=None, lse=None, stream=None):
    """mla_decode with the library's static workspace (no device allocation by
    the library; pass ``out`` and ``lse`` to keep torch from allocating too)."""
    return _mla("mla_decode_noalloc", q, q_pe, kv, k_pe, kv_indptr, scale, out, lse, stream)


def ssd_scan(x, dt, A, B, C, init_state=None, final_state=False, out=None, stream=None):
    """Mamba-2 state-space scan: x [Bt,L,H,64] bf16, dt [Bt,L,H] fp32, A [H] fp32,
    B and C [Bt,L,G,128] bf16, optional init_state [Bt,H,64,128] fp32.
    Returns y bf16 [Bt,L,H,64], and with ``final_state`` (True, or an fp32
    [Bt,H,64,128] tensor to fill) also the state after the last step."""
    torch = _torch()
    if x.dim() != 4 or dt.dim() != 3 or A.dim() != 1 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("x [Bt,L,H,P], dt [Bt,L,H], A [H], B/C [Bt,L,G,N]")
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (Bt, L, H) or tuple(A.shape) != (H,) or tuple(B.shape) != (Bt, L, G, N) \
            or tuple(C.shape) != (Bt, L, G, N):
        raise ValueError("dt/A/B/C shapes do not match x")
    dev = x.device
    for n, t, dty in (("x", x, torch.bfloat16), ("dt", dt, torch.float32), ("A", A, torch.float32),
                      ("B", B, torch.bfloat16), ("C", C, torch.bfloat16)):
        _check_dev(n, t, dty, dev)
    if init_state is not None:
        _check_dev("init_state", init_state, torch.float32, dev)
        if tuple(init_state.shape) != (Bt, H, P, N):
            raise ValueError("init_state must be [Bt, H, P, N]")
    fs = None
    if final_state is True:
        fs = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not False and final_state is not None:
        fs = final_state
        _check_dev("final_state", fs, torch.float32, dev)
        if tuple(fs.shape) != (Bt, H, P, N):
            raise ValueError("final_state must be [Bt, H, P, N]")
    if out is None:
        out = torch.empty_like(x)
    _check_dev("out", out, torch.bfloat16, dev)
    if tuple(out.shape) != (Bt, L, H, P):
        raise ValueError("out has the wrong shape")
    rc = _launch(_LIB.ssd_scan, dev, stream, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(out),
                 _ptr(init_state), _ptr(fs), Bt, L, H, G, P, N)
    if rc != TATTN_OK:
        raise TattnError(rc, "ssd_scan")
    return (out, fs) if fs is not None else out
