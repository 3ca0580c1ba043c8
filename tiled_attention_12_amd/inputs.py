"""Seeded synthetic inputs shared by the tests, the benchmark and the checker.

This module holds no attention arithmetic: it draws iid normal arrays from a
seeded numpy PCG64 generator, scales them, and rounds them to their storage
type. Both sides of a parity check consume exactly the stored values (bf16
bits for the kernels, the same bits widened to float64 for the CPU side).

Draw order is fixed so a seed names one input set: MHA draws Q, K, V; MLA
draws (ragged lengths first, when asked for) Q, Q_pe, KV, K_pe; the
state-space scan draws x, B, C, dt, A and (when asked for) an initial state. Each array is
float32 ``standard_normal`` times ``sigma`` (in float32), then rounded to
bf16 with round-to-nearest-even when the storage type is bf16.
"""

import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape, sigma):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _store(x, dtype):
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown storage dtype {dtype!r}")


def stored_values(arr):
    """The exact values an array holds, as float32 (bf16 bits are widened)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)


def mha_inputs(B, H, Sq, Skv, D, seed, sigma=1.0, dtype="bf16", Hkv=None, Dv=None):
    """Q [B,H,Sq,D], K [B,Hkv,Skv,D], V [B,Hkv,Skv,Dv] as stored arrays.

    bf16 arrays come back as uint16 bit patterns, f32 arrays as float32.
    """
    Hkv = H if Hkv is None else Hkv
    Dv = D if Dv is None else Dv
    rng = np.random.default_rng(seed)
    q = _store(_draw(rng, (B, H, Sq, D), sigma), dtype)
    k = _store(_draw(rng, (B, Hkv, Skv, D), sigma), dtype)
    v = _store(_draw(rng, (B, Hkv, Skv, Dv), sigma), dtype)
    return {"q": q, "k": k, "v": v}


def ragged_lengths(rng, B, lo, hi):
    """Per-batch key counts drawn uniformly from the integers lo..hi inclusive."""
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)


def mla_inputs(B, H, seed, kv_len=None, kv_len_range=None, sigma=0.3, Dl=512, Dr=64):
    """MLA decode inputs, all bf16 bits, with packed KV rows and int32 offsets.

    Exactly one of ``kv_len`` (every batch has that many keys) and
    ``kv_len_range`` ((lo, hi): lengths drawn first, uniform on lo..hi
    inclusive) is given. KV rows of all batches are packed back to back;
    ``indptr[b]`` is the first row of batch b and ``indptr[B]`` the total.
    """
    rng = np.random.default_rng(seed)
    if (kv_len is None) == (kv_len_range is None):
        raise ValueError("give exactly one of kv_len and kv_len_range")
    if kv_len is not None:
        lens = np.full(B, int(kv_len), dtype=np.int64)
    else:
        lens = ragged_lengths(rng, B, *kv_len_range)
    indptr = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(lens, out=indptr[1:])
    if indptr[-1] >= 2**31:
        raise ValueError("total KV rows must fit int32 offsets")
    n = int(indptr[-1])
    q = f32_to_bf16_bits(_draw(rng, (B, H, Dl), sigma))
    q_pe = f32_to_bf16_bits(_draw(rng, (B, H, Dr), sigma))
    kv = f32_to_bf16_bits(_draw(rng, (n, Dl), sigma))
    k_pe = f32_to_bf16_bits(_draw(rng, (n, Dr), sigma))
    return {"q": q, "q_pe": q_pe, "kv": kv, "k_pe": k_pe,
            "indptr": indptr.astype(np.int32), "lens": lens}


def block_mask(B, H, Sq, Skv, density, seed, block=64):
    """uint8 [B, H, ceil(Sq/block), ceil(Skv/block)]: each (query block, key
    block) pair kept (1) independently with probability ``density``."""
    rng = np.random.default_rng(seed)
    shape = (B, H, -(-Sq // block), -(-Skv // block))
    return (rng.random(shape) < density).astype(np.uint8)



def ssd_inputs(Bt, L, H, G, P, N, seed, sigma=1.0, dt_range=(1e-3, 1e-1),
               a_range=(1.0, 16.0), init_state=False, init_sigma=0.1):
    """Inputs of the Mamba-2 state-space scan.

    x [Bt, L, H, P], B and C [Bt, L, G, N]: bf16 bits of float32 normals times
    ``sigma``. dt [Bt, L, H] float32, log-uniform on ``dt_range`` (the range
    Mamba-2 initialises its step sizes to). A [H] float32, minus a uniform draw
    on ``a_range`` (Mamba-2's A = -exp(A_log) initialisation). With
    ``init_state``, an initial state [Bt, H, P, N] float32 of normals times
    ``init_sigma``.
    """
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_draw(rng, (Bt, L, H, P), sigma))
    b = f32_to_bf16_bits(_draw(rng, (Bt, L, G, N), sigma))
    c = f32_to_bf16_bits(_draw(rng, (Bt, L, G, N), sigma))
    lo, hi = np.log(dt_range[0]), np.log(dt_range[1])
    dt = np.exp(rng.uniform(lo, hi, size=(Bt, L, H))).astype(np.float32)
    a = (-rng.uniform(a_range[0], a_range[1], size=H)).astype(np.float32)
    out = {"x": x, "B": b, "C": c, "dt": dt, "A": a}
    if init_state:
        out["init_state"] = _draw(rng, (Bt, H, P, N), init_sigma)
    return out
