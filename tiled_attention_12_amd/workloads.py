"""The benchmark workloads: shapes, distributions, seeds.

Workload i (1-based) draws its inputs from seed 1000 + i. ``scale`` is the
float32 value passed to the kernels; the CPU side widens that same float32.
"""

import math

import numpy as np

F32_SCALE_64 = float(np.float32(1.0 / math.sqrt(64)))
F32_SCALE_128 = float(np.float32(1.0 / math.sqrt(128)))
F32_SCALE_576 = float(np.float32(1.0 / math.sqrt(576)))

WORKLOADS = {
    "mha_tiny_f32": dict(kind="mha", dtype="f32", B=1, H=2, Sq=128, Skv=128, D=64,
                         causal=(False,), sigma=1.0, scale=F32_SCALE_64, seed=1001),
    "mha_prefill_bf16": dict(kind="mha", dtype="bf16", B=4, H=16, Sq=2048, Skv=2048, D=128,
                             causal=(False, True), sigma=1.0, scale=F32_SCALE_128, seed=1002),
    "mha_long_causal_bf16": dict(kind="mha", dtype="bf16", B=1, H=32, Sq=16384, Skv=16384,
                                 D=128, causal=(True,), sigma=0.5, scale=F32_SCALE_128,
                                 seed=1003),
    "mla_decode_bf16": dict(kind="mla", B=64, H=128, kv_len=4096, sigma=0.3,
                            scale=F32_SCALE_576, seed=1004),
    "mla_decode_ragged_bf16": dict(kind="mla", B=128, H=128, kv_len_range=(1024, 16384),
                                   sigma=0.3, scale=F32_SCALE_576, seed=1005),
    # attention variants (grouped KV heads, sliding window, block mask)
    "mha_gqa_bf16": dict(kind="mha", dtype="bf16", B=4, H=16, Hkv=4, Sq=2048, Skv=2048, D=128,
                         causal=(False, True), sigma=1.0, scale=F32_SCALE_128, seed=1006),
    "mha_window_bf16": dict(kind="mha", dtype="bf16", B=4, H=16, Sq=8192, Skv=8192, D=128,
                            causal=(True,), window=256, sigma=1.0, scale=F32_SCALE_128, seed=1007),
    "mha_blocksparse_bf16": dict(kind="mha", dtype="bf16", B=4, H=16, Sq=4096, Skv=4096, D=128,
                                 causal=(False,), density=0.5, sigma=1.0, scale=F32_SCALE_128,
                                 seed=1008),
    # Mamba-2 state-space scan (chunk state + chunk scan), a 1.3B-class layer:
    # 64 heads of width 64, state 128, one B/C group
    "ssd_scan_bf16": dict(kind="ssd", Bt=8, L=4096, H=64, G=1, P=64, N=128, seed=1009),
}


def mha_flops(B, H, Sq, Skv, D, causal, Dv=None):
    """FLOPs of the two contractions (Q*K^T and P*V) over visible pairs only."""
    Dv = D if Dv is None else Dv
    if causal:
        pairs = int(np.clip(np.arange(Sq, dtype=np.int64) + (Skv - Sq) + 1, 0, Skv).sum())
    else:
        pairs = Sq * Skv
    return 2 * B * H * pairs * (D + Dv)


def visible_pairs(Sq, Skv, causal=False, window=0, mask=None, block=64):
    """Number of visible (query, key) pairs: per row the key interval from the
    causal rule and the window, intersected with the kept mask blocks.
    ``mask`` is one (query block, key block) mask [nqb, nkb] or None."""
    i = np.arange(Sq, dtype=np.int64)
    pos = i + (Skv - Sq)
    lo = np.zeros(Sq, dtype=np.int64)
    hi = np.full(Sq, Skv, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, pos + 1)
    if window > 0:
        lo = np.maximum(lo, pos - window)
        hi = np.minimum(hi, pos + window)
    hi = np.maximum(hi, lo)
    if mask is None:
        return int((hi - lo).sum())
    nkb = -(-Skv // block)
    kb0 = np.arange(nkb, dtype=np.int64) * block
    kb1 = np.minimum(kb0 + block, Skv)
    inter = np.clip(np.minimum(hi[:, None], kb1[None, :]) - np.maximum(lo[:, None], kb0[None, :]), 0, None)
    keep = np.asarray(mask)[i // block].astype(np.int64)
    return int((inter * keep).sum())


def mha_bytes(B, H, Sq, Skv, D, elem, Hkv=None, Dv=None):
    """Algorithmic HBM bytes: Q, K, V read once, O written once, fp32 LSE written once."""
    Hkv = H if Hkv is None else Hkv
    Dv = D if Dv is None else Dv
    return elem * (B * H * Sq * D + B * Hkv * Skv * (D + Dv) + B * H * Sq * Dv) + 4 * B * H * Sq


def mla_flops(H, total_keys, Dl=512, Dr=64):
    """FLOPs of the score products (Dl + Dr wide) and P*V (Dl wide) per key."""
    return 2 * H * (Dl + Dr + Dl) * int(total_keys)


def mla_bytes(B, H, total_keys, Dl=512, Dr=64):
    """Algorithmic HBM bytes: KV and K_pe rows, Q and Q_pe read once; O (bf16) and LSE written."""
    return 2 * (Dl + Dr) * int(total_keys) + 2 * B * H * (Dl + Dr) + 2 * B * H * Dl + 4 * B * H


def ssd_bytes(Bt, L, H, G, P, N, init_state=False, final_state=False):
    """Algorithmic HBM bytes of the scan: x, B, C (bf16), dt (fp32) and A read
    once, y (bf16) written once, fp32 initial / final states when used."""
    b = 2 * Bt * L * H * P * 2 + 2 * Bt * L * G * N * 2 + 4 * Bt * L * H + 4 * H
    b += 4 * Bt * H * P * N * (int(bool(init_state)) + int(bool(final_state)))
    return b


def ssd_flops(Bt, L, H, P, N, chunk=64):
    """FLOPs of the chunked form's products: per chunk of q steps, C*B^T and
    the decay-weighted product with x over the causal pairs (q(q+1)/2 each),
    the entering state against C and the state update (q*P*N each)."""
    full, tail = divmod(L, chunk)
    macs = 0
    for q, n in ((chunk, full), (tail, 1 if tail else 0)):
        pairs = q * (q + 1) // 2
        macs += n * (pairs * (N + P) + 2 * q * P * N)
    return 2 * Bt * H * macs
