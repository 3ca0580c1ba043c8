"""Host-side logic of the benchmark: work accounting, the traffic guard and
the one-GPU rule. No GPU needed."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from tiled_attention_12_amd.workloads import (mha_bytes, mha_flops, mla_bytes, mla_flops, ssd_bytes,  # noqa: E402
                                              ssd_flops)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (5, 5), (7, 3), (3, 7), (64, 200)])
@pytest.mark.parametrize("causal", [False, True])
def test_mha_flops_counts_visible_pairs(Sq, Skv, causal):
    # brute force over (i, j): row i sees key j unless causal and j > i + Skv - Sq
    pairs = sum(1 for i in range(Sq) for j in range(Skv) if not causal or j <= i + Skv - Sq)
    D = 16
    assert mha_flops(2, 3, Sq, Skv, D, causal) == 2 * 2 * 3 * pairs * (D + D)


def test_mha_flops_headline_values():
    # non-causal: 4 * B * H * S^2 * D; causal: S(S+1)/2 pairs per head
    assert mha_flops(4, 16, 2048, 2048, 128, False) == 4 * 4 * 16 * 2048 * 2048 * 128
    assert mha_flops(4, 16, 2048, 2048, 128, True) == 4 * 4 * 16 * (2048 * 2049 // 2) * 128


def test_byte_counts():
    # Q, K, V, O in bf16 plus an fp32 LSE per row
    assert mha_bytes(4, 16, 2048, 2048, 128, 2) == 4 * (4 * 16 * 2048 * 128 * 2) + 4 * 16 * 2048 * 4
    # MLA: 576-wide bf16 key rows, 576-wide queries, 512-wide bf16 outputs, fp32 LSE
    assert mla_bytes(64, 128, 262144) == 1152 * 262144 + 1152 * 64 * 128 + 1024 * 64 * 128 + 4 * 64 * 128
    assert mla_flops(128, 10) == 2 * 128 * 1088 * 10


def test_ssd_byte_count_of_the_scan_workload():
    # x and y bf16 [8, 4096, 64, 64]; B and C bf16 [8, 4096, 1, 128]; dt fp32 [8, 4096, 64]; A fp32 [64]
    xy = 8 * 4096 * 64 * 64 * 2
    bc = 8 * 4096 * 1 * 128 * 2
    assert ssd_bytes(8, 4096, 64, 1, 64, 128) == 2 * xy + 2 * bc + 8 * 4096 * 64 * 4 + 64 * 4 == 562036992
    # fp32 states [Bt, H, P, N] in and out
    assert ssd_bytes(2, 10, 4, 2, 64, 128, True, True) - ssd_bytes(2, 10, 4, 2, 64, 128) == 2 * 2 * 4 * 64 * 128 * 4


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_ssd_flops_brute_force(L):
    # per (batch, head) and chunk of q steps: C_t . B_s over the pairs s <= t (N each), the decay-weighted
    # product with x over the same pairs (P each), the entering state against C (q*P*N) and the state
    # update (q*P*N); two flops per multiply-add
    Bt, H, P, N, Q = 2, 3, 5, 7, 64
    macs = 0
    for c0 in range(0, L, Q):
        q = min(Q, L - c0)
        for t in range(q):
            for s in range(t + 1):
                macs += N + P
        macs += 2 * q * P * N
    assert ssd_flops(Bt, L, H, P, N) == 2 * Bt * H * macs


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_null_once_the_kernel_sources_change(monkeypatch):
    import bench
    for name, tr in bench.TRAFFIC.items():
        t = bench._traffic_bytes(name)
        if t is not None:
            assert t == pytest.approx(1024 * (tr["fetch_kib"] * bench.FETCH_FACTOR + tr["write_kib"] * bench.WRITE_FACTOR))
        monkeypatch.setitem(tr, "sources_sha256", "0" * 64)
        assert bench._traffic_bytes(name) is None
    # the written bytes of the headline launch can never be fewer than O (bf16) and LSE (fp32)
    tr = bench.TRAFFIC["mha_prefill_bf16"]
    assert tr["write_kib"] * bench.WRITE_FACTOR * 1024 >= 4 * 16 * 2048 * (128 * 2 + 4)
    assert bench._traffic_bytes("no such workload") is None


def test_cpu_baseline_budget_is_bounded(monkeypatch):
    import bench
    out = bench._cpu_baseline(budget_s=0.5)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert np.isfinite(out["value"])


def test_bf16_output_bound():
    from tests.helpers import bf16_half_ulp, bf16_o_bound
    # half-ulps of bf16 (8 significant bits) at a few magnitudes
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_half_ulp(3.0) == 2.0 ** -7
    assert bf16_half_ulp(-5.0) == 2.0 ** -6
    assert bf16_half_ulp(0.0) == 0.0
    # below |O| = 2 the bound is exactly 1e-2
    assert bf16_o_bound(1.99) == 1e-2 and bf16_o_bound(-0.3) == 1e-2
    assert bf16_o_bound(4.5) == 1e-2 + 2.0 ** -6


@pytest.mark.parametrize("Sq,Skv,causal,W", [(7, 9, True, 2), (9, 7, False, 3), (130, 70, True, 0), (130, 200, False, 50)])
def test_visible_pairs_brute_force(Sq, Skv, causal, W):
    from tiled_attention_12_amd.workloads import visible_pairs
    rng = np.random.default_rng(Sq + Skv)
    m = (rng.random((-(-Sq // 64), -(-Skv // 64))) < 0.5).astype(np.uint8)
    for mask in (None, m):
        bf = sum(1 for i in range(Sq) for j in range(Skv)
                 if (not causal or j <= i + Skv - Sq) and (W == 0 or i + Skv - Sq - W <= j < i + Skv - Sq + W)
                 and (mask is None or mask[i // 64, j // 64]))
        assert visible_pairs(Sq, Skv, causal, W, mask) == bf


def test_window_workload_is_hbm_bound_and_block_mask_mfma_bound():
    """The sliding window (256 keys per row over 8192) moves more bytes per
    FLOP than the ridge of 8 TB/s against 2516.6 TFLOP/s allows, so its
    roofline is HBM; the half-dense block mask stays on the MFMA side."""
    from tiled_attention_12_amd.workloads import WORKLOADS, visible_pairs
    w = WORKLOADS["mha_window_bf16"]
    B, H, S, D = w["B"], w["H"], w["Sq"], w["D"]
    by = mha_bytes(B, H, S, S, D, 2)
    assert by == 2 * 4 * B * H * S * D + 4 * B * H * S
    fl = 4 * D * B * H * visible_pairs(S, S, True, w["window"])
    assert fl == 4 * D * B * H * sum(min(i, w["window"]) + 1 for i in range(S))
    assert by / 8000e9 > fl / 2516.6e12
    m = WORKLOADS["mha_blocksparse_bf16"]
    by_m = mha_bytes(m["B"], m["H"], m["Sq"], m["Skv"], m["D"], 2)
    fl_m = 4 * m["D"] * m["B"] * m["H"] * m["Sq"] * m["Skv"] * m["density"]
    assert by_m / 8000e9 < fl_m / 2516.6e12


def test_bf16_round_ties_to_even_and_mean_bound():
    from tests.helpers import BF16_MEAN_ABS_O, bf16_mean_o_bound, bf16_round
    # halfway cases go to the even significand; others to the nearest
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8), 2 ** -130, 0.0])
    assert list(bf16_round(vals)) == [1.0, 1 + 2 ** -6, 1.0, -1.0, 2 ** -130, 0.0]
    # exactly representable outputs leave the plain 1e-3 gate; |O| near 1
    # adds the mean rounding error, below half an ulp (2^-9)
    assert bf16_mean_o_bound(np.array([0.5, -0.25, 1.0])) == BF16_MEAN_ABS_O
    r = np.random.default_rng(3).uniform(1.0, 2.0, 10000)
    extra = bf16_mean_o_bound(r) - BF16_MEAN_ABS_O
    assert 2 ** -10 * 0.9 < extra < 2 ** -9
