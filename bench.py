"""Benchmark of the tiled attention forward on one MI355X.

One step = one pass of the prefill hot path over the headline workload
(bf16 MHA B=4, H=16, Sq=Skv=2048, D=128), run once non-causal and once
causal. The long causal prefill (B=1, H=32, S=16384), the attention variants
(grouped KV heads, sliding window, block mask), the two MLA decode
workloads and the Mamba-2 state-space scan are measured in the same run and reported under "workloads".
Inputs are seeded synthetic draws, resident in HBM before timing; each
workload rotates three input copies so consecutive launches read cold data.

Prints one JSON line (see --help for the flags).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
N_COPIES = 3

# HBM traffic per launch, from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch, summed over the kernels of one call), each
# scaled by what the same counter reads for a plain 256 MiB device copy in the
# same run (FETCH_SIZE read 131093 KiB for it: factor 2.0; WRITE_SIZE read
# 262144 KiB: factor 1.0). A figure holds for the kernel sources it was taken
# on; once those files change it is reported as null.
MHA_SOURCES = ("tiled_attention_12_amd/csrc/mha_fwd_bf16.hip", "tiled_attention_12_amd/csrc/device_common.h")
MLA_SOURCES = ("tiled_attention_12_amd/csrc/mla_decode.hip", "tiled_attention_12_amd/csrc/device_common.h")
TRAFFIC = {
    "mha_prefill_bf16": {"sources": MHA_SOURCES,
                         "sources_sha256": "80875f2bffcd98ae7166e70421481120b5f3a9fcec4bd8dcfc130a49c3611d4f",
                         "fetch_kib": 82119.4, "write_kib": 33305.4},
    "mha_long_causal_bf16": {"sources": MHA_SOURCES,
                             "sources_sha256": "80875f2bffcd98ae7166e70421481120b5f3a9fcec4bd8dcfc130a49c3611d4f",
                             "fetch_kib": 800855.8, "write_kib": 133120.5},
    # split + merge kernel of one call
    "mla_decode_bf16": {"sources": MLA_SOURCES,
                        "sources_sha256": "2bf1c3ec81376fd2f5e31e3a97d0034be7db53fc28339c22194c5cef33aca193",
                        "fetch_kib": 152247.2 + 16498.2, "write_kib": 32896.3 + 8225.8},
    "mla_decode_ragged_bf16": {"sources": MLA_SOURCES,
                               "sources_sha256": "2bf1c3ec81376fd2f5e31e3a97d0034be7db53fc28339c22194c5cef33aca193",
                               "fetch_kib": 667559.6 + 24533.3, "write_kib": 48959.0 + 16449.3},
}
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0


def _sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic_bytes(name):
    """Counter-measured HBM bytes per call of a workload, or None if not
    measured or the kernels changed since."""
    t = TRAFFIC.get(name)
    if not t or t["fetch_kib"] is None or _sources_sha(t["sources"]) != t["sources_sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * FETCH_FACTOR + t["write_kib"] * WRITE_FACTOR)


def _roofline(bound, achieved, peak, unit, traffic, kernel, alg_per_launch):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic, "kernel": kernel, "alg_per_launch": alg_per_launch}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _to_dev(arr, dev):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def _copies(arrs, dev):
    """N_COPIES device copies of each stored input array."""
    import torch
    out = []
    for c in range(N_COPIES):
        out.append({k: (_to_dev(v, dev) if c == 0 else None) for k, v in arrs.items()})
    for c in range(1, N_COPIES):
        for k in arrs:
            out[c][k] = out[0][k].clone()
    torch.cuda.synchronize()
    return out


class _Runahead:
    """Keeps the GPU ahead of the host during a timed region.

    A spin kernel (outside the timed region) holds the stream while the host
    enqueues every timed launch, so the launches then run back to back and
    the events around each one measure the GPU, not Python's launch rate.
    After the region, check() warns if enqueueing outlasted the spin."""

    SPIN_CYCLES = 200_000_000

    def __init__(self):
        import torch
        self.torch = torch
        torch.cuda.synchronize()
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)
        self.e0.record()
        torch.cuda._sleep(self.SPIN_CYCLES)
        self.e1.record()
        self.t0 = time.perf_counter()

    def enqueued(self):
        self.t_enqueue = time.perf_counter() - self.t0

    def check(self, what):
        spin_ms = self.e0.elapsed_time(self.e1)
        if self.t_enqueue * 1e3 > spin_ms:
            _log(f"bench: warning: enqueueing {what} took {self.t_enqueue * 1e3:.1f} ms, longer than the "
                 f"{spin_ms:.1f} ms spin; the GPU may have waited for the host")
        return spin_ms


def _time_launches(fn, sets, warmup, reps):
    """Average duration (ms) of fn(set) over reps launches, with HIP events on
    the stream the kernels are launched on (torch's current stream)."""
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ra = _Runahead()
    ev[0].record()
    for i in range(reps):
        fn(sets[i % len(sets)])
        ev[i + 1].record()
    ra.enqueued()
    torch.cuda.synchronize()
    ra.check("the launches")
    d = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return float(np.mean(d)), float(np.median(d)), float(np.min(d))


def _mha_workload(ta, dev, name):
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    x = inputs.mha_inputs(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], seed=w["seed"], sigma=w["sigma"])
    return w, _copies(x, dev)


def _variant_workload(ta, dev, name):
    """Grouped-head, window or block-mask workload: (spec, input copies,
    window, mask as numpy or None, mask on the device or None)."""
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS
    wv = WORKLOADS[name]
    xv = inputs.mha_inputs(wv["B"], wv["H"], wv["Sq"], wv["Skv"], wv["D"], seed=wv["seed"],
                           sigma=wv["sigma"], Hkv=wv.get("Hkv"))
    mask_np = mask_dev = None
    if "density" in wv:
        mask_np = inputs.block_mask(wv["B"], wv["H"], wv["Sq"], wv["Skv"], wv["density"], seed=wv["seed"] + 100)
        mask_dev = _to_dev(mask_np, dev)
    return wv, _copies(xv, dev), wv.get("window", 0), mask_np, mask_dev


def _mla_workload(ta, dev, name):
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    kw = {"kv_len": w["kv_len"]} if "kv_len" in w else {"kv_len_range": w["kv_len_range"]}
    m = inputs.mla_inputs(w["B"], w["H"], seed=w["seed"], sigma=w["sigma"], **kw)
    total = int(m["indptr"][-1])
    sets = _copies({k: m[k] for k in ("q", "q_pe", "kv", "k_pe", "indptr")}, dev)
    return w, sets, total


def _ssd_workload(ta, dev, name="ssd_scan_bf16"):
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    x = inputs.ssd_inputs(w["Bt"], w["L"], w["H"], w["G"], w["P"], w["N"], seed=w["seed"])
    return w, _copies(x, dev)


def _cpu_baseline(budget_s=12.0):
    """The CPU oracle, as it stands, on a bounded sample of the headline
    workload: whole (batch, head) slices, non-causal and causal alternately,
    until about budget_s seconds of CPU work. Reported in TFLOP/s."""
    import oracle
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS, mha_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    w = WORKLOADS["mha_prefill_bf16"]
    S, D = w["Sq"], w["D"]
    x = inputs.mha_inputs(1, 8, S, S, D, seed=w["seed"], sigma=w["sigma"])
    q, k, v = (inputs.stored_values(x[n]) for n in "qkv")
    flops = 0
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and n < 4096:
        h = n % 8
        causal = bool(n % 2)
        oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], w["scale"], causal=causal)
        flops += mha_flops(1, 1, S, S, D, causal)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} whole (batch, head) slices of the S=2048, D=128 bf16 prefill "
                      f"(alternating non-causal/causal), {dt:.1f} s of float64 numpy on the host"}


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _cpu_baselines(budget_s=5.0):
    """The CPU oracle, as it stands, timed on a bounded sample of each of the
    five configurations (about budget_s seconds of host work each), in the
    metric's units: TFLOP/s of the two contractions for the prefill
    configurations, GB/s of key rows (and TFLOP/s) for the decode ones."""
    import oracle
    from tiled_attention_12_amd import inputs
    from tiled_attention_12_amd.workloads import WORKLOADS, mha_flops, mla_flops
    out = {}
    cores = _host_threads()

    def timed(fn, units, done):
        n, work, t0 = 0, 0.0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s and not done(n):
            work += units(n)
            fn(n)
            n += 1
        return n, work, time.perf_counter() - t0

    w = WORKLOADS["mha_tiny_f32"]
    x = inputs.mha_inputs(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], seed=w["seed"], dtype="f32")
    f1 = mha_flops(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], False)
    n, fl, dt = timed(lambda i: oracle.attention(x["q"], x["k"], x["v"], w["scale"]), lambda i: f1,
                      lambda i: i >= 2000)
    out["config1_mha_tiny_f32"] = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                                   "sample": f"{n} whole calls of the workload, {dt:.1f} s"}

    w = WORKLOADS["mha_prefill_bf16"]
    x = inputs.mha_inputs(1, 4, w["Sq"], w["Skv"], w["D"], seed=w["seed"], sigma=w["sigma"])
    q, k, v = (inputs.stored_values(x[n]) for n in "qkv")
    for causal in (False, True):
        fh = mha_flops(1, 1, w["Sq"], w["Skv"], w["D"], causal)
        n, fl, dt = timed(lambda i: oracle.attention(q[:, i % 4:i % 4 + 1], k[:, i % 4:i % 4 + 1],
                                                     v[:, i % 4:i % 4 + 1], w["scale"], causal=causal),
                          lambda i: fh, lambda i: i >= 64)
        out[f"config2_mha_prefill_bf16_{'causal' if causal else 'noncausal'}"] = {
            "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} whole (batch, head) slices of the S=2048, D=128 prefill, {dt:.1f} s"}
    del q, k, v, x

    w = WORKLOADS["mha_long_causal_bf16"]
    x = inputs.mha_inputs(w["B"], w["H"], w["Sq"], w["Skv"], w["D"], seed=w["seed"], sigma=w["sigma"])
    S = w["Sq"]
    rows_per = 2048
    q, k, v = (inputs.stored_values(x[n][:, :1]) for n in "qkv")
    del x

    def blk(i):
        r0 = (i * rows_per) % S
        oracle.attention(q, k, v, w["scale"], causal=True, rows=np.arange(r0, r0 + rows_per))
    pairs = lambda i: int(np.sum(np.arange((i * rows_per) % S, (i * rows_per) % S + rows_per) + 1))
    n, pr, dt = timed(blk, pairs, lambda i: i >= S // rows_per)
    out["config3_mha_long_causal_bf16"] = {
        "value": 4 * w["D"] * pr / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{n} blocks of {rows_per} query rows of head 0 of the S=16384 causal prefill, {dt:.1f} s"}
    del q, k, v

    for key, name in (("config4_mla_decode_bf16", "mla_decode_bf16"),
                      ("config5_mla_decode_ragged_bf16", "mla_decode_ragged_bf16")):
        w = WORKLOADS[name]
        kw = {"kv_len": w["kv_len"]} if "kv_len" in w else {"kv_len_range": w["kv_len_range"]}
        m = inputs.mla_inputs(w["B"], w["H"], seed=w["seed"], sigma=w["sigma"], **kw)
        ind = m["indptr"]
        vals = {n: m[n] for n in ("q", "q_pe", "kv", "k_pe")}
        lens = np.diff(ind)

        def one(i):
            b = i % w["B"]
            lo, hi = int(ind[b]), int(ind[b + 1])
            oracle.mla_decode(inputs.stored_values(vals["q"][b:b + 1]), inputs.stored_values(vals["q_pe"][b:b + 1]),
                              inputs.stored_values(vals["kv"][lo:hi]), inputs.stored_values(vals["k_pe"][lo:hi]),
                              np.array([0, hi - lo], np.int64), w["scale"])
        n, keys, dt = timed(one, lambda i: int(lens[i % w["B"]]), lambda i: i >= w["B"])
        keys = int(keys)
        out[key] = {"value": 1152 * keys / dt / 1e9, "unit": "GB/s of key rows", "cores": cores, "kind": "oracle",
                    "tflops": mla_flops(w["H"], keys) / dt / 1e12,
                    "sample": f"{n} whole batches ({keys} keys, all {w['H']} heads), {dt:.1f} s"}
        del m, vals
    return out


# profiling names of the grouped-head, window and block-mask workloads:
# name -> (workload, causal)
VARIANT_ONLY = {"mha_gqa_bf16": ("mha_gqa_bf16", False), "mha_gqa_bf16_causal": ("mha_gqa_bf16", True),
                "mha_window_bf16": ("mha_window_bf16", True),
                "mha_blocksparse_bf16": ("mha_blocksparse_bf16", False)}


def _profile_only(args, ta, dev):
    """Run args.steps launches of one workload (after args.warmup) and print its mean time."""
    import torch
    name = args.only
    if name in VARIANT_ONLY:
        base, causal = VARIANT_ONLY[name]
        w, sets, window, _, mask_dev = _variant_workload(ta, dev, base)
        o, l = ta.attn_fwd_ex(sets[0]["q"], sets[0]["k"], sets[0]["v"], scale=w["scale"])
        fn = lambda s: ta.attn_fwd_ex(s["q"], s["k"], s["v"], causal=causal, scale=w["scale"], window=window,
                                      block_mask=mask_dev, out=o, lse=l)
    elif name.startswith("mha"):
        causal = name != "mha_prefill_bf16"
        w, sets = _mha_workload(ta, dev, name.replace("_causal", "") if name == "mha_prefill_bf16_causal" else name)
        o, l = ta.attn_fwd(sets[0]["q"], sets[0]["k"], sets[0]["v"], causal=causal, scale=w["scale"])
        fn = lambda s: ta.attn_fwd(s["q"], s["k"], s["v"], causal=causal, scale=w["scale"], out=o, lse=l)
    elif name.startswith("ssd"):
        w, sets = _ssd_workload(ta, dev, name)
        s0 = sets[0]
        y = ta.ssd_scan(s0["x"], s0["dt"], s0["A"], s0["B"], s0["C"])
        fn = lambda s: ta.ssd_scan(s["x"], s["dt"], s["A"], s["B"], s["C"], out=y)
    else:
        w, sets, _ = _mla_workload(ta, dev, name)
        s0 = sets[0]
        o, l = ta.mla_decode(s0["q"], s0["q_pe"], s0["kv"], s0["k_pe"], s0["indptr"], w["scale"])
        fn = lambda s: ta.mla_decode(s["q"], s["q_pe"], s["kv"], s["k_pe"], s["indptr"], w["scale"], out=o, lse=l)
    mean, med, mn = _time_launches(fn, sets, args.warmup, args.steps)
    print(json.dumps({"only": name, "ms_mean": mean, "ms_median": med, "ms_min": mn}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-secondary", action="store_true",
                    help="only the headline prefill workload (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["mha_prefill_bf16", "mha_prefill_bf16_causal", "mha_long_causal_bf16",
                                       "mla_decode_bf16", "mla_decode_ragged_bf16", "ssd_scan_bf16"]
                                      + list(VARIANT_ONLY),
                    help="profiling mode: run --steps launches of one workload, print its timing only")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="profiling mode: first run one device-to-device copy of this many MiB "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the kernels run on one GPU's share; see the design notes on sharding).", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_attention_12_amd as ta
    from tiled_attention_12_amd.workloads import mha_bytes, mha_flops, mla_bytes, mla_flops, ssd_bytes, ssd_flops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        _profile_only(args, ta, dev)
        return

    # ---------------------------------------------------------------- headline prefill
    _log("bench: preparing the headline prefill workload")
    w, sets = _mha_workload(ta, dev, "mha_prefill_bf16")
    B, H, S, D = w["B"], w["H"], w["Sq"], w["D"]
    outs = [ta.attn_fwd(s["q"], s["k"], s["v"], causal=False, scale=w["scale"]) for s in sets[:1]]
    o_buf, l_buf = outs[0]
    f_nc, f_c = mha_flops(B, H, S, S, D, False), mha_flops(B, H, S, S, D, True)
    nbytes = mha_bytes(B, H, S, S, D, 2)

    def step(i):
        s = sets[i % N_COPIES]
        ta.attn_fwd(s["q"], s["k"], s["v"], causal=False, scale=w["scale"], out=o_buf, lse=l_buf)
        ta.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w["scale"], out=o_buf, lse=l_buf)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch events: non-causal launch j is bracketed by ev[2j], ev[2j+1]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    ra = _Runahead()
    ev[0].record()
    for i in range(args.steps):
        s = sets[i % N_COPIES]
        ta.attn_fwd(s["q"], s["k"], s["v"], causal=False, scale=w["scale"], out=o_buf, lse=l_buf)
        ev[2 * i + 1].record()
        ta.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w["scale"], out=o_buf, lse=l_buf)
        ev[2 * i + 2].record()
    ra.enqueued()
    torch.cuda.synchronize()
    spin_ms = ra.check("the timed steps")
    t_wall = ra.t_enqueue
    d_nc = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]
    d_c = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)]
    total_ms = ev[0].elapsed_time(ev[-1])
    ms_step = total_ms / args.steps
    value = (f_nc + f_c) / (ms_step * 1e-3) / 1e12
    nc_ms, c_ms = float(np.mean(d_nc)), float(np.mean(d_c))
    _log(f"bench: prefill non-causal {nc_ms * 1e3:.1f} us, causal {c_ms * 1e3:.1f} us, "
         f"step {ms_step * 1e3:.1f} us, host enqueue {t_wall * 1e3:.1f} ms under a {spin_ms:.1f} ms spin")

    workloads = {
        "mha_prefill_bf16_noncausal": {
            "ms": nc_ms, "ms_median": float(np.median(d_nc)), "ms_min": float(np.min(d_nc)),
            "tflops": f_nc / (nc_ms * 1e-3) / 1e12,
            "frac_mfma_peak": f_nc / (nc_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "mha_prefill_bf16_causal": {
            "ms": c_ms, "ms_median": float(np.median(d_c)), "ms_min": float(np.min(d_c)),
            "tflops": f_c / (c_ms * 1e-3) / 1e12,
            "frac_mfma_peak": f_c / (c_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
    }
    del sets

    if not args.skip_secondary:
        _log("bench: tiny fp32 attention")
        from tiled_attention_12_amd import inputs as _inputs
        from tiled_attention_12_amd.workloads import WORKLOADS as _W
        w1 = _W["mha_tiny_f32"]
        x1 = _inputs.mha_inputs(w1["B"], w1["H"], w1["Sq"], w1["Skv"], w1["D"], seed=w1["seed"],
                                sigma=w1["sigma"], dtype="f32")
        sets1 = _copies(x1, dev)
        o1, l1 = ta.attn_fwd_f32(sets1[0]["q"], sets1[0]["k"], sets1[0]["v"], scale=w1["scale"])
        mean1, med1, min1 = _time_launches(
            lambda s: ta.attn_fwd_f32(s["q"], s["k"], s["v"], scale=w1["scale"], out=o1, lse=l1), sets1, 5, 50)
        f1 = mha_flops(w1["B"], w1["H"], w1["Sq"], w1["Skv"], w1["D"], False)
        workloads["mha_tiny_f32"] = {"ms": mean1, "ms_median": med1, "ms_min": min1,
                                     "tflops": f1 / (mean1 * 1e-3) / 1e12}
        del sets1, o1, l1

        _log("bench: long causal prefill")
        w3, sets3 = _mha_workload(ta, dev, "mha_long_causal_bf16")
        o3, l3 = ta.attn_fwd(sets3[0]["q"], sets3[0]["k"], sets3[0]["v"], causal=True, scale=w3["scale"])
        mean3, med3, min3 = _time_launches(
            lambda s: ta.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w3["scale"], out=o3, lse=l3),
            sets3, 2, 10)
        f3 = mha_flops(w3["B"], w3["H"], w3["Sq"], w3["Skv"], w3["D"], True)
        workloads["mha_long_causal_bf16"] = {
            "ms": mean3, "ms_median": med3, "ms_min": min3, "tflops": f3 / (mean3 * 1e-3) / 1e12,
            "frac_mfma_peak": f3 / (mean3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "roofline": _roofline("mfma", f3 / (mean3 * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s",
                                  _traffic_bytes("mha_long_causal_bf16"),
                                  "mha_fwd_bf16_kernel<128, 8, 64, 3, true, false> (causal)", f3)}
        del sets3, o3, l3

        from tiled_attention_12_amd.workloads import visible_pairs
        for name in ("mha_gqa_bf16", "mha_window_bf16", "mha_blocksparse_bf16"):
            _log(f"bench: {name}")
            wv, setsv, window, mask_np, mask_dev = _variant_workload(ta, dev, name)
            ov, lv = ta.attn_fwd_ex(setsv[0]["q"], setsv[0]["k"], setsv[0]["v"], scale=wv["scale"])
            for causal in wv["causal"]:
                fn = (lambda s, c=causal: ta.attn_fwd_ex(s["q"], s["k"], s["v"], causal=c, scale=wv["scale"],
                                                         window=window, block_mask=mask_dev, out=ov, lse=lv))
                mean_v, med_v, min_v = _time_launches(fn, setsv, 2, 10)
                if mask_np is None:
                    pairs = wv["B"] * wv["H"] * visible_pairs(wv["Sq"], wv["Skv"], causal, window)
                else:
                    pairs = sum(visible_pairs(wv["Sq"], wv["Skv"], causal, window, mask_np[b, h])
                                for b in range(wv["B"]) for h in range(wv["H"]))
                fv = 2 * pairs * 2 * wv["D"]
                # Q, K, V read once, O and LSE written once, the mask read once
                bv = mha_bytes(wv["B"], wv["H"], wv["Sq"], wv["Skv"], wv["D"], 2, Hkv=wv.get("Hkv"))
                if mask_np is not None:
                    bv += mask_np.size
                t_hbm, t_mfma = bv / (PEAK_HBM_GBS * 1e9), fv / (PEAK_BF16_TFLOPS * 1e12)
                key = f"{name}_{'causal' if causal else 'noncausal'}"
                workloads[key] = {"ms": mean_v, "ms_median": med_v, "ms_min": min_v, "visible_pairs": pairs,
                                  "tflops": fv / (mean_v * 1e-3) / 1e12,
                                  "frac_mfma_peak": fv / (mean_v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                  "alg_gbs": bv / (mean_v * 1e-3) / 1e9,
                                  "bound": "hbm" if t_hbm > t_mfma else "mfma",
                                  "frac_roofline": max(t_hbm, t_mfma) / (mean_v * 1e-3)}
            del setsv, ov, lv, mask_dev

        for name in ("mla_decode_bf16", "mla_decode_ragged_bf16"):
            _log(f"bench: {name}")
            wm, setsm, total = _mla_workload(ta, dev, name)
            s0 = setsm[0]
            om, lm = ta.mla_decode(s0["q"], s0["q_pe"], s0["kv"], s0["k_pe"], s0["indptr"], wm["scale"])
            mean_m, med_m, min_m = _time_launches(
                lambda s: ta.mla_decode(s["q"], s["q_pe"], s["kv"], s["k_pe"], s["indptr"], wm["scale"],
                                        out=om, lse=lm), setsm, 5, 30)
            fl = mla_flops(wm["H"], total)
            by = mla_bytes(wm["B"], wm["H"], total)
            t_star = max(by / (PEAK_HBM_GBS * 1e9), fl / (PEAK_BF16_TFLOPS * 1e12))
            workloads[name] = {"ms": mean_m, "ms_median": med_m, "ms_min": min_m, "total_keys": total,
                               "kv_gbs": 1152 * total / (mean_m * 1e-3) / 1e9,
                               "alg_gbs": by / (mean_m * 1e-3) / 1e9,
                               "tflops": fl / (mean_m * 1e-3) / 1e12,
                               "frac_roofline": t_star / (mean_m * 1e-3),
                               # one call = the split kernel and the merge kernel; HBM-bound
                               # (arithmetic intensity below the ridge point)
                               "roofline": _roofline("hbm", by / (mean_m * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                                     _traffic_bytes(name),
                                                     "mla_split_kernel<4, 4, true> + mla_combine_kernel", by)}
            del setsm, om, lm

        _log("bench: ssd_scan_bf16")
        ws, setss = _ssd_workload(ta, dev)
        s0 = setss[0]
        ys = ta.ssd_scan(s0["x"], s0["dt"], s0["A"], s0["B"], s0["C"])
        mean_s, med_s, min_s = _time_launches(
            lambda s: ta.ssd_scan(s["x"], s["dt"], s["A"], s["B"], s["C"], out=ys), setss, 3, 20)
        fl = ssd_flops(ws["Bt"], ws["L"], ws["H"], ws["P"], ws["N"])
        by = ssd_bytes(ws["Bt"], ws["L"], ws["H"], ws["G"], ws["P"], ws["N"])
        t_star = max(by / (PEAK_HBM_GBS * 1e9), fl / (PEAK_BF16_TFLOPS * 1e12))
        workloads["ssd_scan_bf16"] = {"ms": mean_s, "ms_median": med_s, "ms_min": min_s,
                                      "alg_gbs": by / (mean_s * 1e-3) / 1e9,
                                      "tflops": fl / (mean_s * 1e-3) / 1e12,
                                      "frac_roofline": t_star / (mean_s * 1e-3)}
        del setss, ys

    achieved = f_nc / (nc_ms * 1e-3) / 1e12
    line = {
        "metric": "prefill attn TFLOP/s & MLA-decode KV GB/s, % of MI355X roofline",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mha_prefill_bf16: B=4 H=16 Sq=Skv=2048 D=128, non-causal + causal per step",
                   "global_batch": B, "seq_len": S, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _traffic_bytes("mha_prefill_bf16"),
                     "kernel": "mha_fwd_bf16_kernel<128, 8, 64, 3, false, false> (non-causal)",
                     "alg_flops_per_launch": f_nc, "alg_bytes_per_launch": nbytes},
        "workloads": workloads,
    }
    if not args.no_cpu_baseline:
        _log("bench: CPU oracle baseline")
        line["cpu_baseline"] = _cpu_baseline()
        _log("bench: CPU oracle baseline per configuration")
        line["cpu_baseline_per_config"] = _cpu_baselines()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
