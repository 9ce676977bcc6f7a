"""Benchmark of the joint-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t2i_2048_bf16]

Workload: FLUX 3 Image Klein 2048x2048 text-to-image joint attention -- batch 2
(classifier-free guidance), 24 heads of 128, 512 text + 16384 image tokens
(N = 16896), seeded synthetic bf16 inputs (joint_attention_amd.synth), resident in HBM
before timing starts.

One timed step of the bf16 path = pack(Q), pack(K), pack(V^T) -> joint_attn_fwd_bf16_splitkv
with the library's suggested split (the query tiles of the last, partial round of
workgroups split into key ranges; workspace allocated before timing).  The same step with
the plain joint_attn_fwd_bf16 is reported under "plain_bf16".
The same attention through joint_attn_fwd_bf16_streams (streams read in place, no pack)
is timed in its own loop and reported under "fused_bf16", and through
joint_attn_fwd_bf16_streams_splitkv (Q and K in place; V^T packed inside the call, or V in
place too) under "fused_bf16_splitkv" and "fused_bf16_splitkv_inplace", each checked to
equal the timed step's output bit for bit; the block-sparse forward with a structured block
mask under "sparse_bf16".
The fp8 path (pack x3 -> joint_attn_quant_fp8 -> joint_attn_fwd_fp8_splitkv, the plain
joint_attn_fwd_fp8 timed beside it) on the same inputs is timed the same way in its own
loop and reported under "fp8", for both modes, from the streams, and with token repair
(rho = 0.005).
value = algorithmic attention flops (4 B H N^2 D) per bf16 step / step time.

Under "shapes", the forward alone is timed on the other shapes: 1024^2 T2I, 2048^2 I2I and
I2I with one or three reference images (same generator), and one GPU's share of a Ulysses
head split of 2048^2 T2I (batch 0 with 6 or 3 of the 24 heads).  Where such a grid holds
fewer than about four workgroups per compute unit, the split-KV forward is timed beside it.

Per-kernel durations come from HIP events recorded on the launch stream around every
launch inside the timed loops.  The CPU baseline times the fp64 oracle on a bounded
sample of query rows of the same workload on this host's cores.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "joint-attention TFLOP/s at 2048^2 (16896 tok, bf16/fp8); % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0

# HBM bytes per timed forward (the split-KV kernel and its merge) on this workload from
# two rocprofv3 --pmc runs (FETCH_SIZE x 2 + WRITE_SIZE x 1, the factors a plain copy of
# known size needs), valid for the kernel sources whose hash is recorded; any later
# change reports null.
MEASURED_TRAFFIC = {
    "workload": "t2i_2048_bf16",
    "bytes": 1897940534,
    "sources": ("joint_attention_amd/csrc/fwd_bf16.hip", "joint_attention_amd/csrc/splitkv_merge.h",
                "joint_attention_amd/csrc/ja_device.h"),
    "sha256_16": "35a7642e521ee655",
    "summary": "profiles/fwd_bf16_t2i_2048.txt",
}


def measured_traffic(workload: str):
    import hashlib
    t = MEASURED_TRAFFIC
    if workload != t["workload"]:
        return None
    h = hashlib.sha256()
    for f in t["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return t["bytes"] if h.hexdigest()[:16] == t["sha256_16"] else None


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class ClockSampler:
    """Samples the GPU's current shader clock (the starred level of the kernel driver's
    pp_dpm_sclk) every `period` seconds in a background thread, and the board power
    (hwmon power1_input) beside it.  Reports None where the files are missing.  (amdsmi's
    gpu_metrics refreshes about once a second.)"""

    def __init__(self, period: float = 0.005):
        import threading
        self.period, self.samples, self.err = period, [], None
        self.power, self.power_cap = [], None
        self._stop = threading.Event()
        self._thread = None
        self.path = self._find()
        self.power_path = None
        if self.path is not None:
            import glob
            hw = sorted(glob.glob(os.path.join(os.path.dirname(self.path), "hwmon", "hwmon*")))
            if hw and os.path.exists(os.path.join(hw[0], "power1_input")):
                self.power_path = os.path.join(hw[0], "power1_input")
                try:
                    with open(os.path.join(hw[0], "power1_cap")) as f:
                        self.power_cap = float(f.read()) / 1e6
                except Exception:
                    self.power_cap = None

    def _find(self):
        import glob
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(cards) > 1:
            try:                                   # the card torch's device 0 sits on
                import torch
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                if bus is not None:
                    cards = [c for c in cards
                             if os.path.realpath(os.path.dirname(c)).endswith(":%02x:00.0" % bus)]
            except Exception as e:
                self.err = repr(e)
        if len(cards) != 1:
            self.err = self.err or "pp_dpm_sclk: %d candidate files" % len(cards)
            return None
        return cards[0]

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    mhz = line.split(":", 1)[1].strip().rstrip("*").strip()
                    return float(mhz.lower().replace("mhz", ""))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None and v > 0:
                    self.samples.append(v)
                if self.power_path is not None:
                    with open(self.power_path) as f:
                        self.power.append(float(f.read()) / 1e6)
            except Exception as e:
                self.err = repr(e)
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.path is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def result(self):
        if not self.samples:
            return {"clock_ghz": None, "clock_source": "unavailable (%s)" % self.err}
        import statistics
        r = {"clock_ghz": round(statistics.fmean(self.samples) / 1000.0, 4),
             "clock_ghz_min": round(min(self.samples) / 1000.0, 4),
             "clock_ghz_max": round(max(self.samples) / 1000.0, 4),
             "clock_samples": len(self.samples),
             "clock_source": "%s (current level), sampled every %d ms"
                             % (self.path, int(self.period * 1000))}
        if self.power:
            r["board_power_w"] = round(statistics.fmean(self.power), 1)
            r["board_power_cap_w"] = self.power_cap
        return r


def sustained_clock(step, ms_per_step: float, seconds: float = 1.0, settle: float = 0.3):
    import torch
    n = int((settle + seconds + 0.3) * 1000.0 / max(ms_per_step, 0.05)) + 1
    for _ in range(n):                 # queued: the GPU runs them back to back
        step(False)
    time.sleep(settle)
    sampler = ClockSampler()
    with sampler:
        time.sleep(seconds)
    torch.cuda.synchronize()
    r = sampler.result()
    r["clock_load"] = "%d untimed steps queued back to back; sampled after %.1f s for %.1f s" % (
        n, settle, seconds)
    return r


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def device_name() -> str:
    import torch
    p = torch.cuda.get_device_properties(0)
    return "%s (%s, %d CUs)" % (p.name, getattr(p, "gcnArchName", "?"), p.multi_processor_count)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t2i_2048_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--skip-fp8", action="store_true")
    ap.add_argument("--skip-shapes", action="store_true",
                    help="skip the forward-only timing of the other shapes")
    return ap.parse_args()


def cpu_baseline(w, host, target_s: float):
    """fp64 oracle on a bounded row sample of the same inputs; TFLOP/s on 4*N*D per row."""
    import numpy as np
    import oracle
    from joint_attention_amd import synth
    qh, kh, vh = host
    scale = 1.0 / math.sqrt(w.D)
    threads = oracle.default_threads()
    probe = synth.row_sample(w, 256, seed=7)
    t0 = time.perf_counter()
    oracle.attention_rows(qh, kh, vh, scale, probe, threads)
    t_probe = time.perf_counter() - t0
    n = int(max(256, min(200000, 256 * target_s / max(t_probe, 1e-6))))
    sel = synth.row_sample(w, n, seed=8)
    t0 = time.perf_counter()
    ref, _ = oracle.attention_rows(qh, kh, vh, scale, sel, threads)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.N * w.D * len(sel)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d query rows (every row near a stream boundary + random rows, "
                      "row_sample seed 8) of %s: B=%d H=%d N=%d D=%d, fp64, %.1f s"
                      % (len(sel), w.name, w.B, w.H, w.N, w.D, dt),
            "seconds": dt, "rows": sel, "ref": ref}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import joint_attention_amd as ja
    from joint_attention_amd import synth

    if not os.path.exists(ja.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    ja.load()

    w = synth.WORKLOADS[args.workload]
    log("generating %s inputs (B=%d H=%d N=%d D=%d)" % (w.name, w.B, w.H, w.N, w.D))
    st = synth.make_streams(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    qs_d = [dev(s) for s in st.q]
    ks_d = [dev(s) for s in st.k]
    vs_d = [dev(s) for s in st.v]
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(w.D)
    N, B, H, D = w.N, w.B, w.H, w.D
    ldv = ja.joint_attn_vt_ld(N)
    q = torch.empty((B, H, N, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.empty((B, H, D, ldv), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # the forward of the timed step: the split-KV call with the library's suggested split
    # (the query tiles of the last, partial round of workgroups run as key ranges in
    # parallel, merged by log-sum-exp; 1 = the plain forward); workspace allocated here,
    # outside the timing, like the outputs
    ns_main = int(ja.load().joint_attn_fwd_bf16_splitkv_suggest(B, H, N, D))
    ws_main = torch.empty((int(ja.load().joint_attn_fwd_bf16_splitkv_workspace(
        B, H, N, D, ns_main)),), dtype=torch.uint8, device="cuda")

    def make_step(fwd):
        def step(rec):
            e0, e1, e2 = (ev(), ev(), ev()) if rec else (None, None, None)
            if rec:
                e0.record(stream)
            ja.joint_attn_pack(qs_d, "bhnd", out=q)
            ja.joint_attn_pack(ks_d, "bhnd", out=k)
            ja.joint_attn_pack(vs_d, "bhdn", out=vt)
            if rec:
                e1.record(stream)
            fwd()
            if rec:
                e2.record(stream)
            return (e0, e1, e2)
        return step

    step_bf16 = make_step(lambda: ja.joint_attn_fwd_bf16_splitkv(
        q, k, vt, scale, n_split=ns_main, workspace=ws_main, out=o))
    step_plain = make_step(lambda: ja.joint_attn_fwd_bf16(q, k, vt, scale, out=o))

    def timed(step, steps, warmup):
        for _ in range(warmup):
            step(False)
        torch.cuda.synchronize()
        evs = []
        t0 = time.perf_counter()
        for _ in range(steps):
            evs.append(step(True))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        durs = [[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in evs]
        return wall, np.asarray(durs)

    log("timing bf16 path (split-KV, n_split %d): %d warmup + %d steps"
        % (ns_main, args.warmup, args.steps))
    wall, durs = timed(step_bf16, args.steps, args.warmup)
    o_timed = o.clone()            # the timed step's output, compared with the oracle below
    ms_step = wall * 1e3 / args.steps
    pack_ms, fwd_ms = durs.mean(axis=0)
    flops = float(w.flops)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (fwd_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "D": D,
                   "stream_lens": list(w.stream_lens),
                   "step": "pack q,k,v + fwd_bf16_splitkv (n_split %d for the last round's "
                           "query tiles)" % ns_main},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "kernel": "fwd_bf16_kernel<128,splitkv> + splitkv_merge_kernel<128>",
                     "avg_launch_ms": round(float(fwd_ms), 4),
                     "median_launch_ms": round(float(np.median(durs[:, 1])), 4),
                     "min_launch_ms": round(float(durs[:, 1].min()), 4)},
        "kernels_ms": {"pack_qkv": round(float(pack_ms), 4),
                       "fwd_bf16_splitkv": round(float(fwd_ms), 4)},
        "pct_of_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "device": device_name(),
    }
    # the shader clock under this load: the same step queued for ~1.6 s (untimed); the
    # driver's current clock level is sampled for 1 s after a 0.3 s settle
    out.update(sustained_clock(step_bf16, ms_step))
    if out.get("clock_ghz"):
        # the dense bf16 peak at the clock these steps ran at (4096 flop/clk/CU, 256 CUs)
        out["roofline"]["frac_of_peak_at_measured_clock"] = round(
            achieved / (PEAK_BF16_TFLOPS * out["clock_ghz"] / 2.4), 4)

    # the same step with the plain forward (every query tile over all keys)
    log("timing bf16 path with the plain forward")
    wall_p, durs_p = timed(step_plain, args.steps, args.warmup)
    ms_p = wall_p * 1e3 / args.steps
    fwd_p = float(durs_p[:, 1].mean())
    out["plain_bf16"] = {
        "step": "pack q,k,v + fwd_bf16", "value": round(flops / (ms_p * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "ms_per_step": round(ms_p, 4), "kernel": "fwd_bf16_kernel<128>",
        "fwd_ms": round(fwd_p, 4), "fwd_tflops": round(flops / (fwd_p * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(flops / (fwd_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }

    # the same step through the call that reads the streams in place (no pack)
    def step_fused(rec):
        e0, e1 = (ev(), ev()) if rec else (None, None)
        if rec:
            e0.record(stream)
        ja.joint_attn_fwd_bf16_streams(qs_d, ks_d, vs_d, scale, out=o)
        if rec:
            e1.record(stream)
        return (e0, e1)

    log("timing fused bf16 path (streams read in place)")
    wall_f, durs_f = timed(step_fused, args.steps, args.warmup)
    ms_f = wall_f * 1e3 / args.steps
    out["fused_bf16"] = {
        "step": "fwd_bf16_streams (pack folded into the forward's loads)",
        "value": round(flops / (ms_f * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "ms_per_step": round(ms_f, 4),
        "kernel_ms": round(float(durs_f.mean()), 4),
        "kernel_tflops": round(flops / (float(durs_f.mean()) * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(flops / (float(durs_f.mean()) * 1e-3) / 1e12
                                   / PEAK_BF16_TFLOPS, 4),
    }

    # the split-KV step over the streams: Q and K read in place, V either transposed into
    # the workspace by the call (pack_v 1) or read in place too (pack_v 0); workspaces
    # allocated before timing.  Its output must equal the timed bf16 step's bit for bit.
    for pack_v, key, what in ((1, "fused_bf16_splitkv", "Q, K in place, V^T packed in the call"),
                              (0, "fused_bf16_splitkv_inplace", "Q, K, V all in place")):
        ws_s = torch.empty((max(int(ja.load().joint_attn_fwd_bf16_streams_splitkv_workspace(
            B, H, N, D, ns_main, pack_v)), 16),), dtype=torch.uint8, device="cuda")

        def step_fused_split(rec, pack_v=pack_v, ws_s=ws_s):
            e0, e1 = (ev(), ev()) if rec else (None, None)
            if rec:
                e0.record(stream)
            ja.joint_attn_fwd_bf16_streams_splitkv(qs_d, ks_d, vs_d, scale, n_split=ns_main,
                                                   pack_v=pack_v, workspace=ws_s, out=o)
            if rec:
                e1.record(stream)
            return (e0, e1)

        log("timing fused bf16 split-KV path (%s)" % what)
        wall_fs, durs_fs = timed(step_fused_split, args.steps, args.warmup)
        ms_fs = wall_fs * 1e3 / args.steps
        same = bool(torch.equal(o.view(torch.int16), o_timed.view(torch.int16)))
        out[key] = {
            "step": "fwd_bf16_streams_splitkv, pack_v %d (%s), n_split %d" % (pack_v, what,
                                                                             ns_main),
            "value": round(flops / (ms_fs * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms_fs, 4),
            "call_ms": round(float(durs_fs.mean()), 4),
            "call_tflops": round(flops / (float(durs_fs.mean()) * 1e-3) / 1e12, 2),
            "equals_bf16_step_output": same,
        }
        del ws_s

    # block-sparse forward with a structured 128x128 block mask (text rows and columns,
    # a band of 2 blocks around the diagonal, 15 % of the other image blocks)
    mask = synth.block_mask(w, "structured", 0.15, band=2, seed=4)
    frac = float(mask.mean())
    m_dev = torch.from_numpy(mask).cuda()

    plan = torch.empty((w.B * w.H * mask.shape[-1],), dtype=torch.int32, device="cuda")

    def step_sparse(rec):
        # the planned call (its dispatch plan rebuilt in every step, so the plan's cost is
        # inside the time) and the unplanned one, interleaved so both see the same clock
        e0, e1, e2 = (ev(), ev(), ev()) if rec else (None, None, None)
        if rec:
            e0.record(stream)
        ja.joint_attn_sparse_plan(m_dev, w.N, out=plan)
        ja.joint_attn_fwd_bf16_sparse_planned(q, k, vt, m_dev, plan, scale, out=o)
        if rec:
            e1.record(stream)
        ja.joint_attn_fwd_bf16_sparse(q, k, vt, m_dev, scale, out=o)
        if rec:
            e2.record(stream)
        return (e0, e1, e2)

    log("timing block-sparse bf16 forward (%.1f %% of blocks)" % (100 * frac))
    _, durs_su = timed(step_sparse, args.steps, args.warmup)
    sp_ms = float(durs_su[:, 0].mean())
    out["sparse_bf16"] = {
        "mask": "structured: text rows/columns, band 2, 15 % random", "block": 128,
        "attended_fraction": round(frac, 4),
        "calls": "joint_attn_sparse_plan + joint_attn_fwd_bf16_sparse_planned",
        "kernel_ms": round(sp_ms, 4),
        "effective_tflops": round(flops * frac / (sp_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(fwd_p / sp_ms, 3),
        "unplanned_ms": round(float(durs_su[:, 1].mean()), 4),
    }

    fp8_outputs = {}
    if not args.skip_fp8:
        out["fp8"] = {}
        for mode, name in ((ja.JA_FP8_SPLIT, "split"), (ja.JA_FP8_PLAIN, "plain")):
            t8 = ja.joint_attn_quant_fp8(q, k, vt, mode)
            # the forward through the split-KV call (last round's tiles split), workspace
            # allocated outside the timing
            ns8 = int(ja.load().joint_attn_fwd_fp8_splitkv_suggest(B, H, N, D, mode))
            ws8 = torch.empty((int(ja.load().joint_attn_fwd_fp8_splitkv_workspace(
                B, H, N, D, ns8)),), dtype=torch.uint8, device="cuda")

            def step_fp8(rec, mode=mode, t8=t8, ns8=ns8, ws8=ws8):
                e = [ev() for _ in range(4)] if rec else None
                if rec:
                    e[0].record(stream)
                ja.joint_attn_pack(qs_d, "bhnd", out=q)
                ja.joint_attn_pack(ks_d, "bhnd", out=k)
                ja.joint_attn_pack(vs_d, "bhdn", out=vt)
                if rec:
                    e[1].record(stream)
                ja.joint_attn_quant_fp8(q, k, vt, mode, out=t8)
                if rec:
                    e[2].record(stream)
                ja.joint_attn_fwd_fp8_splitkv(t8, scale, n_split=ns8, workspace=ws8, out=o)
                if rec:
                    e[3].record(stream)
                return e

            log("timing fp8 path, mode %d (%s), split-KV n_split %d" % (mode, name, ns8))
            wall8, durs8 = timed(step_fp8, args.steps, args.warmup)
            fp8_outputs[name] = o.clone()
            ms8 = wall8 * 1e3 / args.steps
            p8, qn8, f8 = durs8.mean(axis=0)

            # the plain fp8 forward alone (every query tile over all keys)
            def step_f8p(rec, t8=t8):
                e = [ev() for _ in range(2)] if rec else None
                if rec:
                    e[0].record(stream)
                ja.joint_attn_fwd_fp8(t8, scale, out=o)
                if rec:
                    e[1].record(stream)
                return e

            _, durs8p = timed(step_f8p, args.steps, args.warmup)
            f8p = float(durs8p.mean())
            out["fp8"][name] = {
                "workload": "t2i_2048_fp8 (same inputs)", "mode": mode,
                "dtype": "fp8 e4m3" + (" + bf16 outlier channels" if mode else "")
                         + " (fp32 accumulate)",
                "value": round(flops / (ms8 * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms8, 4),
                "step": "pack q,k,v + quant_fp8 + fwd_fp8_splitkv (n_split %d)" % ns8,
                "kernels_ms": {"pack_qkv": round(float(p8), 4), "quant_fp8": round(float(qn8), 4),
                               "fwd_fp8_splitkv": round(float(f8), 4)},
                "fwd_fp8_tflops": round(flops / (f8 * 1e-3) / 1e12, 2),
                "frac_of_fp8_peak": round(flops / (f8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                "frac_of_bf16_peak": round(flops / (f8 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "plain_fwd_fp8_ms": round(f8p, 4),
                "plain_fwd_fp8_tflops": round(flops / (f8p * 1e-3) / 1e12, 2),
            }
            del t8, ws8

            # the same fp8 step with the quantiser reading the streams in place (no pack)
            t8s, _ = ja.joint_attn_quant_fp8_streams(qs_d, ks_d, vs_d, mode)

            def step_fp8s(rec, mode=mode, t8s=t8s):
                e = [ev() for _ in range(3)] if rec else None
                if rec:
                    e[0].record(stream)
                ja.joint_attn_quant_fp8_streams(qs_d, ks_d, vs_d, mode, out=t8s)
                if rec:
                    e[1].record(stream)
                ja.joint_attn_fwd_fp8(t8s, scale, out=o)
                if rec:
                    e[2].record(stream)
                return e

            log("timing fp8 path from the streams, mode %d (%s)" % (mode, name))
            wall8s, durs8s = timed(step_fp8s, args.steps, args.warmup)
            ms8s = wall8s * 1e3 / args.steps
            qn8s, f8s = durs8s.mean(axis=0)
            out["fp8"][name + "_streams"] = {
                "mode": mode, "step": "quant_fp8_streams + fwd_fp8 (no pack)",
                "value": round(flops / (ms8s * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms8s, 4),
                "kernels_ms": {"quant_fp8_streams": round(float(qn8s), 4),
                               "fwd_fp8": round(float(f8s), 4)},
            }
            del t8s

        # token repair (the repair budget rho = 0.005 of VC-Attention FP8): plain codes,
        # the ceil(rho N) = 85 worst Q and K tokens per (b, h) back at their exact values
        rho = 0.005
        t8r = ja.joint_attn_quant_fp8_repair(q, k, vt, rho)

        def step_fp8r(rec):
            e = [ev() for _ in range(4)] if rec else None
            if rec:
                e[0].record(stream)
            ja.joint_attn_pack(qs_d, "bhnd", out=q)
            ja.joint_attn_pack(ks_d, "bhnd", out=k)
            ja.joint_attn_pack(vs_d, "bhdn", out=vt)
            if rec:
                e[1].record(stream)
            ja.joint_attn_quant_fp8_repair(q, k, vt, rho, out=t8r)
            if rec:
                e[2].record(stream)
            ja.joint_attn_fwd_fp8_repair(t8r, scale, out=o)
            if rec:
                e[3].record(stream)
            return e

        log("timing fp8 token-repair path (rho %g, %d tokens per (b, h))" % (rho, t8r.n_repair))
        wall8r, durs8r = timed(step_fp8r, args.steps, args.warmup)
        ms8r = wall8r * 1e3 / args.steps
        p8r, qn8r, f8r = durs8r.mean(axis=0)
        out["fp8"]["repair"] = {
            "mode": ja.JA_FP8_REPAIR, "rho": rho, "repaired_tokens_per_bh": t8r.n_repair,
            "dtype": "fp8 e4m3 + repaired tokens' exact values (fp32 accumulate)",
            "value": round(flops / (ms8r * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms8r, 4),
            "step": "pack q,k,v + quant_fp8_repair + fwd_fp8_repair",
            "kernels_ms": {"pack_qkv": round(float(p8r), 4),
                           "quant_fp8_repair": round(float(qn8r), 4),
                           "fwd_fp8_repair": round(float(f8r), 4)},
            "fwd_fp8_tflops": round(flops / (f8r * 1e-3) / 1e12, 2),
            "frac_of_fp8_peak": round(flops / (f8r * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        }
        del t8r

    # context for the roofline: a plain library GEMM (torch.matmul -> hipBLASLt) on random
    # bf16 operands, under the same board power limit, and the clock and power it runs at
    log("timing the reference bf16 GEMM (torch.matmul, 8192^3)")
    g_n = 8192
    ga = torch.randn((g_n, g_n), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gb = torch.randn((g_n, g_n), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gc = torch.empty((g_n, g_n), device="cuda", dtype=torch.bfloat16)

    def step_gemm(rec=True):
        torch.matmul(ga, gb, out=gc)
        return []

    for _ in range(5):
        step_gemm()
    torch.cuda.synchronize()
    g_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    g_ev[0].record()
    for _ in range(20):
        step_gemm()
    g_ev[1].record()
    torch.cuda.synchronize()
    g_ms = g_ev[0].elapsed_time(g_ev[1]) / 20
    g_tf = 2.0 * g_n ** 3 / (g_ms * 1e-3) / 1e12
    out["reference_gemm"] = {
        "op": "torch.matmul, bf16 %d x %d x %d, random normal operands (vendor GEMM)" % (g_n, g_n, g_n),
        "ms": round(g_ms, 4), "tflops": round(g_tf, 1),
        "frac_of_bf16_peak": round(g_tf / PEAK_BF16_TFLOPS, 4),
        "timed_forward_over_gemm": round(achieved / g_tf, 4)}
    out["reference_gemm"].update(sustained_clock(step_gemm, g_ms))
    del ga, gb, gc

    if not args.skip_shapes:
        # forward-only throughput of the other shapes: 1024^2 T2I and 2048^2 I2I from the
        # same generator, and one GPU's share of a Ulysses head split of 2048^2 T2I
        # (batch element 0, the first 6 or 3 of the 24 heads: what a rank would hold)
        def time_fwd(call, steps, warmup):
            for _ in range(warmup):
                call()
            evs = [(ev(), ev()) for _ in range(steps)]
            for a, b2 in evs:
                a.record(stream)
                call()
                b2.record(stream)
            torch.cuda.synchronize()
            return np.asarray([a.elapsed_time(b2) for a, b2 in evs])

        def shape_row(wl, qq, kk, vv, steps):
            Bq, Hq, Nq, Dq = (int(x) for x in qq.shape)
            oo = torch.empty((Bq, Nq, Hq, Dq), dtype=torch.bfloat16, device="cuda")
            d = time_fwd(lambda: ja.joint_attn_fwd_bf16(qq, kk, vv, scale, out=oo), steps, 2)
            fl = 4.0 * Bq * Hq * Nq ** 2 * Dq
            tf = fl / (d.mean() * 1e-3) / 1e12
            row = {"B": Bq, "H": Hq, "N": Nq,
                   "stream_lens": list(wl), "fwd_bf16_ms_mean": round(float(d.mean()), 4),
                   "fwd_bf16_ms_median": round(float(np.median(d)), 4),
                   "fwd_bf16_ms_min": round(float(d.min()), 4),
                   "fwd_bf16_tflops": round(tf, 2),
                   "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            # grids of fewer than ~4 workgroups per CU: the split-KV forward (key ranges
            # in parallel + a log-sum-exp merge), workspace allocated outside the timing
            ns = int(ja.load().joint_attn_fwd_bf16_splitkv_suggest(Bq, Hq, Nq, Dq))
            if ns > 1:
                wsb = int(ja.load().joint_attn_fwd_bf16_splitkv_workspace(Bq, Hq, Nq, Dq, ns))
                wsp = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
                ds = time_fwd(lambda: ja.joint_attn_fwd_bf16_splitkv(
                    qq, kk, vv, scale, n_split=ns, workspace=wsp, out=oo), steps, 2)
                tfs = fl / (ds.mean() * 1e-3) / 1e12
                row.update({"splitkv_n_split": ns,
                            "fwd_bf16_splitkv_ms_mean": round(float(ds.mean()), 4),
                            "fwd_bf16_splitkv_tflops": round(tfs, 2),
                            "splitkv_frac_of_bf16_peak": round(tfs / PEAK_BF16_TFLOPS, 4)})
                del wsp
            return row

        shapes = {}
        for hs, name in ((6, "ulysses4_share_t2i_2048"), (3, "ulysses8_share_t2i_2048")):
            log("timing %s" % name)
            shapes[name] = shape_row(w.stream_lens, q[:1, :hs].contiguous(),
                                     k[:1, :hs].contiguous(), vt[:1, :hs].contiguous(),
                                     args.steps)
        for name in ("t2i_1024_bf16", "i2i_2048_bf16", "i2i_1024_r1_bf16", "i2i_1024_r3_bf16",
                     "i2i_2048_r3_bf16"):
            w2 = synth.WORKLOADS[name]
            log("generating and timing %s (N=%d)" % (name, w2.N))
            st2 = synth.make_streams(w2)
            q2, _ = ja.joint_attn_pack([dev(x) for x in st2.q], "bhnd")
            k2, _ = ja.joint_attn_pack([dev(x) for x in st2.k], "bhnd")
            v2, _ = ja.joint_attn_pack([dev(x) for x in st2.v], "bhdn")
            del st2
            shapes[name] = shape_row(w2.stream_lens, q2, k2, v2, args.steps)
            del q2, k2, v2
        out["shapes"] = shapes

    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle)")
        qh, _ = oracle.pack_tokens(st.q)
        kh, _ = oracle.pack_tokens(st.k)
        vh, _ = oracle.pack_tokens(st.v)
        cb = cpu_baseline(w, (qh, kh, vh), args.cpu_seconds)
        cb.pop("seconds")
        rows, ref = cb.pop("rows"), cb.pop("ref")
        out["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2)
                               for k2, v2 in cb.items()}

        # parity of the timed steps' outputs on the same oracle rows (bf16 bar: rel_F <=
        # 5e-3, max|err| <= 2e-2; fp8 against the unquantised fp64 oracle: rel_F <= 5e-2
        # for the split mode, the plain mode's recipe loss reported)
        def rows_of(t):
            bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
            bits = bits[rows[:, 0], rows[:, 2], rows[:, 1], :]
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

        def parity(t):
            got = rows_of(t)
            return {"rows": int(len(rows)),
                    "rel_F": float("%.4g" % (np.linalg.norm(got - ref) / np.linalg.norm(ref))),
                    "max_abs_err": float("%.4g" % np.abs(got - ref).max())}
        out["parity"] = {"reference": "fp64 oracle, the cpu_baseline rows",
                         "bf16_step": parity(o_timed)}
        out["parity"]["bf16_step"]["within_bar"] = bool(
            out["parity"]["bf16_step"]["rel_F"] <= 5e-3 and
            out["parity"]["bf16_step"]["max_abs_err"] <= 2e-2)
        for name, t in fp8_outputs.items():
            out["parity"]["fp8_%s_step" % name] = parity(t)
    print(json.dumps(out), flush=True)
    try:                       # anything this process started that is still alive
        import psutil
        kids = psutil.Process().children(recursive=True)
        if kids:
            log("child processes still alive at exit: %s"
                % ", ".join("%d %s" % (c.pid, " ".join(c.cmdline()[:4])) for c in kids))
    except Exception as e:
        log("child-process check failed: %r" % (e,))


if __name__ == "__main__":
    main()
