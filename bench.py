"""Benchmark: causal FP8 prefill attention throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gauss32k]
                    [--mode lean|exact] [--dtype fp8|bf16] [--no-cpu-baseline]

One step = one attn_fwd_fp8 call over the whole workload (Q,K,V resident in HBM
when timing starts).  Throughput uses the causal FLOP count
2*B*Hq*S^2*(d_qk+d_v)/2.  Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal prefill attention TFLOP/s & % FP8 peak (d=128, S=32K); RMS err vs fp64"
# MI355X published dense peaks, TFLOP/s
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
PEAK_SCLK_MHZ = 2400.0          # the shader clock those peaks assume
# The pages' own figure for this workload (ZYFA, FP8, d=128, 32K tokens, Gaussian inputs, MI355X)
PAGES_TFLOPS = {("gauss32k", "fp8"): 2672.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gauss32k")
    ap.add_argument("--mode", default="lean", choices=["lean", "exact"])
    ap.add_argument("--dtype", default="fp8", choices=["fp8", "bf16"])
    ap.add_argument("--both-modes", action="store_true", default=True,
                    help="also time the other FP8 probability path (reported under 'paths')")
    ap.add_argument("--no-both-modes", dest="both_modes", action="store_false")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-rotate", action="store_true",
                    help="skip timing the Hadamard rotation + quantisation of Q and K")
    ap.add_argument("--input-study", action="store_true", default=True,
                    help="also time the FP8 kernel on low-bit-activity inputs (sparse, zero Q) with power "
                         "and clock samples (reported under 'input_study'; on by default)")
    ap.add_argument("--no-input-study", dest="input_study", action="store_false")
    ap.add_argument("--extra-workloads", default="mla:fp8,qwen:bf16",
                    help="comma-separated workload:dtype pairs timed after the headline and reported under "
                         "'other_workloads' (empty to skip); FP8 ones run both probability paths")
    ap.add_argument("--emu-rows", type=int, default=256,
                    help="long query rows per head on which the CPU leg also runs the step-by-step emulation "
                         "of the FP8 method (0 to skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a known-size kernel for scaling HBM byte counters)")
    return ap.parse_args()


def _dpm_current_mhz(path):
    """The level marked '*' in an amdgpu pp_dpm_sclk table, in MHz (None if unreadable)."""
    try:
        for ln in open(path):
            if ln.rstrip().endswith("*"):
                v = ln.split(":", 1)[1].strip().rstrip("*").strip().lower()
                return float(v.replace("mhz", ""))
    except Exception:
        pass
    return None


def sclk_mhz():
    """Current shader clock (MHz) from the amdgpu sysfs DPM table, None if unavailable.

    Read from a file: no helper program is started after the GPU is initialised."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        v = _dpm_current_mhz(path)
        if v is not None:
            return v
    return None


def _gpu_hwmon_dirs():
    """sysfs device directories of the DRM cards whose PCI address is torch's cuda:0 (or, failing
    that, of the only card with a DPM clock table).  Read-only file access."""
    import glob
    cards = [c for c in sorted(glob.glob("/sys/class/drm/card*/device")) if os.path.exists(c + "/pp_dpm_sclk")]
    try:
        import torch
        pr = torch.cuda.get_device_properties(0)
        want = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}"
        match = [c for c in cards if os.path.basename(os.path.realpath(c)).startswith(want)]
        if match:
            return match[:1]
    except Exception:
        pass
    return cards if len(cards) == 1 else []


class PowerClockSampler:
    """Samples the GPU's board power and shader clock from sysfs hwmon in a background thread
    while the timed launches run (file reads only; nothing is executed)."""

    def __init__(self, period_s=0.002):
        import glob
        self.period = period_s
        self.power_file, self.clock_file, self.dpm_file, self.power_cap_w = None, None, None, None
        for dev in _gpu_hwmon_dirs():
            for hw in sorted(glob.glob(dev + "/hwmon/hwmon*")):
                for name in ("power1_average", "power1_input"):
                    if self.power_file is None and os.path.exists(f"{hw}/{name}"):
                        self.power_file = f"{hw}/{name}"
                if os.path.exists(f"{hw}/freq1_input"):
                    self.clock_file = f"{hw}/freq1_input"
                cap = self._read(f"{hw}/power1_cap")
                if cap is not None:
                    self.power_cap_w = cap * 1e-6
            if self.clock_file is None and os.path.exists(dev + "/pp_dpm_sclk"):
                self.dpm_file = dev + "/pp_dpm_sclk"     # current DPM level, marked '*'
        self.power, self.clock = [], []
        self._stop = None
        self._thread = None

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return float(f.read().strip())
        except Exception:
            return None

    def _run(self):
        while not self._stop.is_set():
            if self.power_file:
                v = self._read(self.power_file)
                if v is not None:
                    self.power.append(v * 1e-6)          # microwatts -> W
            if self.clock_file:
                v = self._read(self.clock_file)
                if v is not None:
                    self.clock.append(v * 1e-6)          # Hz -> MHz
            elif self.dpm_file:
                v = _dpm_current_mhz(self.dpm_file)
                if v is not None:
                    self.clock.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        self.power, self.clock = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self, flop, seconds):
        """Average power (W), shader clock (MHz), and FLOP per joule over the sampled window."""
        p = sum(self.power) / len(self.power) if self.power else None
        c = sum(self.clock) / len(self.clock) if self.clock else None
        return {"power_w_avg": p, "power_cap_w": self.power_cap_w, "sclk_mhz_avg": c,
                "samples": len(self.power), "tflop_per_joule": (flop / (p * seconds) / 1e12) if p else None,
                "power_source": self.power_file, "clock_source": self.clock_file or self.dpm_file}


def sources_sha16(paths):
    """First 16 hex digits of the sha256 of the concatenated files (paths relative to the repo)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_counters(workload, mode):
    """The committed rocprofv3 counter record (profiles/traffic.json) for this workload and
    probability path, or None when the kernel's code has changed since those counters were
    taken (or no record exists).  The record names the files that make the kernel (its
    source, the headers it includes, the build script with its compiler flags) and the
    sha256 of their concatenation."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(path))
        digest = sources_sha16(t.get("sources") or [t["source"]])
    except Exception:
        return None
    if digest != t["source_sha256_16"]:
        return None
    if t["workload"] != workload or t["p_mode"] != mode:
        return None
    return t


def measured_traffic(workload, mode):
    """HBM bytes per launch from the committed counters, or None (see committed_counters)."""
    t = committed_counters(workload, mode)
    return None if t is None else t["hbm_read_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]


def valu_roofline(workload, mode):
    """The vector-side figures of the committed counters: vector instructions per score and lane
    (MFMA issue excluded) against the pages' budgets, and the vector pipe's share of the kernel's
    cycles at one wave64 instruction per 4 cycles per SIMD; None when stale (see
    committed_counters)."""
    t = committed_counters(workload, mode)
    if t is None or "valu_per_score" not in t:
        return None
    return {"bound": "valu", "valu_instructions_per_score": t["valu_per_score"],
            "pages_budget_per_score": {"exact": 3.5, "lean": 1.5},
            "valu_cycles_frac": t["valu_cycles_frac"], "mfma_busy_frac": t["mfma_busy_frac"],
            "source": t["summary"]}


def time_launches(fn, steps, warmup, stream, sampler=None):
    import contextlib
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    with sampler if sampler is not None else contextlib.nullcontext():
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))   # ms, HIP events on the launch stream
    return wall, per


HBM_PEAK_GBPS = 8000.0


def time_batched(fn, steps, warmup, stream):
    """Average ms per call of `steps` back-to-back calls between one pair of HIP events on the
    launch stream (for kernels of tens of microseconds, where an event pair around every
    call would add its own overhead to each)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def rotate_quant_timing(w, steps, warmup, stream, attn_ms):
    """Time attn_rotate_quant_bf16 on bf16 tensors of the workload's Q and K shapes
    (seeded N(0,1), resident in HBM).  HBM roofline of the pass: algorithmic bytes =
    the bf16 tensor read once + one e4m3 byte per element written."""
    import torch
    from fp8_causal_prefill_tiled_amd import binding
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(20261202)
    res, pre = {}, {}
    for name, h in (("q", w.Hq), ("k", w.Hkv)):
        x = torch.randn((w.B, w.S, h, w.d_qk), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        out = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        sc = torch.empty(1, dtype=torch.float32, device=dev)
        ms = time_batched(lambda: binding.rotate_quant_bf16(x, out=out, scale=sc, stream=stream), steps, warmup,
                          stream)
        nbytes = x.numel() * 3
        res[name] = {"shape": list(x.shape), "kernel_ms_avg": ms, "algorithmic_bytes": nbytes,
                     "achieved_GBps": nbytes / (ms * 1e-3) / 1e9}
        # one pass with the scale known in advance (here: the one just computed)
        pms = time_batched(lambda: binding.rotate_quant_bf16_prescaled(x, sc, out=out, stream=stream), steps,
                           warmup, stream)
        pre[name] = {"kernel_ms_avg": pms, "achieved_GBps": nbytes / (pms * 1e-3) / 1e9}
        del x, out
    # what plain streaming reaches on this GPU with the same traffic: torch's own bf16 -> e4m3
    # cast of the Q-shaped tensor (read 2 bytes, write 1 byte per element, no rotation)
    x = torch.randn((w.B, w.S, w.Hq, w.d_qk), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    z = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev)
    cast_ms = time_batched(lambda: z.copy_(x), steps, warmup, stream)
    cast_gbps = x.numel() * 3 / (cast_ms * 1e-3) / 1e9
    del x, z
    total_ms = res["q"]["kernel_ms_avg"] + res["k"]["kernel_ms_avg"]
    total_bytes = res["q"]["algorithmic_bytes"] + res["k"]["algorithmic_bytes"]
    achieved = total_bytes / (total_ms * 1e-3) / 1e9
    pre_ms = pre["q"]["kernel_ms_avg"] + pre["k"]["kernel_ms_avg"]
    pre_gbps = total_bytes / (pre_ms * 1e-3) / 1e9
    return {"kernels": "rq_stream max pass + rq_stream quantise pass (+ two 1-thread kernels), Q then K", "q": res["q"], "k": res["k"],
            "ms_q_plus_k": total_ms, "fraction_of_attention_time": total_ms / attn_ms,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBPS, "traffic": None},
            "plain_cast_reference": {"what": "torch bf16 -> e4m3 cast of the Q-shaped tensor (same bytes, no rotation)",
                                     "kernel_ms_avg": cast_ms, "achieved_GBps": cast_gbps,
                                     "frac_of_peak": cast_gbps / HBM_PEAK_GBPS},
            "prescaled": {"kernels": "rq_init + rq_stream quantising with the caller's scale, with an amax output (one pass)",
                          "q": pre["q"], "k": pre["k"], "ms_q_plus_k": pre_ms,
                          "fraction_of_attention_time": pre_ms / attn_ms,
                          "roofline": {"bound": "hbm", "achieved": pre_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                       "frac": pre_gbps / HBM_PEAK_GBPS, "traffic": None}}}


def sparse_codes(x, frac=0.9, sample=1 << 20):
    """e4m3 codes x (uint8 tensor, any device) with every code whose magnitude is below the
    `frac` quantile of |code| set to +0.  The quantile comes from an evenly strided sample taken
    as a strided view (no index tensor), moved to the host."""
    import torch
    flat = x.reshape(-1)
    picked = (flat[:: max(1, flat.numel() // sample)] & 0x7F).cpu().float()
    thr = torch.kthvalue(picked, max(1, int(frac * picked.numel()))).values.item()
    return torch.where((x & 0x7F) < thr, torch.zeros_like(x), x)


def input_study(w, d, q, k, v, out, stream, flops, steps, warmup, modes, paths):
    """Throughput, shader clock, power and TFLOP/J of the FP8 kernel on inputs with less operand
    bit activity than Gaussian ones (the pages: the sustained clock depends on how many operand
    bits flip).  Same shapes, same FLOP count, same kernel:
      gaussian - the workload itself (from `paths`);
      sparse90 - Q, K and V codes of magnitude below each tensor's 90th percentile set to +0;
      zero_q   - Q = 0: every score is 0, so every probability byte is the same (e4m3 256)."""
    import torch
    from fp8_causal_prefill_tiled_amd import binding

    variants = {"sparse90": (sparse_codes(q), sparse_codes(k), sparse_codes(v)),
                "zero_q": (torch.zeros_like(q), k, v)}
    out = torch.empty_like(out)       # the headline output stays as it is
    res = {"gaussian": {m: {"tflops": paths[m]["tflops"], **paths[m]["energy"]} for m in modes}}
    sampler = PowerClockSampler()
    for name, (qq, kk, vv) in variants.items():
        res[name] = {}
        for mode in modes:
            def fn():
                binding.attn_fwd_fp8(qq, kk, vv, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode, out=out,
                                     stream=stream)
            wall, per = time_launches(fn, steps, warmup, stream, sampler)
            res[name][mode] = {"tflops": flops * steps / wall / 1e12, **sampler.summary(flops * steps, wall)}
        del qq
    torch.cuda.synchronize()
    return res


def other_workloads(spec, steps, warmup, stream):
    """Throughput, power and clock of the kernels on further workloads (BASELINE configs other than
    the headline): each runs alone on freshly drawn inputs, FP8 ones on both probability paths."""
    import torch
    from fp8_causal_prefill_tiled_amd import binding
    from fp8_causal_prefill_tiled_amd import workloads as W
    res = {}
    dev = torch.device("cuda:0")
    sampler = PowerClockSampler()
    for item in [x for x in spec.split(",") if x]:
        name, dtype = item.split(":")
        w = W.WORKLOADS[name]
        flops, peak = w.causal_flops, PEAK_TFLOPS[dtype]
        out = torch.empty((w.B, w.S, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)
        if dtype == "fp8":
            d = W.make_fp8(w)
            q, k, v = (d[n].to(dev) for n in ("q8", "k8", "v8"))
            fns = {m: (lambda m=m: binding.attn_fwd_fp8(q, k, v, d["q_scale"], d["k_scale"], d["v_scale"],
                                                        p_mode=m, out=out, stream=stream)) for m in ("lean", "exact")}
        else:
            d = W.make_bf16(w)
            q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
            fns = {"bf16": lambda: binding.attn_fwd_bf16(q, k, v, out=out, stream=stream)}
        torch.cuda.synchronize()
        entry = {"workload": name, "dtype": dtype, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "d_qk": w.d_qk,
                 "d_v": w.d_v, "causal_tflop_per_step": flops / 1e12, "paths": {}}
        for m, fn in fns.items():
            for _ in range(3 * warmup):           # settle the power and clock readings first
                fn()
            wall, per = time_launches(fn, steps, warmup, stream, sampler)
            avg_ms = sum(per) / len(per)
            entry["paths"][m] = {"tflops": flops * steps / wall / 1e12, "kernel_ms_avg": avg_ms,
                                 "frac_of_peak": flops / (avg_ms * 1e-3) / 1e12 / peak,
                                 "energy": sampler.summary(flops * steps, wall)}
        res[f"{name}_{dtype}"] = entry
        del q, k, v, out, d
        torch.cuda.synchronize()
    return res


def _e4m3_floor(mode, n=200_000):
    """Closed-form relative RMS error floor of rounding every probability of a long row to e4m3
    (log2 of the probability uniform modulo 1; the rounded-sum normalisation cancels the mean):
    sd(delta) / (1 + mean(delta)), delta the relative rounding error of one probability."""
    import numpy as np
    f = (np.arange(n) + 0.5) / n
    m = 2.0 ** f
    if mode == "exact":
        val = np.round(8.0 * m) / 8.0
    else:
        code = np.rint(8.0 * f + 56.0)
        val = 2.0 ** (np.floor(code / 8.0) - 7.0) * (1.0 + (code % 8.0) / 8.0)
    delta = val / m - 1.0
    return float(delta.std() / (1.0 + delta.mean()))


def emulation_leg(w, d, outs, n_rows):
    """The step-by-step emulation of the FP8 method (oracle/emulate.py) and fp64 attention on n_rows
    query rows drawn from the second half of the sequence (long causal rows) for three heads: the
    method's own error against fp64 there, the GPU's distance to the emulation, and the closed-form
    e4m3 floor the method's error should sit at."""
    import numpy as np
    from oracle.attention64 import attention_fp64, dequantize
    from oracle.emulate import emulate_fp8
    g = np.random.default_rng(20261202)
    rows = np.sort(g.choice(np.arange(w.S // 2, w.S), size=min(n_rows, w.S // 2), replace=False))
    heads = [0, w.Hq // 2, w.Hq - 1]
    t0 = time.perf_counter()
    res = {m: {"emu": [], "gpu": [], "gpu_emu": []} for m in outs}
    for h in heads:
        gk = h // (w.Hq // w.Hkv)
        q8, k8, v8 = d["q8"][:, :, h:h + 1].numpy(), d["k8"][:, :, gk:gk + 1].numpy(), d["v8"][:, :, gk:gk + 1].numpy()
        ref = attention_fp64(dequantize(q8, d["q_scale"]), dequantize(k8, d["k_scale"]), dequantize(v8, d["v_scale"]),
                             rows=rows)
        for m, o in outs.items():
            emu = emulate_fp8(q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=m, rows=rows)
            got = o[:, rows, h:h + 1].astype(np.float64)

            def per_row(x, y):
                return np.sqrt(np.sum((x - y) ** 2, axis=-1) / np.sum(y ** 2, axis=-1)).reshape(-1)
            res[m]["emu"].append(per_row(emu, ref))
            res[m]["gpu"].append(per_row(got, ref))
            res[m]["gpu_emu"].append(per_row(got, emu))
    out = {"rows": f"{len(rows)} rows drawn uniformly from {w.S // 2}..{w.S - 1} x heads {heads}",
           "seconds": time.perf_counter() - t0}
    for m, r in res.items():
        e, gg, ge = (np.concatenate(r[k]) for k in ("emu", "gpu", "gpu_emu"))
        out[m] = {"emulation_rel_rms_vs_fp64": float(np.sqrt(np.mean(e ** 2))),
                  "gpu_rel_rms_vs_fp64": float(np.sqrt(np.mean(gg ** 2))),
                  "gpu_rel_rms_vs_emulation": float(np.sqrt(np.mean(ge ** 2))),
                  "gpu_vs_emulation_per_row_median": float(np.median(ge)),
                  "gpu_vs_emulation_per_row_max": float(np.max(ge)),
                  "e4m3_floor_closed_form": _e4m3_floor(m),
                  "note": "RMS over rows of each row's relative RMS error (rows weighted equally)"}
    return out


def cpu_baseline(w, d, outs, seconds, dtype, emu_rows=0):
    """Time the CPU oracle (fp64 attention) on a bounded sample of the same workload and
    compare the GPU outputs on those rows.  Returns the cpu_baseline object.

    outs: {path: GPU output as a float array}, the headline path first.
    Sample: query rows spread over 0..S-1 (every 64th row, longest causal prefixes first, then
    the next residue), in chunks of 64, for three heads, until about `seconds` of oracle time
    has been spent.  The GPU error is measured against fp64 attention on the dequantised inputs
    (the method's own error) and, for FP8, also on the unquantised fp32 draws (input quantisation
    included); only the first is timed."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle.attention64 import attention_fp64, dequantize

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    S = w.S
    order = np.arange(S - 1, -1, -1, dtype=np.int64)[np.argsort(np.arange(S) % 64, kind="stable")]
    heads = [0, w.Hq // 2, w.Hq - 1]
    per_head = []
    for h in heads:
        g = h // (w.Hq // w.Hkv)
        if dtype == "fp8":
            per_head.append((h, dequantize(d["q8"][:, :, h:h + 1].numpy(), d["q_scale"]),
                             dequantize(d["k8"][:, :, g:g + 1].numpy(), d["k_scale"]),
                             dequantize(d["v8"][:, :, g:g + 1].numpy(), d["v_scale"])))
        else:
            per_head.append((h, d["q"][:, :, h:h + 1].float().numpy(), d["k"][:, :, g:g + 1].float().numpy(),
                             d["v"][:, :, g:g + 1].float().numpy()))
    raw = None
    if dtype == "fp8":
        from fp8_causal_prefill_tiled_amd import workloads as W
        q32, k32, v32 = W.draw_fp32(w)          # the same seeded draws the codes were quantised from
        raw = {h: (q32[:, :, h:h + 1].numpy(), k32[:, :, h // (w.Hq // w.Hkv):h // (w.Hq // w.Hkv) + 1].numpy(),
                   v32[:, :, h // (w.Hq // w.Hkv):h // (w.Hq // w.Hkv) + 1].numpy()) for h in heads}
        del q32, k32, v32
    flops, el, nrows = 0.0, 0.0, 0
    err = {m: {"deq": [0.0, 0.0], "raw": [0.0, 0.0], "head": {h: [0.0, 0.0] for h in heads}} for m in outs}
    i = 0
    while el < seconds and i < len(order):
        rows = np.sort(order[i:i + 64])
        i += 64
        nrows += len(rows)
        for h, q, k, v in per_head:
            t0 = time.perf_counter()
            ref = attention_fp64(q, k, v, rows=rows)
            el += time.perf_counter() - t0
            flops += float(np.sum(2.0 * (rows + 1) * (w.d_qk + w.d_v)))
            ref_raw = attention_fp64(*raw[h], rows=rows) if raw is not None else None
            for m, out_gpu in outs.items():
                got = out_gpu[:, rows, h:h + 1].astype(np.float64)
                e2, r2 = float(np.sum((got - ref) ** 2)), float(np.sum(ref ** 2))
                for acc in (err[m]["deq"], err[m]["head"][h]):
                    acc[0] += e2
                    acc[1] += r2
                if ref_raw is not None:
                    err[m]["raw"][0] += float(np.sum((got - ref_raw) ** 2))
                    err[m]["raw"][1] += float(np.sum(ref_raw ** 2))

    def rel(a):
        return float(np.sqrt(a[0] / a[1])) if a[1] > 0 else None
    errors = {m: {"rel_rms_vs_fp64_dequantised_inputs": rel(e["deq"]),
                  "rel_rms_vs_fp64_unquantised_inputs": rel(e["raw"]) if raw is not None else None,
                  "per_head_max_rel_rms_dequantised": max(rel(v) for v in e["head"].values())}
              for m, e in err.items()}
    tiny = _cpu_tiny_full()
    emu = emulation_leg(w, d, outs, emu_rows) if dtype == "fp8" and emu_rows > 0 else None
    return {
        "value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "tiny_full": tiny,
        "sample": f"fp64 attention (oracle/attention64.py, numpy+BLAS) on {nrows} query rows "
                  f"(spread over 0..S-1, longest prefixes first) x heads {heads} of the {w.name} workload, "
                  f"{el:.1f} s of oracle time; FLOPs counted 2*(i+1)*(d_qk+d_v) per row i",
        "gpu_rel_rms_vs_oracle_on_sample": errors[next(iter(outs))]["rel_rms_vs_fp64_dequantised_inputs"],
        "gpu_error_on_sample": errors,
        "method_error_on_long_rows": emu,
        "cpu_model": _cpu_model(),
        "os_cpu_count": os.cpu_count(),
    }


def _cpu_tiny_full():
    """The oracle on the whole tiny workload (B=1, H=2, S=256, d=128, FP8 inputs dequantised), on
    all threads and on one thread; best of three runs each, TFLOP/s by the causal formula."""
    from threadpoolctl import threadpool_limits
    from oracle.attention64 import attention_fp64, dequantize
    from fp8_causal_prefill_tiled_amd import workloads as W
    tw = W.WORKLOADS["tiny"]
    td = W.make_fp8(tw)
    q, k, v = (dequantize(td[n + "8"].numpy(), td[n + "_scale"]) for n in ("q", "k", "v"))

    def best():
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            attention_fp64(q, k, v)
            ts.append(time.perf_counter() - t0)
        return min(ts)
    t_all = best()
    with threadpool_limits(limits=1):
        t_one = best()
    return {"workload": "tiny (B=1, Hq=Hkv=2, S=256, d=128)", "all_threads_tflops": tw.causal_flops / t_all / 1e12,
            "one_thread_tflops": tw.causal_flops / t_one / 1e12, "all_threads_s": t_all, "one_thread_s": t_one}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); heads are "
              f"independent, so a multi-GPU run is one independent launch per GPU on its share of heads.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from fp8_causal_prefill_tiled_amd import binding
    from fp8_causal_prefill_tiled_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    flops = w.causal_flops
    peak = PEAK_TFLOPS[args.dtype]

    if args.dtype == "fp8":
        d = W.make_fp8(w)
        q, k, v = (d[n].to(dev) for n in ("q8", "k8", "v8"))
        out = torch.empty((w.B, w.S, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)

        def make_fn(mode):
            return lambda: binding.attn_fwd_fp8(q, k, v, d["q_scale"], d["k_scale"], d["v_scale"],
                                                p_mode=mode, out=out, stream=stream)
        modes = [args.mode] + ([m for m in ("lean", "exact") if m != args.mode] if args.both_modes else [])
    else:
        d = W.make_bf16(w)
        q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
        out = torch.empty((w.B, w.S, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)

        def make_fn(mode):
            return lambda: binding.attn_fwd_bf16(q, k, v, out=out, stream=stream)
        modes = ["exact"]
    torch.cuda.synchronize()

    paths = {}
    clk_before = sclk_mhz()
    sampler = PowerClockSampler()
    if len(modes) > 1:
        # untimed pre-heat of the path timed first, so that its power and clock samples are not
        # taken while the firmware's readings still ramp up from an idle GPU
        fn = make_fn(modes[-1])
        for _ in range(3 * args.warmup):
            fn()
        torch.cuda.synchronize()
    for mode in reversed(modes):          # headline mode last: its output stays in `out`
        wall, per = time_launches(make_fn(mode), args.steps, args.warmup, stream, sampler)
        avg_ms = sum(per) / len(per)
        paths[mode] = {
            "tflops": flops * args.steps / wall / 1e12,
            "ms_per_step": wall / args.steps * 1e3,
            "kernel_ms_avg": avg_ms, "kernel_ms_median": per[len(per) // 2],
            "kernel_ms_min": per[0], "kernel_ms_max": per[-1],
            "frac_of_peak": flops / (avg_ms * 1e-3) / 1e12 / peak,
            "energy": sampler.summary(flops * args.steps, wall),
        }
        # the same fraction against the dense peak scaled to the sampled DPM clock (peak at 2.4 GHz)
        mhz = paths[mode]["energy"].get("sclk_mhz_avg")
        paths[mode]["frac_of_peak_at_sampled_sclk"] = (
            paths[mode]["frac_of_peak"] * PEAK_SCLK_MHZ / mhz if mhz else None)
    clk_after = sclk_mhz()
    study = None
    if args.input_study and args.dtype == "fp8":
        study = input_study(w, d, q, k, v, out, stream, flops, args.steps, args.warmup, modes, paths)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    head = paths[modes[0]]
    value = head["tflops"]
    achieved = flops / (head["kernel_ms_avg"] * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        outs = {modes[0]: out.float().cpu().numpy()}
        for m in modes[1:]:                       # the other probability path, one more launch
            o2 = torch.empty_like(out)
            binding.attn_fwd_fp8(q, k, v, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=m, out=o2, stream=stream)
            torch.cuda.synchronize()
            outs[m] = o2.float().cpu().numpy()
            del o2
        cpu = cpu_baseline(w, d, outs, args.cpu_seconds, args.dtype, args.emu_rows)

    rot = None
    if args.dtype == "fp8" and not args.no_rotate:
        rot = rotate_quant_timing(w, args.steps, args.warmup, stream, head["kernel_ms_avg"])

    others = None
    if args.extra_workloads:
        del q, k, v
        torch.cuda.synchronize()
        others = other_workloads(args.extra_workloads, args.steps, args.warmup, stream)

    pages = PAGES_TFLOPS.get((w.name, args.dtype))
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (value / pages) if pages else None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1), per-tensor e4m3 quantisation)" if args.dtype == "fp8"
                else "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "d_qk": w.d_qk,
                   "d_v": w.d_v, "causal": True, "p_mode": modes[0] if args.dtype == "fp8" else None,
                   "causal_tflop_per_step": flops / 1e12},
        "frac_of_peak": value / peak,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak,
                     "traffic": measured_traffic(w.name, modes[0]) if args.dtype == "fp8" else None,
                     "kernel": ("fp8_causal_fwd_pair" if modes[0] == "lean" else "fp8_causal_fwd")
                               if args.dtype == "fp8" else "bf16_causal_fwd",
                     "per_launch_tflop": flops / 1e12},
        "valu_roofline": valu_roofline(w.name, modes[0]) if args.dtype == "fp8" else None,
        "paths": paths,
        "rotate_quant": rot,
        "input_study": study,
        "other_workloads": others,
        "sclk_mhz": {"before": clk_before, "after": clk_after},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
