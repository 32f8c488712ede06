#!/usr/bin/env python3
"""Benchmark: one step = the whole hot path once -- a causal bf16 FlashAttention
forward (B1 Hq32 N8192 d128, inputs 0.5*N(0,1)) followed by a paged bf16 decode
(64 sequences, Hq32 Hkv8 d128, context U[1024,16384], 16-token pages).

Prints ONE JSON line.  `value` is the forward's throughput in TFLOP/s (causal FLOPs
counted as half: 2*B*Hq*N^2*d) from HIP events around its launches; the decode's
GB/s (algorithmic bytes: every valid K/V token once, plus q, O, L, the used page
table entries and ctx_lens) is reported beside it.  Both carry a roofline object
against the MI355X peaks (bf16 dense MFMA 2516.6 TFLOP/s = 256 CU x 2.4 GHz x 4096
flop/clk; HBM3E 8000 GB/s).  `cpu_baseline` times the fp64 CPU oracle on a bounded
sample of the same workload.

Every timed measurement is warmed for at least --settle-ms of load first, the step
for at least --step-settle-ms; the JSON line records the warm-up, per-step mean/median/min, the graphics
clock sampled during the run, the software versions, and the errors of the timed
step's outputs against the fp64 oracle (`numerics`).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 200] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak; paged decode GB/s + % HBM peak"
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3
PREFILL = "c3_bf16_causal_B1_H32_N8192_d128"
DECODE = "c5_bf16_paged_decode_S64_Hq32_Hkv8_d128"
OTHER_PREFILL = ("c1_f32_B1_H1_N256_d64", "c2_bf16_B4_H16_N2048_d64", "c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128",
                 "c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def warm(fn, n_min, ms_min=100.0):
    """Untimed launches before a measurement: at least n_min, and at least ms_min of
    wall time, since the GPU clock takes tens of milliseconds of load to settle (a
    short kernel warmed by a few launches is timed at a lower clock).  Returns
    (launches, milliseconds)."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < n_min or (time.perf_counter() - t0) * 1e3 < ms_min:
        fn()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i, (time.perf_counter() - t0) * 1e3


class ClockSampler:
    """The GPU's current graphics clock, sampled through amdsmi on a host thread while
    launches run (a driver query; nothing is enqueued on the GPU).  Reports min, mean
    and max MHz per phase, or why no reading was possible."""

    def __init__(self, period_s=0.002):
        import threading

        self.period = period_s
        self.samples = {}
        self.phase = None
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            h = self._match(amdsmi, handles)
            clk = amdsmi.AmdSmiClkType.GFX

            def read():
                # mean of the per-XCD graphics clocks of the firmware's metrics table,
                # else the driver's current-clock query
                try:
                    v = [float(x) for x in amdsmi.amdsmi_get_gpu_metrics_info(h)["current_gfxclks"]
                         if isinstance(x, (int, float)) and 0 < x < 10000]
                    if v:
                        return sum(v) / len(v)
                except Exception:
                    pass
                return float(amdsmi.amdsmi_get_clock_info(h, clk)["clk"])

            self._read = read
            self._read()
        except Exception as e:  # no amdsmi, no permission, no device: report it, keep measuring
            self.error = f"{type(e).__name__}: {e}"[:200]
            self._read = None

    @staticmethod
    def _match(amdsmi, handles):
        import torch

        if not handles:
            raise RuntimeError("amdsmi lists no GPU")
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        if bus is not None and len(handles) > 1:
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                if int(bdf.split(":")[1], 16) == int(bus):
                    return h
        return handles[0]

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                self.samples.setdefault(self.phase, []).append(v)
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            time.sleep(self.period)

    def start(self, phase):
        import threading

        self.phase = phase
        if self._read is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def mark(self, phase):
        self.phase = phase

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        out = {"source": "amdsmi gpu metrics: mean of the per-XCD current graphics clocks, sampled every "
                         f"{self.period * 1e3:.0f} ms on a host thread; the firmware refreshes the table "
                         "with a lag of up to about a second, so a phase's readings trail its load"}
        for ph, v in self.samples.items():
            out[ph] = {"min_mhz": min(v), "mean_mhz": round(sum(v) / len(v), 1), "max_mhz": max(v), "samples": len(v)}
        if self.error:
            out["error"] = self.error
        return out


def versions():
    import torch

    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"torch": torch.__version__, "hip": torch.version.hip, "rocm": rocm, "python": sys.version.split()[0]}


def host_cores():
    return len(os.sched_getaffinity(0))


def blas_threads():
    import threadpoolctl

    return max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1) or 1


def output_check(O, L, Oref, Lref, tol_o=1e-2, tol_l=1e-3):
    """Errors of the timed launch's outputs against the fp64 oracle (every compared
    element): max-abs O and L, the bf16 output floor max|bf16(O_ref) - O_ref|, and the
    number of O elements above the bar (allowed only where half a bf16 ulp of the exact
    value exceeds the bar and the output is one of the two bf16 values around it)."""
    import numpy as np
    import torch

    O = np.asarray(O, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    err = np.abs(O - Oref)
    fin = np.isfinite(Lref)
    rne = torch.from_numpy(np.ascontiguousarray(Oref)).to(torch.bfloat16).double().numpy()
    over = err > tol_o
    _, ex = np.frexp(Oref[over])
    sp = np.ldexp(1.0, ex - 8)
    lo = np.floor(Oref[over] / sp) * sp
    faithful = (sp / 2 > tol_o) & ((O[over] == lo) | (O[over] == lo + sp))
    el = float(np.abs(L[fin] - Lref[fin]).max()) if fin.any() else 0.0
    return {"max_abs_O": float(err.max()), "max_abs_L": el, "bf16_floor": float(np.abs(rne - Oref).max()),
            "tol_O": tol_o, "tol_L": tol_l, "elements": int(O.size), "above_tol_O": int(over.sum()),
            "above_tol_O_faithful_bf16": int(faithful.sum()),
            "pass": bool(np.all(np.isfinite(O)) and faithful.all() and el <= tol_l)}


def _code_only(text):
    """Source text without comments and with whitespace runs collapsed, so that a digest
    changes with the code and not with its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_io_aware_15_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ["fa_device.h", "fa_launch.h", "fa_prefill_bf16.hip"],
    "decode": ["fa_device.h", "fa_launch.h", "fa_decode.hip"],
    "backward": ["fa_device.h", "fa_launch.h", "fa_backward.hip"],
    "window": ["fa_device.h", "fa_launch.h", "fa_prefill_bf16.hip"],
    "chunked": ["fa_device.h", "fa_launch.h", "fa_prefill_bf16.hip"],
    "int8": ["fa_device.h", "fa_launch.h", "fa_decode.hip"],
}


def measured_traffic(kind):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel sources changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_digest") != source_digest(KERNEL_SOURCES[kind]):
        return None
    return t.get("bytes_per_launch")


def prefill_flops(cfg):
    f = 4.0 * cfg.B * cfg.Hq * cfg.N * cfg.N * cfg.d
    return f / 2 if cfg.causal else f


def decode_bytes(x, cfg):
    ctx = x["ctx_lens"].long()
    kv = int(ctx.sum()) * cfg.Hkv * cfg.d * 2 * 2
    qo = 2 * cfg.num_seqs * cfg.Hq * cfg.d * 2
    lse = cfg.num_seqs * cfg.Hq * 4
    pages_used = int(((ctx + cfg.page_size - 1) // cfg.page_size).sum())
    return kv + qo + lse + pages_used * 4 + cfg.num_seqs * 4


def cpu_baseline_prefill(x, cfg, stride):
    """fp64 oracle on every `stride`-th query row of every head (stride 1: the whole
    workload).  Returns the baseline record, the rows and the oracle's O and L."""
    import numpy as np

    from oracle import attention_ref

    q, k, v = (x[n].float().numpy() for n in "qkv")
    rows = np.arange(0, cfg.N, stride)
    t0 = time.perf_counter()
    Oref, Lref = attention_ref(q, k, v, cfg.causal, cfg.scale, rows=rows)
    dt = time.perf_counter() - t0
    vis = (rows + 1) if cfg.causal else np.full(rows.shape, cfg.N)
    flops = 4.0 * cfg.d * float(vis.sum()) * cfg.B * cfg.Hq
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "threads": blas_threads(),
           "kind": "oracle",
           "sample": (f"all {cfg.N} query rows" if stride == 1 else f"every {stride}th query row ({len(rows)} rows)")
                     + f" of all {cfg.B * cfg.Hq} heads of {cfg.name}; {dt:.1f} s of fp64 numpy",
           "seconds": round(dt, 2)}
    return rec, rows, Oref, Lref


def cpu_baseline_backward(x, do, cfg, heads):
    """fp64 oracle gradients for the first `heads` query heads (and their K/V heads) of batch 0."""
    from oracle import attention_bwd_ref

    G = cfg.Hq // cfg.Hkv
    nkv = -(-heads // G)
    q = x["q"][:1, :heads].float().numpy()
    k = x["k"][:1, :nkv].float().numpy()
    v = x["v"][:1, :nkv].float().numpy()
    g = do[:1, :heads].float().numpy()
    t0 = time.perf_counter()
    attention_bwd_ref(q, k, v, g, cfg.causal, cfg.scale)
    dt = time.perf_counter() - t0
    flops = 2.5 * 4.0 * heads * cfg.N * cfg.N * cfg.d / (2 if cfg.causal else 1)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "threads": blas_threads(),
            "kind": "oracle",
            "sample": f"{heads} of {cfg.B * cfg.Hq} query heads of {cfg.name} (every row and key); "
                      f"{dt:.1f} s of fp64 numpy",
            "seconds": round(dt, 2)}


def cpu_baseline_decode(x, cfg, nseq):
    """fp64 oracle on the first nseq sequences.  Returns the baseline record and the
    oracle's O and L for those sequences."""
    from oracle import decode_ref

    kp = x["kpages"].float().numpy()  # bf16 -> fp32 view for numpy, outside the timed region
    vp = x["vpages"].float().numpy()
    sub = slice(0, nseq)
    qs = x["q"][sub].float().numpy()
    t0 = time.perf_counter()
    Oref, Lref = decode_ref(qs, kp, vp, x["page_table"][sub].numpy(), x["ctx_lens"][sub].numpy(), cfg.scale)
    dt = time.perf_counter() - t0
    ctx = x["ctx_lens"][sub].long()
    byts = int(ctx.sum()) * cfg.Hkv * cfg.d * 4 + 2 * nseq * cfg.Hq * cfg.d * 2
    rec = {"value": byts / dt / 1e9, "unit": "GB/s", "cores": host_cores(), "threads": blas_threads(),
           "kind": "oracle",
           "sample": f"{nseq} of {cfg.num_seqs} sequences of {cfg.name} (all heads, every valid token); "
                     f"{dt:.1f} s of fp64 numpy incl. the page gather",
           "seconds": round(dt, 2)}
    return rec, Oref, Lref


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (the GPU clock takes tens of milliseconds of load to settle; "
                         "200 steps are about 0.2 s)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="warm-up floor in milliseconds of load before the timed steps (the clock settles "
                         "within tens of milliseconds)")
    ap.add_argument("--step-settle-ms", type=float, default=1500.0,
                    help="warm-up floor in milliseconds of load before the timed steps themselves (long "
                         "enough for the sampled clock readings, which trail the load, to show it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-row-stride", type=int, default=1,
                    help="oracle baseline on every n-th query row of the prefill (1 = the whole workload)")
    ap.add_argument("--cpu-bwd-heads", type=int, default=1,
                    help="oracle backward baseline on the first n query heads of batch 0")
    ap.add_argument("--cpu-decode-seqs", type=int, default=64,
                    help="oracle baseline on the first n sequences of the decode (64 = the whole workload)")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "window", "chunked", "int8", "configs",
                                       "shard"],
                    default=None,
                    help="time one part only (for profiling runs)")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip the INT8-cache decode measurement (reported beside the step)")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked paged-prefill measurement (reported beside the step)")
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window + ALiBi measurement (reported beside the step)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the forward on the other prefill configurations (reported beside the step)")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip timing one GPU's share of the step split over 8 GPUs by heads")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward measurement (reported beside the step, not part of it)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB 5 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch

        n = args.copy_probe * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU "
              "path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_15_amd as fa
    from exact_io_aware_15_amd.workloads import CONFIGS, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pcfg, dcfg = CONFIGS[PREFILL], CONFIGS[DECODE]
    run_p = args.only in (None, "prefill")
    run_d = args.only in (None, "decode")
    run_b = args.only == "backward" or (args.only is None and not args.no_bwd)
    # the measurements beside the step
    run_w = args.only == "window" or (args.only is None and not args.no_window)
    run_c = args.only == "chunked" or (args.only is None and not args.no_chunked)
    run_i = args.only == "int8" or (args.only is None and not args.no_int8)
    run_o = args.only == "configs" or (args.only is None and not args.no_configs)
    run_s = args.only == "shard" or (args.only is None and not args.no_shard)

    log("generating inputs")
    px = make_inputs(pcfg) if run_p else None
    dx = make_inputs(dcfg) if run_d else None
    if run_p:
        q, k, v = (px[n].to(dev) for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if run_d:
        dq, kp, vp = dx["q"].to(dev), dx["kpages"].to(dev), dx["vpages"].to(dev)
        pt, cl = dx["page_table"].to(dev), dx["ctx_lens"].to(dev)
        do = torch.empty_like(dq)
        dl = torch.empty(dq.shape[:2], dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_paged_workspace_size(dcfg.num_seqs, dcfg.Hq, dcfg.d,
                                                           dx["max_pages_per_seq"]), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        fa.fa_fwd(q, k, v, causal=pcfg.causal, scale=pcfg.scale, out=o, lse=lse)

    def decode():
        fa.fa_decode_paged(dq, kp, vp, pt, cl, scale=dcfg.scale, out=do, lse=dl, workspace=ws)

    def step():
        if run_p:
            prefill()
        if run_d:
            decode()

    # The step gets the same time-floored warm-up as every measurement beside it: at
    # least --warmup steps and at least --settle-ms of load, so the clock has settled.
    clocks = ClockSampler()
    clocks.start("warmup")
    n_warm, warm_ms = warm(step, args.warmup, ms_min=max(args.settle_ms, args.step_settle_ms))
    log(f"warmup {n_warm} steps in {warm_ms:.0f} ms")

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    log(f"timing {K} steps")
    clocks.mark("timed")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        if run_p:
            prefill()
        ev[i][1].record()
        if run_d:
            decode()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clocks.mark("side_measurements")  # sampled on through the measurements beside the step
    p_list = [e[0].elapsed_time(e[1]) for e in ev]
    d_list = [e[1].elapsed_time(e[2]) for e in ev]
    p_ms = sum(p_list) / K
    d_ms = sum(d_list) / K
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / K
    log(f"prefill {p_ms:.4f} ms, decode {d_ms:.4f} ms, step {step_ms:.4f} ms (wall {wall * 1e3 / K:.4f} ms)")

    def stats(v):
        import statistics

        return {"mean_ms": round(sum(v) / len(v), 5), "median_ms": round(statistics.median(v), 5),
                "min_ms": round(min(v), 5), "max_ms": round(max(v), 5)}

    bwd = None
    if run_b or run_w:
        bx = px if px is not None else make_inputs(pcfg)
        bq, bk, bv = (bx[n].to(dev) for n in "qkv")
    if run_b:
        # the backward (not part of the step): gradients of the same causal prefill for a
        # seeded upstream gradient, with O and L from the forward computed beforehand
        from exact_io_aware_15_amd.workloads import make_grad_output
        bdo_cpu = make_grad_output(pcfg.B, pcfg.Hq, pcfg.N, pcfg.d, seed=pcfg.seed)
        bdo = bdo_cpu.to(dev)
        bo, bl = fa.fa_fwd(bq, bk, bv, causal=pcfg.causal, scale=pcfg.scale)
        bws = torch.empty(max(16, fa.fa_bwd_workspace_size(pcfg.B, pcfg.Hq, pcfg.Hkv, pcfg.N, pcfg.d)),
                          dtype=torch.uint8, device=dev)
        bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)

        def backward():
            fa.fa_bwd(bq, bk, bv, bo, bl, bdo, causal=pcfg.causal, scale=pcfg.scale, dq=bdq, dk=bdk, dv=bdv,
                      workspace=bws)

        warm(backward, max(1, args.warmup // 3), ms_min=args.settle_ms)
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            bev[i][0].record()
            backward()
            bev[i][1].record()
        torch.cuda.synchronize()
        b_ms = sum(e[0].elapsed_time(e[1]) for e in bev) / K
        bfl = 2.5 * prefill_flops(pcfg)
        btf = bfl / (b_ms * 1e-3) / 1e12
        log(f"backward {b_ms:.4f} ms ({btf:.1f} TFLOP/s)")
        bwd = {"value": round(btf, 2), "unit": "TFLOP/s", "ms": round(b_ms, 5),
               "roofline": {"bound": "mfma", "achieved": round(btf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(btf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("backward"),
                            "kernel": "bwd_delta + bwd_dq + bwd_dkdv <128, causal>",
                            "algorithmic_flops_per_launch": bfl},
               "workload": "gradients of the causal bf16 prefill B1 Hq32 N8192 d128 (dO ~ N(0,1)); FLOPs 2.5x the "
                           "forward's (five N x N x d products), causal half"}

    wa = None
    if run_w:
        # sliding window (W = 4096) + ALiBi on the same causal prefill (not part of the step);
        # FLOPs count only the visible (query, key) pairs: sum_i min(i + 1, W)
        from exact_io_aware_15_amd.workloads import make_alibi_slopes
        W = 4096
        slopes = make_alibi_slopes(pcfg.Hq).to(dev)
        wo, wl = torch.empty_like(bq), torch.empty((pcfg.B, pcfg.Hq, pcfg.N), dtype=torch.float32, device=dev)

        def windowed():
            fa.fa_fwd_ex(bq, bk, bv, causal=True, scale=pcfg.scale, window=W, alibi_slopes=slopes, out=wo, lse=wl)

        warm(windowed, max(1, args.warmup // 3), ms_min=args.settle_ms)
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            wev[i][0].record()
            windowed()
            wev[i][1].record()
        torch.cuda.synchronize()
        w_ms = sum(e[0].elapsed_time(e[1]) for e in wev) / K
        n = pcfg.N
        pairs = W * (W + 1) // 2 + (n - W) * W
        wfl = 4.0 * pcfg.B * pcfg.Hq * pcfg.d * pairs
        wtf = wfl / (w_ms * 1e-3) / 1e12
        log(f"window+alibi {w_ms:.4f} ms ({wtf:.1f} TFLOP/s)")
        wa = {"value": round(wtf, 2), "unit": "TFLOP/s", "ms": round(w_ms, 5),
              "roofline": {"bound": "mfma", "achieved": round(wtf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(wtf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("window"),
                           "kernel": "fwd_bf16_kernel<128, causal, window/ALiBi>",
                           "algorithmic_flops_per_launch": wfl},
              "workload": f"causal bf16 prefill B1 Hq32 N8192 d128 with a {W}-key sliding window and ALiBi "
                          "slopes 2^(-8(h+1)/32); FLOPs over visible pairs only"}

    cp = None
    if run_c:
        # chunked prefill over a paged cache (not part of the step): 16 sequences, 512-token
        # chunks, contexts U[512, 16384], Hq32 Hkv8 d128; FLOPs over the visible pairs
        from exact_io_aware_15_amd.workloads import make_prefill_paged
        cx = make_prefill_paged(16, 32, 8, 128, 512, 512, 16384, seed=6)
        cg = {kk: (vv.to(dev) if torch.is_tensor(vv) else vv) for kk, vv in cx.items()}
        co = torch.empty_like(cg["q"])
        cl = torch.empty(cg["q"].shape[:3], dtype=torch.float32, device=dev)

        def chunked():
            fa.fa_prefill_paged(cg["q"], cg["kpages"], cg["vpages"], cg["page_table"], cg["ctx_lens"], out=co,
                                lse=cl)

        warm(chunked, max(1, args.warmup // 3), ms_min=args.settle_ms)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            cev[i][0].record()
            chunked()
            cev[i][1].record()
        torch.cuda.synchronize()
        c_ms = sum(e[0].elapsed_time(e[1]) for e in cev) / K
        ctxs = cx["ctx_lens"].long()
        pairs = int((512 * (ctxs - 512) + 512 * 513 // 2).sum())
        cfl = 4.0 * 32 * 128 * pairs
        ctf = cfl / (c_ms * 1e-3) / 1e12
        log(f"chunked prefill {c_ms:.4f} ms ({ctf:.1f} TFLOP/s)")
        cp = {"value": round(ctf, 2), "unit": "TFLOP/s", "ms": round(c_ms, 5),
              "roofline": {"bound": "mfma", "achieved": round(ctf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(ctf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("chunked"),
                           "kernel": "fwd_bf16_kernel<128, causal, paged>", "algorithmic_flops_per_launch": cfl},
              "workload": "chunked prefill over 16-token pages: 16 sequences x 512-token chunks, contexts "
                          f"U[512,16384] (total {int(ctxs.sum())}), Hq32 Hkv8 d128; FLOPs over visible pairs"}

    d8 = None
    if run_i:
        # INT8 group-scaled paged decode on the decode workload's shapes and seed (not part
        # of the step); algorithmic bytes: int8 K/V and their fp32 scales of every valid
        # token, plus q, O, L, the used page-table entries and ctx_lens
        from exact_io_aware_15_amd.workloads import make_decode_int8
        ix = make_decode_int8(dcfg.num_seqs, dcfg.Hq, dcfg.Hkv, dcfg.d, dcfg.ctx_lo, dcfg.ctx_hi, dcfg.seed)
        ig = {kk: (vv.to(dev) if torch.is_tensor(vv) else vv) for kk, vv in ix.items()}
        io = torch.empty_like(ig["q"])
        il = torch.empty(ig["q"].shape[:2], dtype=torch.float32, device=dev)
        iws = torch.empty(fa.fa_decode_paged_workspace_size(dcfg.num_seqs, dcfg.Hq, dcfg.d, ix["max_pages_per_seq"]),
                          dtype=torch.uint8, device=dev)

        def int8_decode():
            fa.fa_decode_paged_int8(ig["q"], ig["kq"], ig["kscale"], ig["vq"], ig["vscale"], ig["page_table"],
                                    ig["ctx_lens"], out=io, lse=il, workspace=iws)

        warm(int8_decode, max(1, args.warmup // 3), ms_min=args.settle_ms)
        iev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            iev[i][0].record()
            int8_decode()
            iev[i][1].record()
        torch.cuda.synchronize()
        i_ms = sum(e[0].elapsed_time(e[1]) for e in iev) / K
        ctx = ix["ctx_lens"].long()
        per_tok = dcfg.Hkv * (2 * dcfg.d + 2 * (dcfg.d // 32) * 4)
        iby = int(ctx.sum()) * per_tok + 2 * dcfg.num_seqs * dcfg.Hq * dcfg.d * 2 + dcfg.num_seqs * dcfg.Hq * 4 + \
            int(((ctx + 15) // 16).sum()) * 4 + dcfg.num_seqs * 4
        igbs = iby / (i_ms * 1e-3) / 1e9
        log(f"int8 decode {i_ms:.4f} ms ({igbs:.1f} GB/s)")
        d8 = {"value": round(igbs, 1), "unit": "GB/s", "ms": round(i_ms, 5),
              "roofline": {"bound": "hbm", "achieved": round(igbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(igbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("int8"),
                           "kernel": "decode_split_int8_kernel<128, 4> + decode_merge_kernel<128>",
                           "algorithmic_bytes_per_launch": iby},
              "workload": "paged decode 64 seqs Hq32 Hkv8 d128 ctx~U[1024,16384] over an INT8 cache with fp32 "
                          "scales per 32 channels (288 B per token and K/V head instead of 512)"}

    oc = None
    if run_o:
        # the forward on the other prefill configurations (not part of the step): fp32 N256 d64,
        # bf16 non-causal d64, causal GQA and MQA at d128; same inputs as their parity tests
        oc = {}
        for name in OTHER_PREFILL:
            ocfg = CONFIGS[name]
            ox = make_inputs(ocfg)
            oq, ok_, ov = (ox[n].to(dev) for n in "qkv")
            oo = torch.empty_like(oq)
            ol = torch.empty(oq.shape[:3], dtype=torch.float32, device=dev)
            fwd = fa.fa_fwd_f32 if ocfg.dtype == "f32" else fa.fa_fwd

            def other():
                fwd(oq, ok_, ov, causal=ocfg.causal, scale=ocfg.scale, out=oo, lse=ol)

            warm(other, max(1, args.warmup // 3), ms_min=args.settle_ms)
            oev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
            for i in range(K):
                oev[i][0].record()
                other()
                oev[i][1].record()
            torch.cuda.synchronize()
            o_ms = sum(e[0].elapsed_time(e[1]) for e in oev) / K
            ofl = prefill_flops(ocfg)
            otf = ofl / (o_ms * 1e-3) / 1e12
            peak = PEAK_F32_TFLOPS if ocfg.dtype == "f32" else PEAK_BF16_TFLOPS
            log(f"{name} {o_ms * 1e3:.1f} us ({otf:.1f} TFLOP/s)")
            oc[name] = {"ms": round(o_ms, 5), "TFLOP/s": round(otf, 2), "peak": peak,
                        "frac": round(otf / peak, 4), "algorithmic_flops_per_launch": ofl,
                        "kernel": ("fwd_f32_kernel" if ocfg.dtype == "f32" else "fwd_bf16_persistent_kernel")
                        + f"<{ocfg.d}, {'causal' if ocfg.causal else 'non-causal'}>"}
            del oq, ok_, ov, oo, ol

    sh = None
    if run_s:
        # one GPU's share of the step when it is split over 8 GPUs by heads (the shares are
        # independent, so no collective is involved): the forward with 4 of its 32 heads, the
        # decode with 1 of its 8 K/V heads and its 4 query heads, same seeds and distributions
        import dataclasses

        from exact_io_aware_15_amd.workloads import make_decode

        scfg = dataclasses.replace(pcfg, name="c3 share (4 of 32 heads)", Hq=pcfg.Hq // 8, Hkv=pcfg.Hkv // 8)
        sdcfg = dataclasses.replace(dcfg, name="c5 share (1 of 8 K/V heads)", Hq=dcfg.Hq // 8, Hkv=dcfg.Hkv // 8)
        sx = make_inputs(scfg)
        sq, sk, sv = (sx[n].to(dev) for n in "qkv")
        so, sl = torch.empty_like(sq), torch.empty(sq.shape[:3], dtype=torch.float32, device=dev)
        sdx = make_decode(sdcfg.num_seqs, sdcfg.Hq, sdcfg.Hkv, sdcfg.d, sdcfg.ctx_lo, sdcfg.ctx_hi, sdcfg.seed,
                          sdcfg.page_size, sdcfg.max_pages_per_seq, sdcfg.fixed_ctx)
        sdq, skp, svp = sdx["q"].to(dev), sdx["kpages"].to(dev), sdx["vpages"].to(dev)
        spt, scl = sdx["page_table"].to(dev), sdx["ctx_lens"].to(dev)
        sdo, sdl = torch.empty_like(sdq), torch.empty(sdq.shape[:2], dtype=torch.float32, device=dev)
        sws = torch.empty(fa.fa_decode_paged_workspace_size(sdcfg.num_seqs, sdcfg.Hq, sdcfg.d,
                                                            sdx["max_pages_per_seq"]), dtype=torch.uint8, device=dev)

        sws_p = torch.empty(max(1, fa.fa_fwd_splitk_workspace_size(scfg.B, scfg.Hq, scfg.N, scfg.d, scfg.causal)),
                            dtype=torch.uint8, device=dev)

        def share_prefill():
            fa.fa_fwd(sq, sk, sv, causal=scfg.causal, scale=scfg.scale, out=so, lse=sl)

        def share_prefill_splitk():
            fa.fa_fwd_splitk(sq, sk, sv, causal=scfg.causal, scale=scfg.scale, out=so, lse=sl, workspace=sws_p)

        def share_decode():
            fa.fa_decode_paged(sdq, skp, svp, spt, scl, scale=sdcfg.scale, out=sdo, lse=sdl, workspace=sws)

        def timed(fn):
            warm(fn, max(1, args.warmup // 3), ms_min=args.settle_ms)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
            for i in range(K):
                ev[i][0].record()
                fn()
                ev[i][1].record()
            torch.cuda.synchronize()
            return sum(e[0].elapsed_time(e[1]) for e in ev) / K

        sp_ms, sk_ms, sd_ms = timed(share_prefill), timed(share_prefill_splitk), timed(share_decode)
        sfl = prefill_flops(scfg)
        sby = decode_bytes(sdx, sdcfg)
        stf, skf, sgb = sfl / (sp_ms * 1e-3) / 1e12, sfl / (sk_ms * 1e-3) / 1e12, sby / (sd_ms * 1e-3) / 1e9
        log(f"share: prefill {sp_ms * 1e3:.1f} us ({stf:.1f} TFLOP/s), split-K {sk_ms * 1e3:.1f} us "
            f"({skf:.1f} TFLOP/s), decode {sd_ms * 1e3:.1f} us ({sgb:.1f} GB/s)")
        sh = {"note": "one GPU's share of the step split over 8 GPUs by heads; no collective needed",
              "prefill": {"workload": f"causal bf16 B{scfg.B} Hq{scfg.Hq} Hkv{scfg.Hkv} N{scfg.N} d{scfg.d}",
                          "fa_fwd": {"ms": round(sp_ms, 5), "TFLOP/s": round(stf, 2),
                                     "frac": round(stf / PEAK_BF16_TFLOPS, 4)},
                          "fa_fwd_splitk": {"ms": round(sk_ms, 5), "TFLOP/s": round(skf, 2),
                                            "frac": round(skf / PEAK_BF16_TFLOPS, 4)},
                          "implied_8gpu_TFLOP/s": round(8 * max(stf, skf), 1)},
              "decode": {"workload": f"paged decode {sdcfg.num_seqs} seqs Hq{sdcfg.Hq} Hkv{sdcfg.Hkv} d{sdcfg.d}",
                         "ms": round(sd_ms, 5), "GB/s": round(sgb, 1), "frac": round(sgb / PEAK_HBM_GBS, 4),
                         "implied_8gpu_GB/s": round(8 * sgb, 1)}}
        del sq, sk, sv, so, sl, sdq, skp, svp, spt, scl, sdo, sdl, sws, sws_p

    clock_rec = clocks.stop()
    res = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) inputs; random page permutation)",
           "timing": {"warmup_steps": n_warm, "warmup_ms": round(warm_ms, 1),
                      "settle_floor_ms": args.settle_ms,
                      "step_settle_floor_ms": max(args.settle_ms, args.step_settle_ms),
                      "events": "HIP events on the launch stream"},
           "sclk": clock_rec, "versions": versions()}
    if run_p:
        res["timing"]["prefill"] = stats(p_list)
    if run_d:
        res["timing"]["decode"] = stats(d_list)
    cfg_desc = {"workload": "one step = causal bf16 prefill B1 Hq32 Hkv32 N8192 d128 (inputs 0.5*N(0,1)) "
                            "+ paged bf16 decode 64 seqs Hq32 Hkv8 d128 ctx~U[1024,16384] 16-token pages"}
    if run_p:
        fl = prefill_flops(pcfg)
        tf = fl / (p_ms * 1e-3) / 1e12
        tr = measured_traffic("prefill")
        res.update({"value": round(tf, 2), "unit": "TFLOP/s"})
        res["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": tr,
                           "kernel": "fwd_bf16_persistent_kernel<128, causal>", "ms": round(p_ms, 5),
                           "algorithmic_flops_per_launch": fl}
        cfg_desc["prefill"] = {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "N": pcfg.N, "d": pcfg.d,
                               "causal": pcfg.causal, "seed": pcfg.seed}
    if run_d:
        by = decode_bytes(dx, dcfg)
        gbs = by / (d_ms * 1e-3) / 1e9
        dec = {"value": round(gbs, 1), "unit": "GB/s", "ms": round(d_ms, 5),
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode"),
                            "kernel": "decode_split_kernel<128, 4> + decode_merge_kernel<128>",
                            "algorithmic_bytes_per_launch": by}}
        res["decode"] = dec
        cfg_desc["decode"] = {"num_seqs": dcfg.num_seqs, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d,
                              "page_size": dcfg.page_size, "ctx_total": int(dx["ctx_lens"].long().sum()),
                              "seed": dcfg.seed}
        if not run_p:
            res.update({"value": dec["value"], "unit": "GB/s", "roofline": dec["roofline"]})
    if wa is not None:
        res["window_alibi"] = wa
    if cp is not None:
        res["chunked_prefill"] = cp
    if d8 is not None:
        res["decode_int8"] = d8
    if bwd is not None:
        res["backward"] = bwd
    if oc is not None:
        res["other_configs"] = oc
    if sh is not None:
        res["shard_share"] = sh
    if "value" not in res:  # one of the measurements beside the step was run alone
        one = next((x for x in (bwd, wa, cp, d8) if x is not None), None)
        if one is not None:
            res.update({"value": one["value"], "unit": one["unit"], "roofline": one["roofline"]})
        else:
            res.update({"value": None, "unit": "TFLOP/s", "roofline": None})
    res["config"] = cfg_desc
    if not args.no_cpu_baseline:
        # the oracle's results also check the outputs of the last timed step
        log("timing the fp64 CPU oracle on a bounded sample")
        numerics = {}
        if run_p:
            cb, rows, Oref, Lref = cpu_baseline_prefill(px, pcfg, args.cpu_row_stride)
            res["cpu_baseline"] = cb
            ri = torch.from_numpy(rows).to(dev)
            numerics[PREFILL] = output_check(o[:, :, ri].double().cpu().numpy(), lse[:, :, ri].double().cpu().numpy(),
                                             Oref, Lref)
            numerics[PREFILL]["rows"] = "all" if args.cpu_row_stride == 1 else f"every {args.cpu_row_stride}th"
            del Oref, Lref
        if run_d:
            nseq = min(args.cpu_decode_seqs, dcfg.num_seqs)
            cb, Oref, Lref = cpu_baseline_decode(dx, dcfg, nseq)
            numerics[DECODE] = output_check(do[:nseq].double().cpu().numpy(), dl[:nseq].double().cpu().numpy(),
                                            Oref, Lref)
            numerics[DECODE]["sequences"] = nseq
            if run_p:
                res["decode"]["cpu_baseline"] = cb
            else:
                res["cpu_baseline"] = cb
        res["numerics"] = numerics
        log("numerics: " + ", ".join(f"{k} max|dO| {v['max_abs_O']:.2e} max|dL| {v['max_abs_L']:.2e} "
                                     f"floor {v['bf16_floor']:.2e} pass {v['pass']}" for k, v in numerics.items()))
        if bwd is not None:
            bcb = cpu_baseline_backward(bx, bdo_cpu, pcfg, args.cpu_bwd_heads)
            if "cpu_baseline" in res:
                res["backward"]["cpu_baseline"] = bcb
            else:
                res["cpu_baseline"] = bcb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
