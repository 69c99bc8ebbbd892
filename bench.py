"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one fa2_fwd (or fa2_fwd_ext, for the causal / grouped-head / unequal
length workloads; fa2_fwd_kv_int8 / fa2_fwd_kv_fp8 for the INT8 / FP8 cache
workloads) launch over the
whole workload (every (b, h) and query row of one batch), inputs resident in
HBM.  FLOPs count the two products over the
(query, key) pairs that enter the softmax: 4*B*H*N^2*d without a mask.  W untimed steps, then exactly K
steps timed with HIP events on the launch stream, bracketed by device
synchronisation.  The default warm-up is long (200 launches, about 0.1 s of
the headline) because per-launch times settle only after roughly the first
hundred launches of a process (the earliest run up to a third slower while
the clock settles); the timed steps then measure the steady rate a long job
sees.  Prints ONE JSON line: forward attention TFLOP/s counting
4*B*H*N^2*d FLOPs, the roofline of the kernel against the dense bf16/fp16 MFMA
peak, and the fp64 CPU oracle's rate on a bounded sample of the same workload
on this host's cores.

With the headline workload (the default) the same run then times the
sequence sweep (N = 512 ... 16384 at B*N = 16384, fp16), the head-dimension
variants (d = 64, 256) and four decoding workloads with key splits (one query
row per head against 32K and 128K keys, and 32K over INT8 and FP8 caches) with the same --warmup / --steps, and
adds them to the line as "sweep" (per N, plus the harmonic mean), "head_dim"
and "decode", each with its roofline fraction (--no-extras leaves them out).  Every output is checked
after the timing (NaN-prefilled buffers fully written with finite values, and
the oracle's parity on the heads the CPU baseline computed): the line is
printed either way, and the exit status is 1 if a check failed.

Other modes: --workload NAME for any of the parity workloads (one line each),
--no-cpu-baseline to skip the oracle timing, --calibrate-copy to run only a
plain device copy of known size (for scaling HBM byte counters), and
--traffic-from to turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs into the traffic
record under profiles/ that the roofline's "traffic" field reads.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s, bf16 d=128 N=4096 non-causal; % of MFMA peak"
# MI355X dense (no sparsity) MFMA peak for bf16/fp16: 256 CUs x 2.4 GHz x
# 4096 FLOP/CU/clk = 2516.6 TFLOP/s, the published 2.5 PFLOP/s figure; int8
# and fp8 run at twice that (the published 5.0 POP/s and 5.0 PFLOP/s).
MFMA_PEAK_TFLOPS = 2516.6
INT8_PEAK_TOPS = 2 * MFMA_PEAK_TFLOPS
FP8_PEAK_TFLOPS = 2 * MFMA_PEAK_TFLOPS
HBM_PEAK_GBS = 8000.0
# Workloads timed after the headline in the default run, each with the same
# --steps / --warmup: the sequence sweep of "Flash Attention 2 from scratch
# on Ampere", Part 1, Performance section (reported per N and as a harmonic
# mean), and the head-dimension variants.
SWEEP = ["sweep_n512", "sweep_n1024", "sweep_n2048", "sweep_n4096", "sweep_n8192",
         "sweep_n16384"]
HEAD_DIMS = ["d64", "d256"]
# ... and decoding against long caches with key splits (fa2_fwd_split).
DECODE = ["decode", "decode_long", "decode_int8", "decode_fp8"]
KERNEL_SRC = os.path.join(ROOT, "flashattention_forward_tile_amd", "csrc", "fa2_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa2_fwd_headline_traffic.json")
CPU_SAMPLE_SECONDS = 12.0


def code_digest(text: str) -> str:
    """sha256 of C++ source with comments, blank lines and trailing space
    removed, so a comment-only edit keeps the digest of the same code."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def kernel_digest() -> str:
    with open(KERNEL_SRC) as f:
        return code_digest(f.read())


def measured_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counts, if they were taken on this workload with this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_digest() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def _mean_counter(csv_path, counter, kernel_substr):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise ValueError("no %s rows for %s in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals)


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload,
                  copy_bytes=1 << 30):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for the copy kernel
    of --calibrate-copy, which moves exactly copy_bytes each way."""
    fetch_kib = _mean_counter(fetch_csv, "FETCH_SIZE", "fa2_fwd")
    write_kib = _mean_counter(write_csv, "WRITE_SIZE", "fa2_fwd")
    copy_fetch_kib = _mean_counter(copy_fetch_csv, "FETCH_SIZE", "elementwise")
    copy_write_kib = _mean_counter(copy_write_csv, "WRITE_SIZE", "elementwise")
    f_scale = copy_bytes / (copy_fetch_kib * 1024.0)
    w_scale = copy_bytes / (copy_write_kib * 1024.0)
    rd = fetch_kib * 1024.0 * f_scale
    wr = write_kib * 1024.0 * w_scale
    out = {"workload": workload, "kernel_sha256": kernel_digest(),
           "fetch_kib_per_launch": fetch_kib, "write_kib_per_launch": write_kib,
           "copy_fetch_kib": copy_fetch_kib, "copy_write_kib": copy_write_kib,
           "copy_bytes_each_way": copy_bytes, "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "hbm_read_bytes_per_launch": round(rd),
           "hbm_write_bytes_per_launch": round(wr), "hbm_bytes_per_launch": round(rd + wr)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def matrix_peak(w):
    """Matrix-core roof for workload w in TFLOP/s.  16-bit workloads: the
    bf16/fp16 peak.  The INT8 cache runs its first product (half the FLOPs)
    on int8 matrix instructions and its second on fp16 ones, so its roof is
    the rate at which both halves finish at their own peaks:
    1 / (0.5 / int8 peak + 0.5 / fp16 peak).  The FP8 cache likewise, with the
    fp8 matrix peak in place of the int8 one."""
    if w.kv_int8:
        return round(1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / MFMA_PEAK_TFLOPS), 1)
    if w.kv_fp8:
        return round(1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / MFMA_PEAK_TFLOPS), 1)
    return MFMA_PEAK_TFLOPS


def roofline_of(w, ms, traffic):
    """The roofline object for workload w at ms per launch.  The bound is the
    roof the workload's arithmetic intensity (FLOPs per algorithmic HBM byte)
    sits under: left of the ridge (peak FLOP/s over peak bytes/s) the HBM
    roof, in GB/s; otherwise the matrix-core roof, in TFLOP/s."""
    peak = matrix_peak(w)
    if w.flops / w.algo_bytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        gbs = w.algo_bytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    tflops = w.flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
            "traffic": traffic}


def cpu_baseline(w, q, k, v, o_gpu=None, lse_gpu=None):
    """The fp64 oracle as it stands, on whole heads of the same inputs, until
    about CPU_SAMPLE_SECONDS of wall time have passed (at least one head).
    With the GPU's outputs (CPU tensors) it also returns the parity of the
    heads it computed: O max-abs and mean-abs error, lse relative and
    absolute error (rows that see no key compared for O = 0, lse = -inf)."""
    import numpy as np

    import oracle
    from flashattention_forward_tile_amd.workloads import bits

    threads = oracle.host_threads()
    group = w.H // w.kv_heads
    heads = 0
    c = np.ascontiguousarray
    if w.quantized:
        qb, kq, ksc, vq, vsc = bits(q), k[0].numpy(), k[1].numpy(), v[0].numpy(), v[1].numpy()
    else:
        qb, kb, vb = bits(q), bits(k), bits(v)
    refs = []
    t0 = time.perf_counter()
    while heads < w.B * w.H:
        b, h = divmod(heads, w.H)
        qs = (slice(b, b + 1), slice(h, h + 1))
        ks = (slice(b, b + 1), slice(h // group, h // group + 1))
        if w.quantized:
            attn = oracle.attention_kv_int8 if w.kv_int8 else oracle.attention_kv_fp8
            o_ref, lse_ref = attn(
                c(qb[qs]), c(kq[ks]), c(ksc[ks]), c(vq[ks]), c(vsc[ks]), w.dtype, w.scale,
                nthreads=threads, causal=w.causal)
        else:
            o_ref, lse_ref = oracle.attention(c(qb[qs]), c(kb[ks]), c(vb[ks]), w.dtype, w.scale,
                                              nthreads=threads, causal=w.causal)
        if o_gpu is not None:
            refs.append((b, h, o_ref, lse_ref))
        heads += 1
        if time.perf_counter() - t0 >= CPU_SAMPLE_SECONDS:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * heads * w.visible_pairs * w.d
    out = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": "%d of %d heads (all %d query rows each) of the %s workload, "
                     "fp64, %.1f s wall" % (heads, w.B * w.H, w.N, w.name, dt)}
    if not refs:
        return out, None
    o_all = o_gpu.double().numpy()
    lse_all = lse_gpu.double().numpy()
    o_max = o_sum = lse_rel = lse_abs = 0.0
    count = 0
    empty_ok = lse_ok = True
    # The FP8 matrix instruction truncates its products, which moves a logit
    # by up to about 1e-4: rows whose logsumexp lies near zero (the first
    # causal rows) also pass at an absolute error of 1e-3.
    lse_floor = 1e-3 if w.kv_fp8 else 0.0
    for b, h, o_ref, lse_ref in refs:
        og, lg = o_all[b, h], lse_all[b, h]
        o_ref, lse_ref = o_ref[0, 0], lse_ref[0, 0]
        seen = np.isfinite(lse_ref)
        empty_ok &= bool(np.all(og[~seen] == 0.0) and np.all(lg[~seen] == -np.inf))
        e = np.abs(og[seen] - o_ref[seen])
        if e.size:
            o_max = max(o_max, float(e.max()))
            o_sum += float(e.sum())
            count += e.size
            le = np.abs(lg[seen] - lse_ref[seen])
            lse_rel = max(lse_rel, float(np.max(le / np.maximum(np.abs(lse_ref[seen]), 1e-30))))
            lse_abs = max(lse_abs, float(le.max()))
            lse_ok &= bool(np.all((le <= 1e-3 * np.abs(lse_ref[seen])) | (le <= lse_floor)))
    parity = {"heads": len(refs), "o_max_abs": o_max,
              "o_mean_abs": o_sum / count if count else 0.0, "lse_max_rel": lse_rel,
              "lse_max_abs": lse_abs, "unseen_rows_ok": empty_ok,
              "within_tolerance": bool(empty_ok and o_max <= 2e-2 and
                                       (o_sum / count if count else 0.0) <= 2e-3 and lse_ok)}
    return out, parity


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A copy-shaped elementwise kernel (dst = -src, fp32) that reads and
    writes exactly nbytes each, to scale the HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": nbytes, "bytes_written": nbytes,
                      "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline only (not the sweep and head-dim workloads)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                         "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the HBM traffic record from rocprofv3 counter CSVs")
    args = ap.parse_args()

    if args.traffic_from:
        write_traffic(*args.traffic_from, workload=args.workload)
        return

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the per-GPU share of "
              "independent (batch, head) work); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return

    from flashattention_forward_tile_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    extras = [] if args.no_extras or w.name != "headline" else SWEEP + HEAD_DIMS + DECODE
    # Every workload's inputs are drawn and made resident first, so that no
    # input generation sits between the timed runs.
    runs = [Resident(WORKLOADS[n]) for n in [w.name] + extras]
    main_run = runs[0]
    ms, wall = main_run.time(args.warmup, args.steps)
    tflops = w.flops / (ms * 1e-3) / 1e12
    roofline = roofline_of(w, ms, measured_traffic(w.name))
    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": dict(w.describe(), kernel="fa2_fwd_kernel", launches_per_step=1,
                       algo_hbm_bytes=w.algo_bytes,
                       algo_hbm_gbs=round(w.algo_bytes / (ms * 1e-3) / 1e9, 1),
                       wall_ms_per_step=round(wall * 1e3 / args.steps, 5)),
        "roofline": roofline,
    }
    # The other workloads right after, with the same warm-up and step count.
    others = {}
    for r in runs[1:]:
        r_ms, _ = r.time(args.warmup, args.steps)
        rl = roofline_of(r.w, r_ms, None)
        others[r.w.name] = {"ms_per_step": round(r_ms, 5),
                            "tflops": round(r.w.flops / (r_ms * 1e-3) / 1e12, 3),
                            "roofline": {k: rl[k] for k in ("bound", "achieved", "unit", "frac")}}
    ok = all(r.fully_written() for r in runs)
    if extras:
        sweep = {n: others[n] for n in SWEEP}
        hm = len(sweep) / sum(1.0 / x["tflops"] for x in sweep.values())
        out["sweep"] = dict(sweep, harmonic_mean_tflops=round(hm, 3),
                            config="B*N = 16384, H 16, d 128, fp16, N(0,1), non-causal")
        out["head_dim"] = {n: others[n] for n in HEAD_DIMS}
        out["decode"] = {n: others[n] for n in DECODE}
    if not args.no_cpu_baseline:
        q, k, v = main_run.host_qkv()
        o, lse = main_run.outputs()
        out["cpu_baseline"], out["parity"] = cpu_baseline(w, q, k, v, o, lse)
        ok &= out["parity"] is None or out["parity"]["within_tolerance"]
    out["outputs_ok"] = bool(ok)
    print(json.dumps(out), flush=True)
    if not ok:
        # a wrong result must not leave a clean benchmark record
        print("bench.py: output check failed (unwritten / non-finite values, or parity "
              "outside tolerance)", file=sys.stderr)
        sys.exit(1)


class Resident:
    """One workload's inputs and outputs resident on the GPU, and its launch."""

    def __init__(self, w):
        import torch

        from flashattention_forward_tile_amd import fa2
        from flashattention_forward_tile_amd.workloads import workload_inputs

        self.w = w
        dev = torch.device("cuda:0")
        self.inputs = workload_inputs(w, seed=0)
        self.dev_in = [t.to(dev) for t in self.inputs]
        self.o = torch.full_like(self.dev_in[0], float("nan"))
        self.lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=dev)
        if w.quantized and w.split:
            cache = fa2.CACHE_INT8 if w.kv_int8 else fa2.CACHE_FP8
            nbytes = fa2.split_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.keys, w.d, w.causal,
                                               self.dev_in[0].dtype, 0, cache)
            self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
            self.launch = lambda: fa2.fwd_kv_split(*self.dev_in, cache, scale=w.scale,
                                                   causal=w.causal, splits=0, workspace=self.ws,
                                                   out=self.o, lse=self.lse)
        elif w.quantized:
            fwd = fa2.fwd_kv_int8 if w.kv_int8 else fa2.fwd_kv_fp8
            self.launch = lambda: fwd(*self.dev_in, scale=w.scale, causal=w.causal,
                                      out=self.o, lse=self.lse)
        elif w.split:
            # the workspace is allocated once, outside the timed launches
            nbytes = fa2.split_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.keys, w.d, w.causal,
                                               self.dev_in[0].dtype, 0)
            self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
            self.launch = lambda: fa2.fwd_split(*self.dev_in, scale=w.scale, causal=w.causal,
                                                splits=0, workspace=self.ws, out=self.o,
                                                lse=self.lse)
        else:
            self.launch = lambda: fa2.fwd(*self.dev_in, scale=w.scale, causal=w.causal,
                                          out=self.o, lse=self.lse)

    def time(self, warmup, steps):
        """W untimed launches, then K timed with HIP events on the launch
        stream, bracketed by device synchronisation.  Returns (ms per launch,
        wall seconds of the timed region)."""
        import torch

        dev = self.o.device
        for _ in range(warmup):
            self.launch()
        # No other GPU work between the warm-up and the timed launches: an
        # idle gap restarts the slow first launches (outputs are checked after).
        stream = torch.cuda.current_stream(dev)  # fa2.fwd launches on this stream
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        wall0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            self.launch()
        stop.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - wall0
        return start.elapsed_time(stop) / max(steps, 1), wall

    def fully_written(self):
        """Every element of O and LSE finite (they start as NaN)."""
        import torch
        return bool(torch.isfinite(self.o.float()).all() and torch.isfinite(self.lse).all())

    def host_qkv(self):
        if self.w.quantized:
            i = self.inputs
            return i[0], (i[1], i[2]), (i[3], i[4])
        return self.inputs

    def outputs(self):
        return self.o.cpu(), self.lse.cpu()


if __name__ == "__main__":
    main()
