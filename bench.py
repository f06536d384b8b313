#!/usr/bin/env python3
"""Ring-fold attention throughput on one MI355X.

One step = one ra_ring_forward over the whole workload: all P virtual ring
steps (fold launches plus the double-buffered K/V hand-off) for every resident
query block, including the final normalisation.  Inputs are resident in HBM
before timing starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
                    [--causal contiguous|striped|zigzag] [--backward] [--graph]
                    [--no-cpu-baseline] [--cpu-seconds S]

The default workload is the 128K-token ring (B1 H32 d128 N131072 P16, all 16
query blocks resident), non-causal.  With --causal the same inputs are taken
as dealt to the devices in that token layout and the causal ring runs; its
TFLOP/s count only the visible (query, key) pairs, 4 d FLOP each.  With
--backward one step is one ra_ring_backward (dQ, dK, dV on the same ring; the
forward that gives O and the log-sum-exp runs once, untimed), counted as the
five products of the backward, 10 d FLOP per (query, key) pair.  With --graph
the step is captured once into a HIP graph (stream capture: fold launches and,
where the hand-off is copied, the copies, side stream and events all become nodes) and the timed steps
are graph replays; the fold-launch times in `roofline` then come from eager
steps.  --device-sweep instead times one device's ring step at its real shape
(one ra_fold_block of a b-row query block with one b-row visiting block, B1 H32
d128 bf16) for several b, next to the time one K/V block of that size takes
over one xGMI link, and prints one JSON line with a row per b.  `config.handoff`
says how the ring's K/V hand-off ran: with every block resident in ring order
(bf16, no mask) the folds write it themselves, and a full run (with the CPU
baseline) also times the same steps with the side-stream copies
(RA_HANDOFF_COPY=1) and reports them as `handoff_copy`.  `clock` is the shader clock the driver reported while the timed steps
ran (sampled from pp_dpm_sclk by a host thread) and the step throughput as a
share of the peak scaled to that clock (null where the file is not readable);
`clock.power` is the socket power sampled beside it (hwmon power1_input) with
the board's cap (power1_cap).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring-fold attention TFLOP/s and % MFMA bf16 peak, 128K tokens P=16, 1 GPU"
PEAK = {"bf16": 2500.0, "f32": 157.3}  # MI355X published dense TFLOP/s: bf16 MFMA, fp32 vector
FOLD_SOURCES = {"bf16": "fold_bf16.hip", "f32": "fold_f32.hip"}
BWD_SOURCES = {"bf16": "fold_bwd_bf16.hip", "f32": "fold_bwd_f32.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fold_traffic.json")


def _source_hash(dtype: str, backward: bool = False, d: int = 128) -> str:
    """Hash of the source file that holds the kernel of this dtype, head dim and pass."""
    if backward:
        name = BWD_SOURCES[dtype]
    else:
        name = FOLD_SOURCES.get(f"{dtype}/d{d}", FOLD_SOURCES[dtype])
    path = os.path.join(ROOT, "blockwise_online_softmax_fold_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic_key(workload: str, backward: bool) -> str:
    return workload + ("/backward" if backward else "")


def _traffic(workload: str, dtype: str, backward: bool = False, d: int = 128):
    """HBM bytes per launch (a fold launch, or one backward step's dQ + dK/dV
    launch pair) from the committed rocprofv3 counter summary, only if it was
    taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(_traffic_key(workload, backward))
    if not ent or ent.get("source_sha256_16") != _source_hash(dtype, backward, d):
        return None
    return ent.get("hbm_bytes_per_launch")


def traffic_from(fetch_dir: str, write_dir: str, workload: str, dtype: str, backward: bool, d: int = 128) -> int:
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-calibration` (one with
    FETCH_SIZE, one with WRITE_SIZE; KiB per dispatch) into HBM bytes per launch
    and record them in the traffic file under the current kernel source's hash.
    Each counter is scaled by what it read for a transfer of known size: the
    1 GiB device copy for FETCH_SIZE, the 1 GiB fill before it for WRITE_SIZE."""
    import glob
    import sqlite3

    def rows(d: str, counter: str):
        dbs = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
        if len(dbs) != 1:
            raise SystemExit(f"expected one *_results.db under {d}, found {len(dbs)}")
        with sqlite3.connect(dbs[0]) as db:
            return list(db.execute("select dispatch_id, kernel_name, value from counters_collection "
                                   "where counter_name = ? order by dispatch_id", (counter,)))

    f, w = rows(fetch_dir, "FETCH_SIZE"), rows(write_dir, "WRITE_SIZE")
    gib = float(1 << 30)
    plain_copy = lambda n: n.startswith("__amd_rocclr_copyBuffer") and "Rect" not in n  # noqa: E731
    # the calibration copy is the largest plain device copy of the run; the fill
    # that wrote its 1 GiB source is the last fill dispatched before it
    cal_f = max(v for _, name, v in f if plain_copy(name))
    copy_id = max(((v, i) for i, name, v in w if plain_copy(name)))[1]
    fills = [(i, v) for i, name, v in w if i < copy_id and "Fill" in name]
    if not fills:
        raise SystemExit("no fill dispatch before the calibration copy: run bench.py with --copy-calibration")
    cal_w = max(fills)[1]
    kf, kw = gib / (cal_f * 1024), gib / (cal_w * 1024)
    pick = (lambda n: "bwd_dq_kernel" in n or "bwd_dkdv_kernel" in n) if backward else (lambda n: "fold_" in n)
    fb = [v * 1024 * kf for _, name, v in f if pick(name)]
    wb = [v * 1024 * kw for _, name, v in w if pick(name)]
    per = 2 if backward else 1  # a backward "launch" is the dQ + dK/dV pair of one ring step
    if not fb or len(fb) != len(wb) or len(fb) % per:
        raise SystemExit(f"unexpected dispatch counts: {len(fb)} fetch, {len(wb)} write")
    n = len(fb) // per
    ent = {"read_scale": kf, "write_scale": kw, "launches": n,
           "read_bytes_per_launch": sum(fb) / n, "write_bytes_per_launch": sum(wb) / n}
    ent["hbm_bytes_per_launch"] = ent["read_bytes_per_launch"] + ent["write_bytes_per_launch"]
    ent["source_sha256_16"] = _source_hash(dtype, backward, d)
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec[_traffic_key(workload, backward)] = ent
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps({_traffic_key(workload, backward): ent}, indent=1))
    return 0


def _positions(layout: str, P: int, b: int):
    """Sequence position of row r of device j's block for a causal layout."""
    import numpy as np

    j = np.arange(P)[:, None]
    r = np.arange(b)[None, :]
    if layout == "contiguous":
        return j * b + r
    if layout == "striped":
        return r * P + j
    h = b // 2
    return np.where(r < h, j * h + r, (2 * P - 1 - j) * h + (r - h))


def _visible_pairs(w, layout: str) -> float:
    """(query, key) pairs a causal ring attends to: a row at position x sees
    the x + 1 positions 0..x, per batch and head."""
    pos = _positions(layout, w.P, w.b)
    return float(w.B) * w.H * float(sum(int(pos[i].sum()) + w.b for i in w.resident))


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def parity_figures(got, ref, dtype: str) -> dict:
    """Error of the timed run's output rows against the oracle's, with the
    bar the parity tests apply (bf16: max-abs <= 2e-2 and mean-abs <= 2e-3;
    fp32: max-abs <= 1e-5 max|ref|)."""
    import numpy as np

    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    max_abs, mean_abs = float(err.max()), float(err.mean())
    if dtype == "bf16":
        ok = max_abs <= 2e-2 and mean_abs <= 2e-3
        bar = "max-abs <= 2e-2, mean-abs <= 2e-3"
    else:
        ok = max_abs <= 1e-5 * float(np.abs(ref).max())
        bar = "max-abs <= 1e-5 max|ref|"
    return {"max_abs": max_abs, "mean_abs": mean_abs, "within_bar": bool(ok), "bar": bar}


def cpu_baseline(w, q, k, v, seconds: float, out=None) -> dict:
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole query rows against all N keys of one head, in chunks, until
    about ``seconds`` of CPU work.  Rate in the metric's unit (TFLOP/s).  With
    ``out`` (the timed run's output) the rows the oracle computed are also
    compared with it: the bench line carries its own parity figure."""
    import numpy as np
    import torch

    import oracle

    k64 = k[0, 0].to("cpu", torch.float64).numpy()
    v64 = v[0, 0].to("cpu", torch.float64).numpy()
    q64 = q[0, 0].to("cpu", torch.float64).numpy()
    chunk = 256
    rows_done, elapsed, r0 = 0, 0.0, 0
    ref_rows, ref_vals = [], []
    while elapsed < seconds and rows_done < q64.shape[0]:
        qs = q64[r0:r0 + chunk]
        t0 = time.perf_counter()
        o_ref = oracle.dense_attention(qs, k64, v64)
        elapsed += time.perf_counter() - t0
        if out is not None:
            ref_rows.append(np.arange(r0, r0 + qs.shape[0]))
            ref_vals.append(o_ref)
        rows_done += qs.shape[0]
        r0 = (r0 + chunk) % q64.shape[0]
    flops = 4.0 * rows_done * w.N * w.d
    parity = None
    if out is not None:
        rows = np.concatenate(ref_rows)
        got = out[0, 0, torch.from_numpy(rows).to(out.device)].to("cpu", torch.float64).numpy()
        parity = parity_figures(got, np.concatenate(ref_vals), w.dtype)
        parity["rows"] = int(len(rows))
        parity["sample"] = f"head 0, query rows {int(rows.min())}..{int(rows.max())} of the timed run's output"
    # the naive ring loop (init, P folds in ring order, finalize) on rows of
    # query block 0, for about a third of the time
    from oracle import ring as oring

    bounds = oring.block_bounds(w.N, w.P)
    q0 = q64[bounds[0][0]:bounds[0][1]]
    ring_rows, ring_elapsed, r0 = 0, 0.0, 0
    while ring_elapsed < seconds / 3 and ring_rows < q0.shape[0]:
        qs = q0[r0:r0 + chunk]
        t0 = time.perf_counter()
        st = oring.init_state((), qs.shape[0], w.d)
        for j in oring.ring_schedule(w.P, 0):
            st = oring.fold(st, qs, k64[bounds[j][0]:bounds[j][1]], v64[bounds[j][0]:bounds[j][1]])
        oring.finalize(st)
        ring_elapsed += time.perf_counter() - t0
        ring_rows += qs.shape[0]
        r0 = (r0 + chunk) % q0.shape[0]
    del np
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"fp64 dense oracle, {rows_done} query rows x {w.N} keys x d={w.d} of head 0 "
                  f"({elapsed:.1f} s; full workload is {w.B * w.H * w.n_q * w.b} rows)",
        "full_workload_s_extrapolated": round(w.flops() / (flops / elapsed), 1),
        "ring_loop": {"value": 4.0 * ring_rows * w.N * w.d / ring_elapsed / 1e12, "unit": "TFLOP/s",
                      "sample": f"fp64 naive ring loop, {ring_rows} rows of query block 0 folding all "
                                f"{w.P} blocks ({ring_elapsed:.1f} s)"},
        "host_cpus": len(os.sched_getaffinity(0)),
        "parity": parity,
    }


class ClockSampler:
    """Samples the shader clock the driver reports (the starred level of
    pp_dpm_sclk, in MHz) and the socket power (hwmon power1_input, in W, with
    the board's power1_cap) from a host thread while the timed steps run;
    reads sysfs files only, never the GPU."""

    def __init__(self, period_s: float = 0.02):
        import glob
        import threading

        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        hw = sorted(glob.glob(os.path.join(os.path.dirname(self.path), "hwmon", "hwmon*"))) if self.path else []
        self.power_path = os.path.join(hw[0], "power1_input") if hw else None
        self.cap_w = _read_watts(os.path.join(hw[0], "power1_cap")) if hw else None
        self.period = period_s
        self.samples: list[float] = []
        self.watts: list[float] = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            mhz = self._read()
            if mhz is not None:
                self.samples.append(mhz)
            w = _read_watts(self.power_path)
            if w is not None:
                self.watts.append(w)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self, value: float, peak: float) -> dict | None:
        if not self.samples:
            return None
        med = float(sorted(self.samples)[len(self.samples) // 2])
        # the published peak holds at the 2.4 GHz maximum shader clock
        at_clock = peak * med / 2400.0
        rec = {"source": "pp_dpm_sclk", "median_mhz": med, "min_mhz": min(self.samples),
               "max_mhz": max(self.samples), "samples": len(self.samples),
               "peak_at_clock": round(at_clock, 1), "pct_peak_at_clock": round(100.0 * value / at_clock, 2)}
        if self.watts:
            w = sorted(self.watts)
            rec["power"] = {"source": "hwmon power1_input", "median_w": round(w[len(w) // 2], 1),
                            "max_w": round(w[-1], 1), "cap_w": self.cap_w, "samples": len(w)}
        return rec


def _read_watts(path):
    """A hwmon power file (microwatts) in watts, or None."""
    if path is None:
        return None
    try:
        with open(path) as f:
            return int(f.read().strip()) / 1e6
    except (OSError, ValueError):
        return None


XGMI_LINK_GBPS = 153.0  # one MI355X xGMI link, one direction (GB/s)


def min_block_for_overlap(flop_rate: float, link_bytes_per_s: float, elem_bytes: int = 2) -> float:
    """Smallest block c (tokens per device) whose fold hides the next K/V block's
    transfer (vibeengines.com "Ring attention, explained", method step 7 and
    "At the extremes"): a step folds c keys into c queries, 4 d c^2 FLOP, while
    the next block, K and V of c rows of d elements, 2 c d elem_bytes bytes,
    crosses the link; the transfer hides when 4 d c^2 / F >= 2 c d e / B, i.e.
    c >= F e / (2 B), which is F / B for 16-bit elements (d cancels)."""
    return flop_rate * elem_bytes / (2.0 * link_bytes_per_s)


def links_needed(fold_flops: float, fold_s: float, kv_bytes: float, link_bytes_per_s: float) -> float:
    """How many links' bandwidth one ring step needs to hide its hand-off behind
    a fold of fold_flops FLOP that takes fold_s seconds: transfer time over one
    link divided by the fold time (<= 1: one link hides it).  Equals
    min_block_for_overlap(fold_flops / fold_s, link) / c for a c-token block."""
    return (kv_bytes / link_bytes_per_s) / fold_s


def device_sweep(torch, ra, steps: int, warmup: int) -> int:
    """One device's share of a ring step: fold one visiting block of b keys into
    the state of the resident block's b query rows (B1 H32 d128 bf16), timed with
    HIP events on the launch stream, against the time the next K/V block (2 b d
    bf16 per head) takes over one xGMI link.  The step hides the hand-off when the
    fold takes at least as long as the transfer on the links the ring uses.  The
    same fold run as a one-device ring (no state loaded or stored) gives the share
    of the step the state spill costs."""
    B, H, d = 1, 32, 128
    rows = []
    for b in (1024, 2048, 4096, 8192, 16384, 32768):
        g = torch.Generator(device="cuda").manual_seed(5000 + b)
        q, k, v = (torch.randn((B, H, b, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        m = torch.empty((B, H, b), device="cuda")
        l = torch.empty_like(m)
        o = torch.empty((B, H, b, d), device="cuda")
        ra.ra_state_init(m, l, o)
        out = torch.empty_like(q)
        ws = torch.empty(ra.ra_ring_workspace_bytes(q.dtype, B, H, b, d, 1, 1), dtype=torch.uint8, device="cuda")
        n = max(steps, 10) if b >= 8192 else max(steps, 50)

        def timed(fn):
            for _ in range(max(warmup, 3)):
                fn()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for _ in range(n):
                fn()
            end.record()
            torch.cuda.synchronize()
            return start.elapsed_time(end) / n

        ms = timed(lambda: ra.ra_fold_block(q, k, v, m, l, o))
        # the same fold as a one-device ring: no state loaded or stored, O written directly
        ms_nospill = timed(lambda: ra.ra_ring_forward(q, k, v, 1, out=out, workspace=ws))
        flops = 4.0 * B * H * b * b * d
        kv_bytes = 2.0 * B * H * b * d * 2
        xfer_ms = kv_bytes / (XGMI_LINK_GBPS * 1e9) * 1e3
        row = {"b": b, "fold_ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
               "fold_no_spill_ms": round(ms_nospill, 4), "spill_share": round(1.0 - ms_nospill / ms, 4),
               "kv_block_mb": round(kv_bytes / 1e6, 2), "xgmi_1link_ms": round(xfer_ms, 4),
               "links_needed": round(links_needed(flops, ms * 1e-3, kv_bytes, XGMI_LINK_GBPS * 1e9), 2),
               "min_b_one_link": round(min_block_for_overlap(flops / (ms * 1e-3), XGMI_LINK_GBPS * 1e9))}
        print(f"[bench] device sweep {row}", file=sys.stderr, flush=True)
        rows.append(row)
        del q, k, v, m, l, o, out, ws
    print(json.dumps({"mode": "device-sweep", "shape": {"B": B, "H": H, "d": d, "dtype": "bf16"},
                      "xgmi_link_gbps": XGMI_LINK_GBPS, "rows": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--causal", choices=("contiguous", "striped", "zigzag"), default=None,
                    help="run the causal ring with the inputs in this token layout")
    ap.add_argument("--backward", action="store_true", help="time the ring backward instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph (stream capture) and time its replays")
    ap.add_argument("--device-sweep", action="store_true",
                    help="time one device's fold step for several block sizes b against one block's xGMI transfer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a known-size reference for HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: record HBM bytes per launch of the selected workload and pass from two "
                         "rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of --copy-calibration runs")
    args = ap.parse_args()
    if args.traffic_from:
        sys.path.insert(0, ROOT)
        import workloads

        w = workloads.WORKLOADS[args.workload]
        return traffic_from(*args.traffic_from, w.name, w.dtype, args.backward, w.d)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the ring's P devices run as virtual steps on a single MI355X, "
              "so --gpus must be 1 (no multi-GPU path is built).", file=sys.stderr)
        return 2

    import torch

    import blockwise_online_softmax_fold_amd as ra
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    ra.load()
    if args.device_sweep:
        return device_sweep(torch, ra, args.steps, args.warmup)
    w = workloads.WORKLOADS[args.workload]
    print(f"[bench] workload {w.describe()} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    q, k, v = workloads.make_inputs(w, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(ra.ra_ring_workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, w.P, w.n_q), dtype=torch.uint8,
                     device="cuda")
    qb = w.query_blocks

    if args.backward:
        out, lse = ra.ra_ring_forward_ex(q, k, v, w.P, args.causal, query_blocks=qb)
        dout = torch.randn(out.shape, generator=torch.Generator(device="cuda").manual_seed(w.seed + 7),
                           device="cuda").to(out.dtype)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        del ws
        ws = torch.empty(ra.ra_ring_backward_workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, w.P, w.n_q),
                         dtype=torch.uint8, device="cuda")

    def step():
        if args.backward:
            ra.ra_ring_backward(q, k, v, out, dout, lse, w.P, args.causal, query_blocks=qb, dq=grads[0],
                                dk=grads[1], dv=grads[2], workspace=ws)
        elif args.causal:
            ra.ra_ring_forward_causal(q, k, v, w.P, args.causal, query_blocks=qb, out=out, workspace=ws)
        else:
            ra.ra_ring_forward(q, k, v, w.P, query_blocks=qb, out=out, workspace=ws)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    run_step = step
    if args.graph:
        # The fold launches are timed on eager steps; the step time on replays.
        ra.ra_profile_folds(True)
        prof_steps = max(1, min(args.steps, 3))
        for _ in range(prof_steps):
            step()
        torch.cuda.synchronize()
        launches, fold_ms_total, fold_ms_max = ra.ra_profile_read()
        ra.ra_profile_folds(False)
        launches = launches * args.steps / prof_steps
        fold_ms_total = fold_ms_total * args.steps / prof_steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run_step = graph.replay
        print("[bench] step captured into a HIP graph", file=sys.stderr, flush=True)
    else:
        ra.ra_profile_folds(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        start.record()
        for _ in range(args.steps):
            run_step()
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if not args.graph:
        launches, fold_ms_total, fold_ms_max = ra.ra_profile_read()
        ra.ra_profile_folds(False)
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # With every block resident in ring order (bf16, no mask) the library's folds
    # write the ring's hand-off themselves; in a full run (with the CPU baseline:
    # not the profiling runs, whose kernel counts this would change) the
    # side-stream copies (RA_HANDOFF_COPY=1), the stand-in the library uses
    # elsewhere, are timed on the same steps as a second figure.
    fused = (not args.backward and not args.causal and w.dtype == "bf16" and w.query_blocks is None
             and w.N % w.P == 0 and not os.environ.get("RA_HANDOFF_COPY"))
    copy_ms = None
    if fused and not (args.no_cpu_baseline or args.copy_calibration or args.graph):
        os.environ["RA_HANDOFF_COPY"] = "1"
        try:
            step()
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            for _ in range(args.steps):
                step()
            c1.record()
            torch.cuda.synchronize()
            copy_ms = c0.elapsed_time(c1) / args.steps
        finally:
            del os.environ["RA_HANDOFF_COPY"]
        print(f"[bench] same steps with the side-stream copies: {copy_ms:.3f} ms/step", file=sys.stderr, flush=True)

    pairs = (w.flops() / (4.0 * w.d)) if not args.causal else _visible_pairs(w, args.causal)
    flops = (10.0 if args.backward else 4.0) * w.d * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK[w.dtype]
    launches_per_step = launches / args.steps
    fold_avg_ms = fold_ms_total / launches
    flops_per_launch = flops / launches_per_step
    achieved = flops_per_launch / (fold_avg_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma" if w.dtype == "bf16" else "alu",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": None if args.causal else _traffic(w.name, w.dtype, args.backward, w.d),
        "kernel": (f"bwd_dq_kernel<{w.d}> + bwd_dkdv_kernel<{w.d}> (one step)" if args.backward
                   else f"fold_{w.dtype}_kernel<{w.d}>"),
        "flop_per_launch": flops_per_launch,
        "avg_launch_ms": round(fold_avg_ms, 4),
        "max_launch_ms": round(fold_ms_max, 4),
        "launches": launches,
    }
    rec = {
        "metric": METRIC if not args.backward else METRIC.replace("ring-fold attention", "ring-fold attention backward"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "P": w.P, "b": w.b,
                   "resident_query_blocks": w.n_q, "seed": w.seed, "causal": args.causal or False,
                   "pass": "backward" if args.backward else "forward",
                   "launch": "hip-graph" if args.graph else "eager",
                   "handoff": ("written by the folds" if fused else
                               "none (K, V read in place)" if args.backward else "side-stream copies")},
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "exps_per_s": pairs * (2.0 if args.backward else 1.0) / (ms * 1e-3),
        "roofline": roofline,
        "clock": clock.summary(tflops, peak),
    }
    if copy_ms is not None:
        rec["handoff_copy"] = {"ms_per_step": round(copy_ms, 4), "value": round(flops / (copy_ms * 1e-3) / 1e12, 2),
                               "unit": "TFLOP/s", "steps": args.steps,
                               "note": "the same ring with the hand-off as hipMemcpy2DAsync on a side stream "
                                       "(RA_HANDOFF_COPY=1), timed after the main steps"}
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        # the output rows the oracle computes are checked against the last timed
        # step's output (full attention, forward only: what the oracle computes)
        check = out if not (args.backward or args.causal) else None
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, out=check)
        rec["parity"] = rec["cpu_baseline"].pop("parity")
    else:
        rec["cpu_baseline"] = None
        rec["parity"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
