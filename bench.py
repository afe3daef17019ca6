"""Benchmark of the block-scaled attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]
    python bench.py --trace-summary DIR --steps K --warmup W

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM: quantise Q, K, V (FP8 per block or MXFP4 for Q/K, FP8
per channel for V; for sliding-tile workloads with the fused 3D tile
reorder) and run the fused attention kernel.  The sliding-tile plan is built
once per shape on the host (it is a per-shape cost, like a compiled graph).

Prints one JSON line: the metric is effective attention TFLOPS =
algorithmic FLOPs / time, with FLOPs = 4 N^2 d H for dense attention (causal:
4 d H N(N+1)/2; sliding-tile and padded grids: only real query-key pairs that
are computed).  `value` uses the whole step (quantisers + attention);
`roofline` is for the attention kernel alone, timed with events on the stream
it runs on.  `cpu_baseline` times the CPU oracle: its quantisers on the full
tensors and its attention on 4096 seeded (head, query) rows.

`roofline.traffic` (HBM bytes per attention launch) comes from the committed
counter summary profiles/attention_<workload>_counters.md, made by two
rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script with
--copy-bytes, which adds a plain device copy of known size to calibrate the
counters.  It is reported only while the attention kernel's sources hash to
the value recorded there, and is null otherwise.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, make_inputs, sample_rows  # noqa: E402

DEFAULT_CONFIG = "dense_mxfp4_16k"
# MI355X dense peaks (no sparsity), TFLOP/s
PEAK_FP8 = 5000.0
PEAK_FP4 = 10100.0
PEAK_BF16 = 2500.0
# sources that define the attention kernel's code; a counter summary is valid
# only for the sources it was taken on
KERNEL_SOURCES = ("attention.hip", "pab_device.h", "pab_internal.h", "pab_lds.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attention_%s_counters.md")


def kernel_sources_sha256():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "precision_attention_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or
    None if there is none or the kernel sources changed since it was taken."""
    path = TRAFFIC_SUMMARY % workload
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "kernel_sources_sha256", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes, reps=3):
    """A plain device-to-device copy of nbytes, for calibrating the HBM byte
    counters (each launch reads and writes exactly nbytes)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def algorithmic_flops(cfg, plan=None):
    d, H, B = cfg.d, cfg.H, cfg.B
    if cfg.mode == "sta":
        real = plan.kv_valid.reshape(plan.n_tiles, plan.tile_tokens).sum(axis=1).astype(np.float64)
        pairs = 0.0
        for u in range(plan.n_tiles):
            lst = plan.win_idx[plan.win_off[u]:plan.win_off[u + 1]]
            pairs += real[u] * real[lst].sum()
        return 4.0 * d * H * B * pairs
    n = float(cfg.n_real)
    if cfg.mode == "causal":
        return 4.0 * d * H * B * n * (n + 1) / 2
    return 4.0 * d * H * B * n * n


def roofline_peak(cfg):
    """Peak of the attention contraction for this recipe: MXFP4 QK^T + FP8 P.V
    blend the FP4 and FP8 rates; both products in MXFP4 run at the FP4 rate;
    the FP8 recipe is priced at the FP8 rate."""
    if cfg.recipe == "mxfp4":
        return 2.0 / (1.0 / PEAK_FP4 + 1.0 / PEAK_FP8)
    if cfg.recipe == "mxfp4_pv":
        return PEAK_FP4
    return PEAK_FP8


class GpuPath:
    """Device tensors and one step of the path through the C ABI."""

    def __init__(self, cfg, x, lib, tau=0):
        import torch
        self.cfg, self.lib, self.tau = cfg, lib, tau
        dev = torch.device("cuda:0")
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q_t", "k_t", "v_t"))
        self.plan = None
        self.dplan = None
        if cfg.grid is not None:
            self.plan = lib.sta_plan(cfg.grid, cfg.real_grid, cfg.tile,
                                     cfg.window if cfg.window else (99, 99, 99))
            self.dplan = lib.DevicePlan(self.plan, dev)
        self.out = torch.empty((cfg.B, cfg.H, cfg.n_real, cfg.d), dtype=torch.float32, device=dev)
        self.q_operand = False

    def quantize(self):
        cfg, lib = self.cfg, self.lib
        perm = self.dplan.perm if self.dplan is not None else None
        n_out = cfg.n_kernel
        if cfg.recipe == "fp8":
            # the forward reads K's bf16 operand copy and decodes Q's codes itself;
            # the backward reads both copies
            qq = lib.quantize(self.q, "fp8_block", cfg.blk, perm, n_out, operand=self.q_operand)
            kq = lib.quantize(self.k, "fp8_block", cfg.blk, perm, n_out)
        else:
            qq = lib.quantize(self.q, "mxfp4", None, perm, n_out)
            kq = lib.quantize(self.k, "mxfp4", None, perm, n_out)
        vq = lib.quantize(self.v, "mxfp4_v" if cfg.recipe == "mxfp4_pv" else "fp8_channel", None,
                          perm, n_out)
        return qq, kq, vq

    def attend(self, qq, kq, vq):
        cfg, lib = self.cfg, self.lib
        if cfg.mode == "sta":
            return lib.attention_sta(qq, kq, vq, self.dplan, out=self.out, tau=self.tau, steps=True)
        if self.dplan is not None:
            return lib.attention_dense(qq, kq, vq, kv_valid=self.dplan.kv_valid,
                                       out_perm=self.dplan.perm, n_out=cfg.n_real, out=self.out,
                                       tau=self.tau, key_tiles=self.dplan.key_tiles)
        return lib.attention_dense(qq, kq, vq, causal=cfg.mode == "causal", out=self.out,
                                   tau=self.tau)


def time_gpu(path, steps, warmup):
    import torch
    st = torch.cuda.current_stream()
    for _ in range(warmup):
        path.attend(*path.quantize())
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(st)
        ops = path.quantize()
        e1.record(st)
        path.attend(*ops)
        e2.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = [a.elapsed_time(b) for a, b, _ in ev]
    a_ms = [b.elapsed_time(c) for _, b, c in ev]
    return wall, q_ms, a_ms


def time_backward(cfg, path, steps, warmup):
    """The backward pass (prep kernels, dK/dV, dQ) of the dense, causal or
    sliding-tile workload: one forward with the row statistic (sliding-tile:
    in the kernel's token order), then `steps` timed backward calls on a seeded
    bf16 dO; returns per-call milliseconds."""
    import torch
    lib = path.lib
    path.q_operand = True
    qq, kq, vq = path.quantize()
    causal = cfg.mode == "causal"
    sta = cfg.mode == "sta"
    if sta:
        out, lse = lib.attention_sta(qq, kq, vq, path.dplan, use_out_perm=False, lse=True, steps=True)
    else:
        out, lse = lib.attention_dense(qq, kq, vq, causal=causal, lse=True)
    g = torch.Generator(device="cpu").manual_seed(1000 * cfg.index + 7)
    dout = torch.randn(out.shape, generator=g).to(torch.bfloat16).cuda()
    ws = torch.empty(lib.backward_workspace_bytes(cfg.B, cfg.H, cfg.n_kernel, cfg.d),
                     dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(out) for _ in range(3))
    if sta:
        call = lambda: lib.attention_sta_backward(qq, kq, vq, path.dplan, out, dout, lse,
                                                  workspace=ws, grads=grads)
    else:
        call = lambda: lib.attention_backward(qq, kq, vq, out, dout, lse, causal=causal,
                                              workspace=ws, grads=grads)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(st)
        call()
        e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in ev]


def backward_main(args, cfg, path):
    if cfg.mode not in ("dense", "causal", "sta") or (cfg.mode != "sta" and path.dplan is not None):
        print("--backward runs the dense, causal and sliding-tile workloads (the backward pass "
              "has no token-permuted dense form)", file=sys.stderr)
        sys.exit(2)
    print("[bench] timing %d backward steps after %d warm-up" % (args.steps, args.warmup),
          file=sys.stderr, flush=True)
    wall, ms = time_backward(cfg, path, args.steps, args.warmup)
    # five products of 2 d per computed (query, key) pair (causal: half; sliding-tile: the
    # real pairs of the windows)
    flops = 2.5 * algorithmic_flops(cfg, path.plan if cfg.mode == "sta" else None)
    ms_call = float(np.mean(ms))
    achieved = flops / (ms_call * 1e-3) / 1e12
    result = {
        "metric": "effective attention backward TFLOPS (10*N^2*d*H: dQ, dK, dV) + % of bf16 "
                  "MFMA peak, 1 GPU",
        "value": round(flops / (wall / args.steps) / 1e12, 2),
        "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16, outlier channels as configured; dO N(0,1) bf16)",
        "config": {"workload": cfg.name + "_backward", "desc": "backward pass of " + cfg.desc,
                   "B": cfg.B, "H": cfg.H, "N": cfg.n_real, "d": cfg.d, "mode": cfg.mode,
                   "recipe": cfg.recipe, "algorithmic_flops": flops,
                   "backward_ms": round(ms_call, 4),
                   "backward_ms_median": round(float(np.median(ms)), 4),
                   "backward_ms_min_max": [round(min(ms), 4), round(max(ms), 4)]},
        "roofline": {"bound": "mfma", "kernel": "whole backward call (prep, dK/dV, dQ)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result))


_ORACLE_PLAN = {}


def _oracle_plan_cached(cfg):
    if cfg.name not in _ORACLE_PLAN:
        _ORACLE_PLAN[cfg.name] = _oracle_plan(cfg)
    return _ORACLE_PLAN[cfg.name]


def _oracle_quantize_head(job):
    """Worker: the oracle's quantisers on one head's full Q, K and V (after the
    3D token reorder on grid workloads); returns the operands and the time."""
    from oracle import attention as OA
    from oracle import quant as OQ
    from oracle import sta as OS
    name, q, k, v = job
    cfg = CONFIGS[name]
    t0 = time.perf_counter()
    if cfg.grid is not None:
        perm = _oracle_plan_cached(cfg).perm
        q, k, v = (OS.gather_tokens(a[None], perm)[0] for a in (q, k, v))
    if cfg.recipe == "fp8":
        qo = OA.Operand("fp8_block", *OQ.fp8_block_quantize(q, cfg.blk), cfg.blk)
        ko = OA.Operand("fp8_block", *OQ.fp8_block_quantize(k, cfg.blk), cfg.blk)
    else:
        qo = OA.Operand("mxfp4", *OQ.mxfp4_quantize(q))
        ko = OA.Operand("mxfp4", *OQ.mxfp4_quantize(k))
    if cfg.recipe == "mxfp4_pv":
        vo = OA.Operand("mxfp4_tokens", *OQ.mxfp4_token_quantize(v))
    else:
        vo = OA.Operand("fp8_channel", *OQ.fp8_channel_quantize(v))
    return (qo, ko, vo), time.perf_counter() - t0


def _oracle_rows(job):
    """Worker: the oracle recipe for one head's sampled query rows (raster
    tokens); returns the computed (query, key) pairs and the time."""
    from oracle import attention as OA
    from oracle import sta as OS
    name, ops, tokens, bn = job
    cfg = CONFIGS[name]
    qo, ko, vo = ops
    sm = 1.0 / np.sqrt(cfg.d)
    t0 = time.perf_counter()
    pairs = 0.0
    if cfg.grid is not None:
        plan = _oracle_plan_cached(cfg)
        ok = plan.perm >= 0
        inv = np.empty(int(ok.sum()), np.int64)
        inv[plan.perm[ok]] = np.nonzero(ok)[0]
        rows = inv[np.asarray(tokens, np.int64)]
        tiles = rows // plan.tile_tokens
        for u in np.unique(tiles):
            sel = rows[tiles == u]
            kb = OS.key_blocks_for_tile(plan, int(u), bn)
            OA.recipe_attention(qo, ko, vo, sel, sm_scale=sm, bn=bn, kv_valid=plan.kv_valid,
                                key_blocks=kb)
            keys = plan.kv_valid[np.concatenate([np.arange(s, s + bn) for s in kb])].sum()
            pairs += float(len(sel)) * float(keys)
    else:
        rows = np.sort(np.asarray(tokens, np.int64))
        OA.recipe_attention(qo, ko, vo, rows, sm_scale=sm, bn=bn, causal=cfg.mode == "causal")
        pairs = float((rows + 1).sum()) if cfg.mode == "causal" else float(len(rows)) * cfg.n_real
    return pairs, time.perf_counter() - t0


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def cpu_baseline(cfg, x, bn, rows=4096):
    """The oracle (as it stands) on the host cores: its quantisers on the full
    Q, K, V tensors, then the recipe on `rows` seeded (head, query) rows drawn
    uniformly over heads x real tokens; one worker process per core, heads
    dealt over them, one BLAS thread each.  The value is the attention's
    effective TFLOPS on the sampled rows (the same FLOP formula as the GPU:
    4 d per computed pair); the quantisers' wall time is reported beside it."""
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    heads, tokens = sample_rows(cfg, rows)
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        qjobs = [(cfg.name, x["q"][0, h], x["k"][0, h], x["v"][0, h]) for h in range(cfg.H)]
        quant = pool.map(_oracle_quantize_head, qjobs, chunksize=1)
        t_quant = time.perf_counter() - t0
        t1 = time.perf_counter()
        ajobs = [(cfg.name, quant[h][0], tokens[heads == h], bn) for h in range(cfg.H)
                 if np.any(heads == h)]
        res = pool.map(_oracle_rows, ajobs, chunksize=1)
        t_att = time.perf_counter() - t1
    pairs = sum(p for p, _ in res)
    in_bytes = 3 * x["q"].size * (2 if cfg.dtype == "bf16" else 4)
    return {"value": 4.0 * cfg.d * pairs / t_att / 1e12, "unit": "TFLOPS", "cores": cores,
            "kind": "oracle",
            "sample": "oracle quantisers on the full Q, K, V (%d heads) in %.1f s (%.2f GB/s of "
                      "input); oracle recipe attention on %d seeded (head, query) rows in %.1f s; "
                      "%d worker processes" % (cfg.H, t_quant, in_bytes / t_quant / 1e9,
                                               len(tokens), t_att, cores),
            "quantize_s": round(t_quant, 3), "attention_s": round(t_att, 3), "rows": int(len(tokens)),
            "attention_s_full_problem_extrapolated": round(
                t_att / len(tokens) * cfg.H * cfg.n_real, 1)}


def trace_summary(path, steps, warmup):
    """Markdown summary of a rocprofv3 --kernel-trace CSV run of this script
    (with the same --steps and --warmup): per kernel, the launches of the
    timed steps only, the first `warmup` steps' launches left out.  A kernel
    whose launch count is not a multiple of the step count (the counter
    calibration copy) is listed with all its launches."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit("no *kernel_trace.csv under %s" % path)
    launches = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                launches.setdefault(r["Kernel_Name"], []).append((t0, (t1 - t0) / 1e3))
    total_steps = steps + warmup
    rows, timed_total = [], 0.0
    for name, lst in launches.items():
        lst.sort()
        per_step = len(lst) // total_steps
        if per_step >= 1 and per_step * total_steps == len(lst):
            durs = [d for _, d in lst[per_step * warmup:]]
            note = "%d per step" % per_step
        else:
            durs = [d for _, d in lst]
            note = "not per step: all launches"
        timed_total += sum(durs)
        rows.append((name.split("(")[0].replace("void ", ""), durs, note))
    rows.sort(key=lambda r: -sum(r[1]))
    out = ["| kernel | launches counted | median µs | mean µs | min µs | max µs | share of counted GPU time |",
           "|---|---|---|---|---|---|---|"]
    for name, durs, note in rows:
        out.append("| `%s` | %d (%s) | %.1f | %.1f | %.1f | %.1f | %.2f%% |" % (
            name, len(durs), note, float(np.median(durs)), float(np.mean(durs)), min(durs), max(durs),
            100.0 * sum(durs) / timed_total))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--tau", type=int, default=0,
                    help="softmax rescale threshold in log2 units (0 = rescale on every rise of "
                         "the running maximum, the default recipe)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV) of a dense or causal workload "
                         "instead of the forward step")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain device copy of this many bytes "
                         "(counter calibration for rocprofv3 --pmc runs)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print the per-kernel summary of a rocprofv3 --kernel-trace CSV run of this "
                         "script made with the same --steps and --warmup (warm-up launches left out) "
                         "and exit; needs no GPU")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.steps, args.warmup))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from precision_attention_block_amd import binding as lib
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib.lib()
    cfg = CONFIGS[args.config]
    print("[bench] config %s: generating inputs" % cfg.name, file=sys.stderr, flush=True)
    x = make_inputs(cfg, as_torch=True)
    path = GpuPath(cfg, x, lib, args.tau)
    if args.backward:
        backward_main(args, cfg, path)
        return
    mode = {"dense": 0, "causal": 1, "sta": 2}[cfg.mode]
    _, bn = lib.attention_info("fp8_block" if cfg.recipe == "fp8" else "mxfp4", cfg.d, mode)
    print("[bench] timing %d steps after %d warm-up" % (args.steps, args.warmup), file=sys.stderr,
          flush=True)
    wall, q_ms, a_ms = time_gpu(path, args.steps, args.warmup)
    flops = algorithmic_flops(cfg, path.plan)
    ms_step = wall * 1e3 / args.steps
    att_ms = float(np.mean(a_ms))
    achieved = flops / (att_ms * 1e-3) / 1e12
    peak = roofline_peak(cfg)
    dense_equiv = 4.0 * cfg.d * cfg.H * cfg.B * float(cfg.n_real) ** 2
    result = {
        "metric": "effective attention TFLOPS (4*N^2*d*H) + % of FP8/MXFP4 MFMA peak, 1 GPU",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp4": "mxfp4+fp8", "mxfp4_pv": "mxfp4"}.get(cfg.recipe, "fp8"),
        "data": "synthetic (seeded N(0,1), bf16, outlier channels as configured)",
        "config": {"workload": cfg.name, "desc": cfg.desc, "B": cfg.B, "H": cfg.H,
                   "N": cfg.n_real, "N_kernel": cfg.n_kernel, "d": cfg.d, "mode": cfg.mode,
                   "recipe": cfg.recipe, "block_tokens": cfg.blk if cfg.recipe == "fp8" else 32,
                   "BN": bn, "tau": args.tau, "algorithmic_flops": flops,
                   "dense_equivalent_flops": dense_equiv,
                   "quantize_ms": round(float(np.mean(q_ms)), 4),
                   "attention_ms": round(att_ms, 4),
                   "attention_ms_median": round(float(np.median(a_ms)), 4),
                   "attention_ms_min_max": [round(min(a_ms), 4), round(max(a_ms), 4)],
                   "attention_tflops": round(achieved, 2),
                   "pct_fp8_peak": round(100 * achieved / PEAK_FP8, 2),
                   "pct_fp4_peak": round(100 * achieved / PEAK_FP4, 2) if cfg.recipe != "fp8" else None},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(cfg.name) if args.tau == 0 else None},
    }
    if args.copy_bytes > 0:
        copy_calibration(args.copy_bytes)
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, x, bn)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


def _oracle_plan(cfg):
    from oracle import sta as OS
    return OS.plan(cfg.grid, cfg.real_grid, cfg.tile, cfg.window if cfg.window else (99, 99, 99))


if __name__ == "__main__":
    main()
