"""Benchmark of the SmoothQuant W8A8 linear path (+ bf16 LoRA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of the workload, for
every input group: calibrate the per-channel maxima, compute the smoothing
vector and fold it into INT8 weights, quantize the activations per token,
run the INT8 GEMM with its dequant epilogue for every projection, and add the
bf16 LoRA delta. The default workload is the Llama-3-8B projection set at
M=2048 tokens. Inputs are seeded synthetic tensors, resident in HBM before the
timed region starts.

The input groups are independent, so a timed step issues every group as one
native call (sq_linear_group_run: calibrate, fold, quantize, LoRA shrink,
GEMM) on one of three streams, largest group first, and the groups' kernels
overlap. The timed steps are issued back to back, each group staying on its
own stream.

Output: one JSON line. `value` is GEMM INT8 tera-operations per second of the
whole step (2*M*N*K summed over the projections, divided by the step time).
HIP events that the library records on each GEMM's stream right around its
launch give the GEMM's own rate, reported as its roofline fraction against the
MI355X dense INT8 MFMA peak. Per-stage times come from a few extra untimed steps issued in order
on one stream. The CPU oracle is timed on a bounded sample of the same step
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
DEFAULT_WORKLOAD = "llama3_8b_proj_m2048"
GEMM_KERNEL_SRC = os.path.join(ROOT, "w8a8_smoothquant_int8_amd", "csrc", "k_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_{tile}_hbm_traffic_llama3_8b_proj_m2048.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="activation rows per input in the CPU-oracle sample")
    ap.add_argument("--no-stages", action="store_true",
                    help="skip the untimed per-stage pass (so a kernel trace of the run covers "
                         "only the warmup and timed steps)")
    ap.add_argument("--row", choices=sorted(ROWS), default=None,
                    help="measure one of the widened rows instead of the whole step "
                         "(one JSON line of its own)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the timed region, run one plain device copy of this many MiB "
                         "(a kernel of known traffic, to scale rocprofv3 byte counters)")
    return ap.parse_args()


def kernel_hash(path: str) -> str:
    """Hash of a kernel source's code: comments and whitespace are stripped, so
    editing a comment does not invalidate the counters taken on the code."""
    with open(path, encoding="utf-8") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def stored_traffic(tile: str):
    """HBM bytes per launch of the dominant GEMM kernel from the rocprofv3
    FETCH_SIZE/WRITE_SIZE runs, if they were taken on the current GEMM source."""
    path = TRAFFIC_FILE.format(tile=tile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("gemm_source_sha256_16") != kernel_hash(GEMM_KERNEL_SRC):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timeline:
    """HIP events recorded on the launch stream between kernel calls."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self, tag, group=None):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append((tag, group, e))

    def durations(self):
        """{tag: [ms, ...]} and {group: [ms, ...]} for the GEMM launches."""
        out, gemm = {}, {}
        for (tag, grp, e0), (_, _, e1) in zip(self.marks, self.marks[1:]):
            if tag is None:
                continue
            ms = e0.elapsed_time(e1)
            out.setdefault(tag, []).append(ms)
            if tag == "gemm":
                gemm.setdefault(grp, []).append(ms)
        return out, gemm


def setup(wl, torch):
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    groups = []
    for inp, _K in wl.inputs:
        rows = wl.group_rows(inp)
        loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows} if wl.lora_rank else {}
        g = LinearGroup(wl.w_group(inp).cuda(), rows, wl.alpha, wl.out_dtype, wl.M, lora=loras)
        groups.append((inp, g, wl.x(inp).cuda(), wl.x_cal(inp).cuda()))
    torch.cuda.synchronize()
    return groups


def run_step(groups, tl=None):
    """One pass of the whole path over one batch, every input group, in issue
    order on the current stream (the instrumented pass: HIP events between
    the launches give the per-stage times)."""
    mark = tl.mark if tl is not None else (lambda tag, **kw: None)
    for inp, g, X, Xc in groups:
        mark("calibrate")
        g.calibrate(Xc)
    for inp, g, X, Xc in groups:
        mark("smooth_fold")
        g.fold()
    for inp, g, X, Xc in groups:
        mark("quant")
        g.quantize(X)
        if g.fused:
            mark("lora_shrink")
            g.lora_shrink(X)
            mark("gemm", group=inp)
            g.gemm_all_lora()
        else:
            mark("gemm", group=inp)
            g.gemm_all()
    mark(None)


# HIP maps streams onto a few hardware queues (4 by default, one of them taken
# by the null stream); two streams that share a queue run in order. Three
# streams get a queue each.
N_STREAMS = 3


class Streams:
    """The step's streams (default priority) and the group -> stream plan:
    groups in descending order of GEMM work, each on the stream with the least
    work so far (longest-processing-time first). The longest chain starts
    first and never queues behind another group. Measured on the Llama-3-8B
    step: 0.78 ms against 0.85 ms for one stream per group in workload order
    (two of those four streams then shared a hardware queue)."""

    def __init__(self, torch, groups, n_streams=N_STREAMS):
        self.torch = torch
        work = [2.0 * g.M * g.Ntot * g.K for _inp, g, _x, _c in groups]
        self.plan = plan_streams(work, n_streams)       # (group index, stream index), issue order
        self.main = [torch.cuda.Stream() for _ in range(min(n_streams, len(groups)))]


def plan_streams(work, n_streams):
    """Longest-processing-time plan: groups in descending work (ties in input
    order), each to the stream with the least work so far (ties: the lowest
    index). Returns [(group index, stream index)] in issue order."""
    n = min(n_streams, len(work))
    load = [0.0] * n
    plan = []
    for gi in sorted(range(len(work)), key=lambda i: (-work[i], i)):
        si = min(range(n), key=lambda j: (load[j], j))
        load[si] += work[gi]
        plan.append((gi, si))
    return plan


def run_step_streams(groups, st, gemm_ev=None, join=True):
    """One pass of the whole path over one batch. The input groups are
    independent: each runs calibrate -> fold -> quantize -> LoRA shrink ->
    GEMM as one native call (sq_linear_group_run) on the stream the plan gives
    it, so the groups' short, latency-bound kernels fill each other's gaps and
    a GEMM whose tiles leave CUs idle in its last round shares the chip with
    another group's work. gemm_ev: {group: [(start, end), ...]} collects HIP
    events that the library records on the group's stream right around its
    GEMM, for the groups in gemm_ev["groups"].

    join=False leaves out the step's fork from and join into the current
    stream: back-to-back steps then run as the streams allow. A group always
    runs on the same stream, so its consecutive steps stay in order and its
    buffers are never touched by two steps at once; groups share no buffers."""
    torch = st.torch
    cur = torch.cuda.current_stream()
    if join:
        for sm in st.main:
            sm.wait_stream(cur)
    for gi, si in st.plan:
        inp, g, X, Xc = groups[gi]
        e0 = e1 = None
        if gemm_ev is not None and inp in gemm_ev["groups"]:
            e0, e1 = gemm_ev["pool"].pop()
            gemm_ev.setdefault(inp, []).append((e0, e1))
        g.run(X, Xc, stream=st.main[si], gemm_begin=e0, gemm_end=e1)
    if join:
        for sm in st.main:
            cur.wait_stream(sm)


def event_pool(torch, n):
    """n (start, end) pairs of timing events, created up front (a first record
    creates the underlying HIP event) so the library can record them."""
    pool = []
    for _ in range(n):
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in pair:
            e.record()
        pool.append(pair)
    torch.cuda.synchronize()
    return pool


def _tile_score(M, N, bm, bn, resident, rate):
    tm, tn = -(-M // bm), -(-N // bn)
    tiles = tm * tn
    rounds = -(-tiles // resident)
    pad = (M / (tm * bm)) * (N / (tn * bn))
    return rate * pad * tiles / (rounds * resident)


def gemm_tile(M: int, N: int, K: int) -> str:
    """The tile configuration libsq picks for an INT8 GEMM of this shape (the
    library's rule: the generic kernel when K is not a multiple of 128 or an
    operand reaches 4 GiB, the skinny kernel for M <= 64 with fewer than 96
    column tiles of 128, else the best of
    256x256 tiles and 256x192 tiles,
    one block per CU, at rates 1 and 0.93, and 128x128 tiles, two blocks per
    CU, at 0.8, each scored by the padding and the fraction of the last round
    of blocks that does useful work; ties go to 256x256, then 256x192)."""
    if K % 128 or M * K >= 1 << 32 or N * K >= 1 << 32:
        return "generic"
    if M <= 64 and (N + 127) // 128 < 96:
        return "skinny"
    s256 = _tile_score(M, N, 256, 256, 256, 1.0)
    s192 = _tile_score(M, N, 256, 192, 256, 0.93)
    s128 = _tile_score(M, N, 128, 128, 512, 0.8)
    if s256 >= s192 and s256 >= s128:
        return "256x256"
    return "256x192" if s192 >= s128 else "128x128"


def cpu_baseline(wl, rows_per_input: int):
    """The oracle as it stands, on a bounded sample of one step: weights are
    folded in full; the activation path (quantize, INT8 GEMM, dequant, LoRA)
    runs on `rows_per_input` rows of each input and is scaled to all M rows."""
    import numpy as np
    import oracle.sq_oracle as O
    from threadpoolctl import threadpool_info

    t_fixed = 0.0
    t_rows = 0.0
    m = min(rows_per_input, wl.M)
    for inp, _K in wl.inputs:
        X = wl.x(inp).float().numpy()[:m]
        Xc = wl.x_cal(inp).float().numpy()
        W = wl.w_group(inp).float().numpy()
        rows = wl.group_rows(inp)
        t0 = time.perf_counter()
        act_max = O.calibrate_absmax(Xc)
        s = O.smoothing_scale(act_max, O.weight_absmax(W), wl.alpha)
        wq, wsc = O.fold_and_quantize_weights(W, s)
        t1 = time.perf_counter()
        xq, a = O.quantize_per_token(X, s)
        for p, (r0, r1) in rows.items():
            y = O.dequantize(O.int8_gemm(xq, wq[r0:r1]), a, wsc[r0:r1], wl.out_dtype)
            if wl.lora_rank:
                A, B = wl.lora(p)
                O.lora_apply(y, X, wl.dtype, A.float().numpy(), B.float().numpy(), 1.0, wl.out_dtype)
        t2 = time.perf_counter()
        t_fixed += t1 - t0
        t_rows += t2 - t1
    step_s = t_fixed + t_rows * (wl.M / m)
    threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    return {
        "value": wl.gemm_ops() / step_s / 1e12,
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one step of {wl.name}: weights calibrated/smoothed/folded in full "
                   f"({t_fixed:.1f} s); quantize+GEMM+dequant+LoRA on {m} of {wl.M} rows per input "
                   f"({t_rows:.1f} s) scaled x{wl.M / m:g}; numpy oracle, BLAS threads={threads}"),
        "step_s": step_s,
    }


def time_launches(torch, fn, reps: int, warm: int = 3) -> float:
    """Average ms of fn() over reps launches on the current stream (HIP events)."""
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def row_f3(args, torch):
    """Static per-tensor quant with and without the clipped-code counter on the
    OPT-13B layer inputs at M = 4096 (fp16), and the cost of the range-checked
    forward pass. Algorithmic bytes per element: the fp16 input read and the
    INT8 code written (3 bytes)."""
    from synth.workloads import get_workload
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    import w8a8_smoothquant_int8_amd as sq
    wl = get_workload("opt13b_layer_prefill_m4096")
    reps = max(args.steps, 10)
    per_input, best = {}, None
    for inp, K in wl.inputs:
        g = LinearGroup(wl.w_group(inp).cuda(), wl.group_rows(inp), wl.alpha, wl.out_dtype, wl.M,
                        modes=("dynamic", "static"))
        g.calibrate(wl.x_cal(inp).cuda())
        g.fold()
        X = wl.x(inp).cuda()
        plain = time_launches(torch, lambda: g.quantize(X, "static"), reps)
        g.reset_clips()
        clip = time_launches(torch, lambda: g.quantize(X, "static", count_clips=True), reps)
        rate = g.clip_rate()
        fwd = time_launches(torch, lambda: g.forward(X, "static"), max(reps // 4, 5))
        chk = time_launches(torch, lambda: g.forward_static_checked(X, max_rate=1.0),
                            max(reps // 4, 5))
        nbytes = 3.0 * wl.M * K
        per_input[inp] = {"K": K, "plain_us": round(plain * 1e3, 2), "clip_us": round(clip * 1e3, 2),
                          "plain_gbs": round(nbytes / plain / 1e6, 1),
                          "clip_gbs": round(nbytes / clip / 1e6, 1),
                          "counter_overhead_pct": round(100 * (clip / plain - 1), 2),
                          "clip_rate": rate,
                          "forward_static_ms": round(fwd, 4),
                          "forward_static_checked_ms": round(chk, 4)}
        if best is None or nbytes / clip > best[0]:
            best = (nbytes / clip, clip, nbytes, inp)
        del g, X
        torch.cuda.empty_cache()
    gbs, ms, nbytes, inp = best
    return {
        "row": "f3", "metric": "static per-tensor quant with clip counter, GB/s",
        "value": round(nbytes / ms / 1e6, 1), "unit": "GB/s",
        "higher_is_better": True, "dtype": "f16->int8", "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "reps": reps},
        "roofline": {"bound": "hbm", "kernel": f"k_quant (STATIC_CLIP) on {inp}",
                     "achieved": round(nbytes / ms / 1e6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 5), "bytes_per_launch": nbytes},
        "inputs": per_input,
    }


def row_f4(args, torch):
    """Per-layer alpha sweep over the Llama-3-8B projection groups: 21 alphas
    (0, 0.05, ..., 1) on the 512-row calibration batch, one native call per
    group. Also times the sweep's largest memory-bound kernel, the weight fold
    + quant, alone at each group's shape (3 bytes per weight element: 16-bit
    read, INT8 write)."""
    from synth.workloads import get_workload
    import w8a8_smoothquant_int8_amd as sq
    wl = get_workload(args.workload)
    alphas = [round(0.05 * i, 2) for i in range(21)]
    reps = max(min(args.steps, 20), 3)
    groups, total_ms, best_fold = {}, 0.0, None
    for inp, K in wl.inputs:
        X = wl.x_cal(inp).cuda()
        W = wl.w_group(inp).cuda()
        M, N = X.shape[0], W.shape[0]
        ws = torch.empty(sq.sq_alpha_sweep_workspace_bytes(M, N, K), dtype=torch.uint8,
                         device="cuda")
        err = torch.empty(len(alphas), 2, dtype=torch.float64, device="cuda")
        ms = time_launches(torch, lambda: sq.sq_alpha_sweep(X, W, alphas, err, ws), reps, warm=1)
        host = err.cpu().numpy()
        rel = host[:, 0] / host[0, 1]
        ib = int(rel.argmin())
        # the fold + quant kernel alone, at the sweep's shape
        s = torch.empty(K, dtype=torch.float32, device="cuda")
        am = torch.zeros(K, dtype=torch.float32, device="cuda")
        sq.sq_calibrate_absmax(X, am)
        sq.sq_smooth_scale(am, W, 0.5, s)
        Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
        wsc = torch.empty(N, dtype=torch.float32, device="cuda")
        fold_ms = time_launches(torch, lambda: sq.sq_fold_quant_weights(W, s, Wq, wsc), reps * 5)
        fold_bytes = 3.0 * N * K
        groups[inp] = {"M_cal": M, "N": N, "K": K, "sweep_ms": round(ms, 4),
                       "ms_per_alpha": round(ms / len(alphas), 4),
                       "best_alpha": alphas[ib], "rel_err_best": float(rel[ib]),
                       "rel_err_at_0.5": float(rel[alphas.index(0.5)]),
                       "fold_us": round(fold_ms * 1e3, 2),
                       "fold_gbs": round(fold_bytes / fold_ms / 1e6, 1)}
        total_ms += ms
        if best_fold is None or fold_bytes > best_fold[1]:
            best_fold = (fold_ms, fold_bytes, inp)
        del X, W, ws, Wq
        torch.cuda.empty_cache()
    fold_ms, fold_bytes, finp = best_fold
    evals = len(alphas) * len(wl.inputs)
    return {
        "row": "f4", "metric": "per-layer alpha sweep, layer-alpha evaluations per second",
        "value": round(evals / (total_ms * 1e-3), 1), "unit": "evaluations/s",
        "higher_is_better": True, "dtype": wl.dtype + "->int8", "data": "synthetic",
        "config": {"workload": wl.name, "alphas": len(alphas), "calibration_rows": 512,
                   "reps": reps},
        "sweep_ms_all_groups": round(total_ms, 3),
        "roofline": {"bound": "hbm", "kernel": f"k_quant (FOLD) on the {finp} weights",
                     "achieved": round(fold_bytes / fold_ms / 1e6, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(fold_bytes / fold_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_ms": round(fold_ms, 5),
                     "bytes_per_launch": fold_bytes},
        "groups": groups,
    }


def row_f2(args, torch):
    """Normalization with the folded 1/s fused with the quantizer, on the
    hidden-size inputs (the ones a norm precedes): Llama-3-8B (RMSNorm, bf16,
    M=2048, K=4096), OPT-13B prefill (LayerNorm, fp16, M=4096, K=5120),
    Llama-2-70B MLP (RMSNorm, bf16, M=8192, K=8192). Algorithmic bytes per
    element: the 16-bit residual read and the INT8 code written (3), the same
    as the quantizer alone; the unfused sequence (a norm kernel writing its
    16-bit output, then the quantizer) moves 7."""
    import w8a8_smoothquant_int8_amd as sq
    from synth.workloads import cast_to
    import numpy as np
    cases = [("llama3_8b_hidden", "rms", "bf16", 2048, 4096),
             ("opt13b_hidden", "layer", "f16", 4096, 5120),
             ("llama2_70b_hidden", "rms", "bf16", 8192, 8192)]
    reps = max(args.steps, 10)
    out, best = {}, None
    for name, kind, dt, M, K in cases:
        rng = np.random.default_rng(M + K)
        h = cast_to((rng.standard_normal((M, K)) * 2.0).astype(np.float32), dt).cuda()
        g = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32)).to(h.dtype).cuda()
        b = torch.zeros(K, dtype=h.dtype, device="cuda") if kind == "layer" else None
        s = torch.from_numpy(np.exp(rng.uniform(-1.5, 2.0, K)).astype(np.float32)).cuda()
        go = torch.empty(K, dtype=torch.float32, device="cuda")
        bo = torch.empty(K, dtype=torch.float32, device="cuda") if b is not None else None
        sq.sq_fold_norm_weight(g, b, s, go, bo)
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        a = torch.empty(M, dtype=torch.float32, device="cuda")
        fused = time_launches(torch, lambda: sq.sq_norm_quant(h, kind, go, bo, 1e-5, Xq, a), reps)
        quant = time_launches(torch, lambda: sq.sq_quant_per_token(h, s, Xq, a), reps)
        if kind == "rms":
            norm_fn = lambda: torch.nn.functional.rms_norm(h, (K,), g, eps=1e-5)
        else:
            norm_fn = lambda: torch.nn.functional.layer_norm(h, (K,), g, b, eps=1e-5)
        xn = norm_fn()
        unfused = time_launches(torch, lambda: (norm_fn(), sq.sq_quant_per_token(xn, s, Xq, a)), reps)
        nbytes = 3.0 * M * K
        out[name] = {"norm": kind, "dtype": dt, "M": M, "K": K,
                     "fused_us": round(fused * 1e3, 2), "fused_gbs": round(nbytes / fused / 1e6, 1),
                     "quant_alone_us": round(quant * 1e3, 2),
                     "unfused_torch_norm_plus_quant_us": round(unfused * 1e3, 2)}
        if best is None or nbytes > best[1]:
            best = (fused, nbytes, name)
        del h, Xq, xn
        torch.cuda.empty_cache()
    ms, nbytes, name = best
    return {
        "row": "f2", "metric": "fused norm + smoothing + per-token INT8 quant, GB/s",
        "value": round(nbytes / ms / 1e6, 1), "unit": "GB/s", "higher_is_better": True,
        "dtype": "bf16/f16->int8", "data": "synthetic",
        "config": {"workload": "hidden-size norm inputs", "reps": reps},
        "roofline": {"bound": "hbm", "kernel": f"k_norm_quant on {name}",
                     "achieved": round(nbytes / ms / 1e6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 5), "bytes_per_launch": nbytes},
        "cases": out,
    }


def row_f1(args, torch):
    """The quant and the LoRA shrink from one read of X (sq_quant_shrink) against
    the two separate calls (sq_quant_per_token, then sq_lora_shrink and its
    reduce), on the workload's input groups with their stacked adapters.
    Algorithmic bytes of the fused kernel: X read once (2 M K), codes written
    (M K), T written (2 M r); the separate calls read X twice."""
    from synth.workloads import get_workload
    import w8a8_smoothquant_int8_amd as sq
    wl = get_workload(args.workload)
    reps = max(args.steps, 10)
    out, best = {}, None
    for inp, K in wl.inputs:
        rows = wl.group_rows(inp)
        X = wl.x(inp).cuda()
        M = X.shape[0]
        A = torch.cat([wl.lora(p)[0] for p in rows], dim=0).contiguous().cuda()
        r = A.shape[0]
        s = torch.rand(K, device="cuda") + 0.5
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        a = torch.empty(M, dtype=torch.float32, device="cuda")
        T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
        sep = time_launches(torch, lambda: (sq.sq_quant_per_token(X, s, Xq, a),
                                            sq.sq_lora_shrink(X, A, T, ws)), reps)
        rec = {"K": K, "r": r, "separate_us": round(sep * 1e3, 2)}
        if K <= 8192:
            fused = time_launches(torch, lambda: sq.sq_quant_shrink(X, s, Xq, a, A, T), reps)
            nbytes = 3.0 * M * K + 2.0 * M * r
            rec.update(fused_us=round(fused * 1e3, 2), fused_gbs=round(nbytes / fused / 1e6, 1),
                       speedup=round(sep / fused, 3))
            if best is None or nbytes > best[1]:
                best = (fused, nbytes, inp)
        else:
            rec["fused_us"] = None        # K beyond the fused kernel's register budget
        out[inp] = rec
        del X, Xq, T, ws
        torch.cuda.empty_cache()
    ms, nbytes, inp = best
    return {
        "row": "f1", "metric": "per-token quant + LoRA shrink from one read of X, GB/s",
        "value": round(nbytes / ms / 1e6, 1), "unit": "GB/s", "higher_is_better": True,
        "dtype": wl.dtype + "->int8+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "reps": reps},
        "roofline": {"bound": "hbm", "kernel": f"k_quant_shrink on {inp}",
                     "achieved": round(nbytes / ms / 1e6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 5), "bytes_per_launch": nbytes},
        "groups": out,
    }


KERNEL_WORKLOADS = ("tiny_m16_k256_n256", "llama3_8b_proj_m2048", "opt13b_layer_decode_m64",
                    "opt13b_layer_prefill_m4096", "multitenant_lora_m8192", "llama2_70b_mlp_m8192")


def time_rotated(torch, fns, reps):
    """Average ms per call over reps calls cycling through fns (one per input
    copy), after one warm call each: with enough copies the inputs do not stay
    in the 256 MB MALL between their calls."""
    for f in fns:
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def row_kernels(args, torch):
    """Every kernel of the path (a1-a9), timed alone at every configuration's
    shapes: each input group's calibration absmax (a1), smoothing scale and
    fold (a2, a3: two passes over W), per-token quant (a4), INT8 GEMM with
    the dequant epilogue (a5, a6), stacked LoRA shrink with its reduce (a7),
    the same GEMM with the LoRA expand in its epilogue (a8), and the
    segmented LoRA (a9, shrink + expand). Inputs are seeded device-random
    tensors of the shapes; each kernel cycles through enough copies of its
    streamed input that the set exceeds 512 MB (at most 64 copies), so the
    MALL does not serve repeats. Memory-bound kernels report algorithmic GB/s
    and the fraction of 8 TB/s, the GEMMs TOP/s and the fraction of 5 POP/s."""
    from synth.workloads import get_workload
    import w8a8_smoothquant_int8_amd as sq
    torch.manual_seed(0)
    reps = max(args.steps, 20)
    dt_of = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    out, fracs = {}, []

    def copies(nbytes):
        return int(min(64, max(2, -(-(512 << 20) // max(nbytes, 1)))))

    def rec(ms, nbytes=None, ops=None, big=False):
        r = {"us": round(ms * 1e3, 2)}
        if nbytes is not None:
            gbs = nbytes / ms / 1e6
            r.update(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 3))
            if big:
                fracs.append(gbs / HBM_PEAK_GBS)
        if ops is not None:
            tops = ops / ms / 1e9
            r.update(tops=round(tops, 1), frac_int8=round(tops / INT8_PEAK_TOPS, 3))
        return r

    for name in KERNEL_WORKLOADS:
        wl = get_workload(name)
        dt, esz = dt_of[wl.dtype], (4 if wl.dtype == "f32" else 2)
        odt = dt_of[wl.out_dtype]
        M, C = wl.M, wl.calib_rows()
        big = M >= 4096
        res = {}
        for inp, K in wl.inputs:
            N = sum(p.N for p in wl.group(inp))
            g = {"M": M, "N": N, "K": K}
            Xs = [torch.randn(M, K, device="cuda").to(dt) for _ in range(copies(M * K * esz))]
            Xc = [x[:C] for x in Xs]
            amax = torch.zeros(K, device="cuda")
            ms = time_rotated(torch, [lambda x=x: sq.sq_calibrate_absmax(x, amax) for x in Xc], reps)
            g["a1_calibrate"] = rec(ms, esz * C * K, big=big)
            Ws = [(torch.randn(N, K, device="cuda") * 0.02).to(dt) for _ in range(copies(N * K * esz))]
            s = torch.empty(K, device="cuda")
            Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
            ws_ = torch.empty(N, device="cuda")
            amax.copy_(torch.rand(K, device="cuda") * 10 + 0.1)
            ms = time_rotated(torch, [lambda w=w: sq.sq_smooth_fold(amax, w, wl.alpha, s, Wq, ws_)
                                      for w in Ws], max(reps // 2, 10))
            g["a2_a3_smooth_fold"] = rec(ms, 2 * esz * N * K + N * K + 4 * N, big=big)
            del Ws
            Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
            a = torch.empty(M, device="cuda")
            ms = time_rotated(torch, [lambda x=x: sq.sq_quant_per_token(x, s, Xq, a) for x in Xs], reps)
            g["a4_quant"] = rec(ms, (esz + 1) * M * K + 4 * M, big=big)
            Wq.copy_(torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda"))
            Xq.copy_(torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda"))
            a.copy_(torch.rand(M, device="cuda") * 1e-2)
            ws_.copy_(torch.rand(N, device="cuda") * 1e-3)
            Y = torch.empty(M, N, dtype=odt, device="cuda")
            # decode-sized shapes split K across blocks with a workspace (0 bytes elsewhere)
            gws = sq.sq_w8a8_gemm_workspace_bytes(M, N, K)
            wsg = torch.empty(gws, dtype=torch.uint8, device="cuda") if gws else None
            ms = time_launches(torch, lambda: sq.sq_w8a8_gemm_ws(Xq, Wq, a, ws_, Y, wsg), reps)
            g["a5_a6_gemm"] = rec(ms, ops=2.0 * M * N * K)
            r = wl.lora_rank * len(wl.group(inp))
            if r:
                A = (torch.randn(r, K, device="cuda") * 0.01).bfloat16()
                Bb = (torch.randn(N, r, device="cuda") * 0.01).bfloat16()
                T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
                wsp = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
                ms = time_rotated(torch, [lambda x=x: sq.sq_lora_shrink(x, A, T, wsp) for x in Xs], reps)
                g["a7_shrink"] = rec(ms, esz * M * K + 2 * r * K + 2 * M * r, big=big)
                g["a7_shrink"]["rank"] = r
                ms = time_launches(torch, lambda: sq.sq_w8a8_gemm_lora(Xq, Wq, a, ws_, T, Bb, Y), reps)
                g["a8_gemm_lora"] = rec(ms, ops=2.0 * M * N * K)
            if wl.segmented:
                seg = wl.segments(0)
                ranks = seg["ranks"]
                for proj in [p.name for p in wl.group(inp)][:1]:
                    Np = [p.N for p in wl.group(inp) if p.name == proj][0]
                    As = [(torch.randn(int(rk), K, device="cuda") * 0.01).bfloat16() for rk in ranks]
                    Bs = [(torch.randn(Np, int(rk), device="cuda") * 0.01).bfloat16() for rk in ranks]
                    Yp = torch.zeros(M, Np, dtype=odt, device="cuda")
                    mr = int(ranks.max())
                    wsp = torch.empty(sq.sq_lora_workspace_bytes(M, K, mr), dtype=torch.uint8, device="cuda")
                    st_ = torch.from_numpy(seg["seg_start"]).cuda()
                    sa_ = torch.from_numpy(seg["seg_adapter"]).cuda()
                    rk_ = torch.from_numpy(ranks).cuda()
                    ap, bp = sq.pointer_table(As, "cuda"), sq.pointer_table(Bs, "cuda")
                    ms = time_rotated(torch, [lambda x=x: sq.sq_lora_apply_segmented(
                        x, st_, sa_, ap, bp, rk_, mr, Yp, wsp) for x in Xs], reps)
                    nbytes = esz * M * K + 2 * 2 * M * Np + sum(2 * int(rk) * (K + Np) for rk in ranks)
                    g["a9_segmented_" + proj] = rec(ms, nbytes, big=big)
            res[inp] = g
            del Xs, Xc, Xq, Y
            torch.cuda.empty_cache()
        out[name] = res
    fracs.sort()
    med = fracs[len(fracs) // 2] if fracs else None
    return {
        "row": "kernels", "metric": "per-kernel rates of the path at every configuration (median "
                                    "HBM fraction of the memory-bound kernels at M >= 4096)",
        "value": round(med, 3) if med is not None else None, "unit": "fraction of 8 TB/s",
        "higher_is_better": True, "data": "synthetic (device-random tensors of each configuration's shapes)",
        "config": {"workloads": list(KERNEL_WORKLOADS), "reps": reps}, "kernels": out,
    }


ROWS = {"f1": row_f1, "f2": row_f2, "f3": row_f3, "f4": row_f4, "kernels": row_kernels}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.row:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        print(json.dumps(ROWS[args.row](args, torch)))
        return
    from synth.workloads import get_workload
    import w8a8_smoothquant_int8_amd as sq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if not sq.sq_query_support(0):
        raise SystemExit("device 0 is not gfx950")
    wl = get_workload(args.workload)
    groups = setup(wl, torch)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    st = Streams(torch, groups)
    for _ in range(args.warmup):
        run_step_streams(groups, st, join=False)
    torch.cuda.synchronize()

    # The dominant kernel: the GEMM instantiation (tile configuration) with the
    # most GEMM work per step. Only its launches carry timing events (each
    # event pair costs some step time).
    cfg_ops = {}
    for inp, _K in wl.inputs:
        Ntot = sum(p.N for p in wl.group(inp))
        cfg = gemm_tile(wl.M, Ntot, wl.K_of(inp))
        cfg_ops[cfg] = cfg_ops.get(cfg, 0.0) + 2.0 * wl.M * Ntot * wl.K_of(inp)
    dom = max(cfg_ops, key=cfg_ops.get)
    dom_groups = {inp for inp, _K in wl.inputs
                  if gemm_tile(wl.M, sum(p.N for p in wl.group(inp)), wl.K_of(inp)) == dom}

    # Timed region: exactly `steps` steps, synchronized on both sides and
    # issued back to back (no join between steps; see run_step_streams). HIP
    # events on the dominant GEMM's stream time its launches for the roofline.
    gemm_ev = {"pool": event_pool(torch, args.steps * len(dom_groups)), "groups": dom_groups}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step_streams(groups, st, gemm_ev, join=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    ops = wl.gemm_ops()
    value = ops * args.steps / elapsed / 1e12
    gemm_ev.pop("pool")
    gemm_ev.pop("groups")
    gemm_by_group = {g: [a.elapsed_time(b) for a, b in evs] for g, evs in gemm_ev.items()}

    # Per-stage times: a few more steps, untimed, with every launch issued in
    # order on one stream and HIP events between the launches; the GEMMs there
    # run alone on the chip.
    stage_ms, gemm_alone = {}, {}
    if not args.no_stages:
        run_step(groups)                  # first use of the single-purpose calls, untimed
        torch.cuda.synchronize()
        tl = Timeline(torch)
        n_inst = min(args.steps, 5)
        for _ in range(n_inst):
            run_step(groups, tl)
        torch.cuda.synchronize()
        d, gemm_alone = tl.durations()
        stage_ms = {k: sum(v) / n_inst for k, v in d.items()}
    # The dominant kernel's timed launches
    kd = {"ms": [], "ops": 0.0, "launches": 0}
    for inp in sorted(dom_groups):
        Ntot = sum(p.N for p in wl.group(inp))
        kd["ms"] += gemm_by_group[inp]
        kd["ops"] += 2.0 * wl.M * Ntot * wl.K_of(inp) * len(gemm_by_group[inp])
        kd["launches"] += len(gemm_by_group[inp])
    gemm_avg_ms = sum(kd["ms"]) / kd["launches"]
    gemm_tops = (kd["ops"] / kd["launches"]) / (gemm_avg_ms * 1e-3) / 1e12
    traffic = stored_traffic(dom)
    # The same kernel's launches in the serialized pass, where nothing else runs
    alone_tops = None
    if gemm_alone:
        ms, ops = 0.0, 0.0
        for inp, _K in wl.inputs:
            Ntot = sum(p.N for p in wl.group(inp))
            if gemm_tile(wl.M, Ntot, wl.K_of(inp)) == dom:
                ms += sum(gemm_alone[inp])
                ops += 2.0 * wl.M * Ntot * wl.K_of(inp) * len(gemm_alone[inp])
        alone_tops = ops / (ms * 1e-3) / 1e12

    quant_bytes = sum((2 if wl.dtype != "f32" else 4) * wl.M * K + wl.M * K + 4 * wl.M
                      for _i, K in wl.inputs)
    line = {
        "metric": "W8A8 GEMM+LoRA INT8 TOPS and % of MI355X INT8 MFMA peak (1 GPU)",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "act_dtype": wl.dtype, "out_dtype": wl.out_dtype,
                   "alpha": wl.alpha, "lora_rank": wl.lora_rank,
                   "projections": {p.name: [p.N, wl.K_of(p.input)] for p in wl.projections},
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma",
                     "kernel": f"k_gemm_pipe {dom} tiles, LoRA epilogue" if any(
                         g.fused for _i, g, _x, _c in groups) else f"k_gemm_pipe {dom} tiles",
                     "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": traffic,
                     "launches_per_step": kd["launches"] // args.steps,
                     "avg_launch_ms": round(gemm_avg_ms, 5),
                     "note": "timed-region launches, which share the chip with the other "
                             "groups' kernels; achieved_alone: the same kernel with nothing "
                             "else running (serialized pass)",
                     "achieved_alone": round(alone_tops, 1) if alone_tops else None},
        "value_pct_of_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2),
    }
    if stage_ms:
        line["stages_ms_per_step_serialized"] = {k: round(v, 4) for k, v in stage_ms.items()}
        line["quant_gbs"] = round(quant_bytes / (stage_ms["quant"] * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_rows)
        cb.pop("step_s")
        cb["value"] = round(cb["value"], 6)
        line["cpu_baseline"] = cb
    print(json.dumps(line))


if __name__ == "__main__":
    main()
