"""Benchmark of the SmoothQuant W8A8 linear path (+ bf16 LoRA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of the workload, for
every input group: calibrate the per-channel maxima, compute the smoothing
vector and fold it into INT8 weights, quantize the activations per token,
run the INT8 GEMM with its dequant epilogue for every projection, and add the
bf16 LoRA delta (the stacked shrink, then the expand inside the GEMM
epilogue; per-request adapters as a segmented call). The default workload is
the Llama-2-70B MLP block at M=8192 tokens, the largest configuration that
fits one GPU. Inputs are seeded synthetic tensors, resident in HBM before the
timed region starts.

Each input group runs as one native call (sq_linear_group_run), which records
HIP events between its launches on its stream. By default every group runs on
one stream, in order of decreasing GEMM work, so each kernel has the chip to
itself and the events time it alone; --streams N spreads the groups over N
streams instead (their kernels then overlap).

Output: one JSON line. `value` is the GEMM+LoRA effective INT8 rate:
2*M*N*K summed over the projections, divided by the summed time of the GEMMs
(dequant and LoRA expand in their epilogue), the LoRA shrinks and any
segmented LoRA calls, all measured with HIP events inside the timed steps.
`full_step_tops` divides the same operations by the wall-clock step time,
which also holds the calibration, the fold and the activation quant.
`roofline` is the dominant GEMM kernel against the MI355X dense INT8 MFMA
peak. The CPU oracle is timed stage by stage on a bounded sample of the same
step (cpu_baseline).
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
DEFAULT_WORKLOAD = "llama2_70b_mlp_m8192"
GEMM_KERNEL_SRC = os.path.join(ROOT, "w8a8_smoothquant_int8_amd", "csrc", "k_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_{tile}_hbm_traffic_{workload}.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--streams", type=int, default=1,
                    help="streams the input groups are spread over (1: in order on one stream)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="activation rows per input in the CPU-oracle sample")
    ap.add_argument("--cpu-wrows", type=int, default=1024,
                    help="weight rows (output columns) per input in the CPU-oracle sample")
    ap.add_argument("--row", choices=sorted(ROWS), default=None,
                    help="measure one of the widened rows instead of the whole step "
                         "(one JSON line of its own)")
    ap.add_argument("--kernel-workloads", default=None,
                    help="with --row kernels: a comma-separated subset of the configurations "
                         "(default: all of them)")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="print the CPU-oracle baseline of --workload as JSON and exit (no GPU; "
                         "bench.py runs this in a child process of its own)")
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


def stored_traffic(tile: str, workload: str):
    """HBM bytes per launch of the dominant GEMM kernel from the rocprofv3
    FETCH_SIZE/WRITE_SIZE runs on this workload, if they were taken on the
    current GEMM source."""
    path = TRAFFIC_FILE.format(tile=tile, workload=workload)
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


def segmented_lora(wl, proj, torch, seed=0):
    """The per-request adapters of a multi-tenant workload for one projection."""
    import w8a8_smoothquant_int8_amd as sq
    from w8a8_smoothquant_int8_amd.pipeline import SegmentedLora
    seg = wl.segments(seed)
    ranks = seg["ranks"]
    As, Bs = [], []
    for ad, r in enumerate(ranks):
        a, b = wl.lora(proj, rank=int(r), adapter=ad, seed=seed)
        As.append(a.cuda())
        Bs.append(b.cuda())
    return SegmentedLora(
        seg_start=torch.from_numpy(seg["seg_start"]).cuda(),
        seg_adapter=torch.from_numpy(seg["seg_adapter"]).cuda(),
        A=As, B=Bs, ranks=torch.from_numpy(ranks).cuda(),
        A_ptrs=sq.pointer_table(As, "cuda"), B_ptrs=sq.pointer_table(Bs, "cuda"),
        max_rank=int(ranks.max()))


def setup(wl, torch):
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    groups = []
    for inp, _K in wl.inputs:
        rows = wl.group_rows(inp)
        loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows} if wl.lora_rank else {}
        segs = {p: segmented_lora(wl, p, torch) for p in rows} if wl.segmented else {}
        g = LinearGroup(wl.w_group(inp).cuda(), rows, wl.alpha, wl.out_dtype, wl.M, lora=loras,
                        seg_lora=segs)
        groups.append((inp, g, wl.x(inp).cuda(), wl.x_cal(inp).cuda()))
    torch.cuda.synchronize()
    return groups


class Streams:
    """The step's streams (default priority) and the group -> stream plan:
    groups in descending order of GEMM work, each on the stream with the least
    work so far (longest-processing-time first)."""

    def __init__(self, torch, groups, n_streams):
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


STAGE_EVENTS = ("begin", "quant_begin", "shrink_begin", "gemm_begin", "gemm_end")


def run_step_streams(groups, st, rec=None, join=True):
    """One pass of the whole path over one batch: each input group runs
    calibrate -> fold -> quantize -> LoRA shrink -> GEMM (LoRA expand in its
    epilogue) as one native call, plus its segmented LoRA calls, on the stream
    the plan gives it. rec: None, or a recorder whose take(group) gives the
    HIP events the library records between that group's launches.

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
        ev, seg_ev = rec.take(inp) if rec is not None else (None, None)
        g.run(X, Xc, stream=st.main[si], events=ev, seg_events=seg_ev)
    if join:
        for sm in st.main:
            cur.wait_stream(sm)


class StageRecorder:
    """Pre-created HIP event sets, one per (step, group): the group call's
    stage events and a pair around its segmented LoRA calls."""

    def __init__(self, torch, groups, steps):
        import w8a8_smoothquant_int8_amd as sq
        self.sq = sq
        self.sets = {inp: [] for inp, _g, _x, _c in groups}
        self.seg = {inp: bool(g.seg_lora) for inp, g, _x, _c in groups}
        for inp in self.sets:
            for _ in range(steps):
                evs = {k: torch.cuda.Event(enable_timing=True) for k in STAGE_EVENTS}
                pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for e in list(evs.values()) + list(pair):
                    e.record()          # the first record creates the HIP event
                self.sets[inp].append((evs, pair))
        torch.cuda.synchronize()
        self.used = {inp: [] for inp in self.sets}

    def take(self, inp):
        evs, pair = self.sets[inp][len(self.used[inp])]
        self.used[inp].append((evs, pair))
        return self.sq.sq_group_events(**evs), (pair if self.seg[inp] else None)

    def stage_ms(self, inp, has_lora):
        """Per-step average ms of each stage of a group's call."""
        out = {"calibrate_fold": 0.0, "quant": 0.0, "shrink": 0.0, "gemm": 0.0, "seg_lora": 0.0,
               "gemm_launches": []}
        for evs, pair in self.used[inp]:
            out["calibrate_fold"] += evs["begin"].elapsed_time(evs["quant_begin"])
            nxt = evs["shrink_begin"] if has_lora else evs["gemm_begin"]
            out["quant"] += evs["quant_begin"].elapsed_time(nxt)
            if has_lora:
                out["shrink"] += evs["shrink_begin"].elapsed_time(evs["gemm_begin"])
            g = evs["gemm_begin"].elapsed_time(evs["gemm_end"])
            out["gemm"] += g
            out["gemm_launches"].append(g)
            if self.seg[inp]:
                out["seg_lora"] += pair[0].elapsed_time(pair[1])
        n = max(len(self.used[inp]), 1)
        for k in ("calibrate_fold", "quant", "shrink", "gemm", "seg_lora"):
            out[k] /= n
        return out


def _tile_score(M, N, bm, bn, resident, rate):
    tm, tn = -(-M // bm), -(-N // bn)
    tiles = tm * tn
    rounds = -(-tiles // resident)
    pad = (M / (tm * bm)) * (N / (tn * bn))
    return rate * pad * tiles / (rounds * resident)


def gemm_tile(M: int, N: int, K: int, lora: bool = False) -> str:
    """The tile configuration libsq picks for an INT8 GEMM of this shape (the
    library's rule: the generic kernel when K is not a multiple of 128 or an
    operand reaches 4 GiB, the decode kernel for M <= 64 without a LoRA
    epilogue (128-column blocks where 64-column ones would outnumber 256 CUs),
    the skinny kernel for M <= 64 with one and fewer than 96
    column tiles of 128, else the best of
    256x256 tiles and 256x192 tiles,
    one block per CU, at rates 1 and 0.93, and 128x128 tiles, two blocks per
    CU, at 0.8, each scored by the padding and the fraction of the last round
    of blocks that does useful work; ties go to 256x256, then 256x192)."""
    if K % 128 or M * K >= 1 << 32 or N * K >= 1 << 32:
        return "generic"
    if M <= 64 and not lora:
        return "decode" if (N + 63) // 64 <= 256 else "decode128"
    if M <= 64 and (N + 127) // 128 < 96:
        return "skinny"
    s256 = _tile_score(M, N, 256, 256, 256, 1.0)
    s192 = _tile_score(M, N, 256, 192, 256, 0.93)
    s128 = _tile_score(M, N, 128, 128, 512, 0.8)
    if s256 >= s192 and s256 >= s128:
        return "256x256"
    return "256x192" if s192 >= s128 else "128x128"


def tile_dims(tile: str):
    """(rows, columns) of one output tile of a configuration."""
    return {"256x256": (256, 256), "256x192": (256, 192), "128x128": (128, 128),
            "generic": (128, 128), "skinny": (64, 32), "decode": (64, 64),
            "decode128": (64, 128)}[tile]


def host_info():
    """nproc and the CPU model of this host."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return nproc, model


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([d.get("num_threads", 1) for d in threadpool_info()
                if d.get("user_api") == "blas"] or [1])


def cpu_baseline(wl, rows_per_input: int, wrows_per_input: int):
    """The oracle as it stands, timed stage by stage on a bounded sample of one
    step, each stage scaled to the whole workload by its own size:
    calibration absmax over the full calibration batch; weight absmax and the
    fold + weight quant on `wrows_per_input` weight rows (scaled by N / rows);
    the smoothing vector in full; per-token quant on `rows_per_input`
    activation rows (scaled by M / rows); the INT8 GEMM + dequant on those
    rows against the sampled weight rows (scaled by M N / (rows wrows)); the
    LoRA shrink on the sampled rows (scaled by M / rows) and the expand on
    the sampled rows and columns (scaled like the GEMM); segmented adapters
    likewise on the sampled rows' requests."""
    import numpy as np
    import oracle.sq_oracle as O

    st = {k: 0.0 for k in ("calibrate", "weight_absmax", "smoothing_scale", "fold_quant",
                           "quant", "gemm_dequant", "lora_shrink", "lora_expand")}
    m = min(rows_per_input, wl.M)
    for inp, K in wl.inputs:
        X = wl.x(inp).float().numpy()[:m]
        Xc = wl.x_cal(inp).float().numpy()
        W = wl.w_group(inp).float().numpy()
        N = W.shape[0]
        n = min(wrows_per_input, N)
        cols = np.linspace(0, N - 1, n).astype(np.int64)
        Ws = np.ascontiguousarray(W[cols])
        del W
        t = time.perf_counter
        t0 = t(); act_max = O.calibrate_absmax(Xc); st["calibrate"] += t() - t0
        t0 = t(); w_max = O.weight_absmax(Ws); st["weight_absmax"] += (t() - t0) * N / n
        t0 = t(); s = O.smoothing_scale(act_max, w_max, wl.alpha); st["smoothing_scale"] += t() - t0
        t0 = t(); wq, wsc = O.fold_and_quantize_weights(Ws, s); st["fold_quant"] += (t() - t0) * N / n
        t0 = t(); xq, a = O.quantize_per_token(X, s); st["quant"] += (t() - t0) * wl.M / m
        # one untimed call first: the first product of this size in a process
        # pays the kernel's page faults on its fresh float64 operands (5-8x)
        O.dequantize(O.int8_gemm(xq, wq), a, wsc, wl.out_dtype)
        t0 = t()
        y = O.dequantize(O.int8_gemm(xq, wq), a, wsc, wl.out_dtype)
        st["gemm_dequant"] += (t() - t0) * (wl.M / m) * (N / n)
        if wl.lora_rank:
            # the group's adapters stacked along r, as the GPU path runs them
            rows = wl.group_rows(inp)
            A = np.concatenate([wl.lora(p)[0].float().numpy() for p in rows], axis=0)
            B = np.zeros((n, A.shape[0]), dtype=np.float32)
            c = 0
            for p, (r0, r1) in rows.items():
                Bp = wl.lora(p)[1].float().numpy()
                sel = (cols >= r0) & (cols < r1)
                B[sel, c:c + wl.lora_rank] = Bp[cols[sel] - r0]
                c += wl.lora_rank
            t0 = t(); T = O.lora_shrink(X, wl.dtype, A); st["lora_shrink"] += (t() - t0) * wl.M / m
            t0 = t(); O.lora_expand_add(y, T, B, 1.0, wl.out_dtype)
            st["lora_expand"] += (t() - t0) * (wl.M / m) * (N / n)
        elif wl.segmented:
            seg = wl.segments(0)
            ranks = seg["ranks"]
            for p, (r0, r1) in wl.group_rows(inp).items():
                As, Bs = [], []
                for ad, rk in enumerate(ranks):
                    a_, b_ = wl.lora(p, rank=int(rk), adapter=ad)
                    As.append(a_.float().numpy())
                    Bs.append(b_.float().numpy())
                sel = (cols >= r0) & (cols < r1)
                if not sel.any():
                    continue
                Bsel = [b[cols[sel] - r0] for b in Bs]
                t0 = t()
                O.lora_apply_segmented(y[:, sel], X, wl.dtype, np.minimum(seg["seg_start"], m),
                                       seg["seg_adapter"], As, Bsel, 1.0, wl.out_dtype)
                # shrink and expand together; scaled like the expand (rows x columns)
                st["lora_expand"] += (t() - t0) * (wl.M / m) * ((r1 - r0) / sel.sum())
    ops = wl.gemm_ops()
    gemm_lora_s = st["gemm_dequant"] + st["lora_shrink"] + st["lora_expand"]
    full_s = sum(st.values())
    nproc, model = host_info()
    thr = blas_threads()
    return {
        "value": ops / gemm_lora_s / 1e12,
        "unit": "TOPS",
        "cores": int(thr),
        "kind": "oracle",
        "sample": (f"one step of {wl.name}, stage by stage: calibration batch in full; "
                   f"{n} weight rows and {m} activation rows per input, each stage's time "
                   f"scaled to the full sizes; value = GEMM+LoRA ops over the GEMM + dequant + "
                   f"LoRA time, as for the GPU; numpy oracle, BLAS threads={thr}"),
        "nproc": nproc,
        "cpu_model": model,
        "stages_s": {k: round(v, 4) for k, v in st.items()},
        "full_step_s": round(full_s, 3),
        "full_step_tops": ops / full_s / 1e12,
    }


_SLEEP_PER_S = None


def gpu_head_start(torch, seconds: float) -> None:
    """Keep the current stream busy for about `seconds` (a spin kernel), so that
    the launches enqueued next are all queued before the first of them runs:
    they then run back to back, and HIP events around them time the GPU work
    alone, not the host's launch overhead (two Python binding calls can take
    longer to issue than small kernels take to run)."""
    global _SLEEP_PER_S
    if seconds <= 0:
        return
    if _SLEEP_PER_S is None:                     # spin cycles per second, measured once
        n = 1 << 20
        torch.cuda._sleep(n)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_PER_S = n / max(e0.elapsed_time(e1) / 1e3, 1e-6)
    torch.cuda._sleep(int(min(seconds, 0.5) * _SLEEP_PER_S))


def time_calls(torch, fns, reps: int) -> float:
    """Average ms per call over reps calls cycling through fns, after one warm
    call each, timed with HIP events around GPU work that runs back to back
    (gpu_head_start covers three times the host time the warm calls took to
    issue, plus 0.2 ms)."""
    t0 = time.perf_counter()
    for f in fns:
        f()
    host = (time.perf_counter() - t0) / len(fns)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_head_start(torch, 3.0 * host * reps + 2e-4)
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_launches(torch, fn, reps: int, warm: int = 3) -> float:
    """Average ms of fn() over reps launches on the current stream (HIP events,
    back to back: see time_calls)."""
    for _ in range(warm - 1):
        fn()
    return time_calls(torch, [fn], reps)


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


def mfma_probe(torch, mode: int, blocks: int = 256, iters: int = 4000, reps: int = 3):
    """Run the INT8 MFMA-only probe (libsq_probe): returns (TOP/s, mean shader
    clock in GHz over the blocks' timed loops), the best of `reps` runs."""
    import ctypes
    path = os.path.join(ROOT, "w8a8_smoothquant_int8_amd", "libsq_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with python -m w8a8_smoothquant_int8_amd.build")
    L = ctypes.CDLL(path)
    L.sq_probe_mfma_i8.restype = ctypes.c_int
    L.sq_probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    g = torch.Generator(device="cuda").manual_seed(1234)
    rnd = torch.randint(-2 ** 31, 2 ** 31 - 1, (blocks * 512 * 64,), dtype=torch.int32,
                        device="cuda", generator=g)
    clk = torch.zeros(blocks, 2, dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    best = None
    for _ in range(reps + 1):                  # the first run warms up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.sq_probe_mfma_i8(mode, blocks, iters, rnd.data_ptr(), clk.data_ptr(),
                                sink.data_ptr(), ctypes.c_void_p(st.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0, rc
        ms = e0.elapsed_time(e1)
        c = clk.cpu().double()
        ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1        # reference clock: 100 MHz
        tops = blocks * 8 * iters * 64 * 65536.0 / (ms * 1e-3) / 1e12
        if best is None or tops > best[0]:
            best = (tops, ghz)
    return best


def row_mfma(args, torch):
    """The practical INT8 matrix-core ceiling: the MFMA-only probe at the
    GEMM's occupancy with constant and with random operands, and the shader
    clock each sustains."""
    const_tops, const_ghz = mfma_probe(torch, 0)
    rand_tops, rand_ghz = mfma_probe(torch, 1)
    per_clk = lambda tops, ghz: tops / (INT8_PEAK_TOPS * ghz / 2.4)
    return {
        "row": "mfma", "metric": "INT8 MFMA-only rate (probe at the GEMM's occupancy)",
        "value": round(rand_tops, 1), "unit": "TOPS", "higher_is_better": True, "dtype": "int8",
        "data": "random operand fragments held in registers",
        "config": {"blocks": 256, "waves_per_block": 8, "mfma": "V_MFMA_I32_32X32X32_I8",
                   "accumulators_per_wave": 8},
        "random_operands": {"tops": round(rand_tops, 1), "shader_clock_ghz": round(rand_ghz, 3),
                            "frac_of_peak": round(rand_tops / INT8_PEAK_TOPS, 4),
                            "frac_of_rate_at_clock": round(per_clk(rand_tops, rand_ghz), 4)},
        "constant_operands": {"tops": round(const_tops, 1), "shader_clock_ghz": round(const_ghz, 3),
                              "frac_of_peak": round(const_tops / INT8_PEAK_TOPS, 4),
                              "frac_of_rate_at_clock": round(per_clk(const_tops, const_ghz), 4)},
        "peak_note": "5.0 POP/s = 256 CUs x 4 SIMDs x 2048 int8 ops/clock x 2.4 GHz",
    }


def row_lora_window(args, torch):
    """The GEMM with the stacked-LoRA epilogue, with and without the
    per-projection rank windows, and without LoRA, on the same group (the
    workload's data), timed by the group call's own events around the GEMM,
    alternating the three settings."""
    from synth.workloads import get_workload
    import w8a8_smoothquant_int8_amd as sq
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    cases = [("llama2_70b_mlp_m8192", "mlp_in"), ("llama3_8b_proj_m2048", "attn_in"),
             ("llama3_8b_proj_m2048", "mlp_in")]
    reps = max(min(args.steps, 20), 5)
    out = {}
    for name, inp in cases:
        wl = get_workload(name)
        rows = wl.group_rows(inp)
        W = wl.w_group(inp).cuda()
        X, Xc = wl.x(inp).cuda(), wl.x_cal(inp).cuda()
        loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows}
        g = LinearGroup(W, rows, wl.alpha, wl.out_dtype, wl.M, lora=loras)
        g0 = LinearGroup(W, rows, wl.alpha, wl.out_dtype, wl.M)
        g.run(X, Xc)
        g0.run(X, Xc)
        table = g.lora_parts
        settings = {"windows": (g, table), "full_rank": (g, None), "no_lora": (g0, None)}
        ms = {k: [] for k in settings}
        for _ in range(reps):
            for k, (grp, parts) in settings.items():
                if grp is g:
                    grp.lora_parts = parts
                    grp._desc_key = None            # rebuild the call's descriptor
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                e1.record()
                grp.run(X, Xc, sq.SQ_GROUP_FORWARD,
                        events=sq.sq_group_events(gemm_begin=e0, gemm_end=e1))
                torch.cuda.synchronize()
                ms[k].append(e0.elapsed_time(e1))
        g.lora_parts = table
        med = {k: sorted(v)[len(v) // 2] for k, v in ms.items()}
        out[f"{name}/{inp}"] = {
            "M": wl.M, "N": g.Ntot, "K": g.K, "stacked_rank": g.A_stack.shape[0],
            "parts": table, "gemm_us": {k: round(v * 1e3, 1) for k, v in med.items()},
            "lora_epilogue_us": {"windows": round((med["windows"] - med["no_lora"]) * 1e3, 1),
                                 "full_rank": round((med["full_rank"] - med["no_lora"]) * 1e3, 1)}}
        del g, g0, W, X, Xc
        torch.cuda.empty_cache()
    first = out[f"{cases[0][0]}/{cases[0][1]}"]
    return {"row": "lora_window", "metric": "GEMM time with the stacked LoRA epilogue, "
            "per-projection rank windows vs the full stacked rank (median of alternated launches)",
            "value": first["lora_epilogue_us"]["windows"], "unit": "us of LoRA epilogue",
            "higher_is_better": False, "data": "synthetic (the workloads' tensors)",
            "config": {"reps": reps}, "cases": out}


def row_oracle(args, torch):
    """The CPU oracle, stage by stage, on every configuration (the bounded
    sample of cpu_baseline), and once more on a single core for the
    Llama-3-8B projections. No GPU work."""
    from threadpoolctl import threadpool_limits
    from synth.workloads import get_workload
    out = {}
    for name in KERNEL_WORKLOADS:
        cb = cpu_baseline(get_workload(name), args.cpu_rows, args.cpu_wrows)
        out[name] = {k: cb[k] for k in ("value", "stages_s", "full_step_s", "full_step_tops",
                                        "cores")}
        print(f"oracle {name}: {cb['value']:.4g} TOPS, full step {cb['full_step_s']:.1f} s",
              file=sys.stderr, flush=True)
    with threadpool_limits(limits=1):
        cb1 = cpu_baseline(get_workload("llama3_8b_proj_m2048"), args.cpu_rows, args.cpu_wrows)
    nproc, model = host_info()
    return {"row": "oracle", "metric": "CPU oracle GEMM+LoRA TOPS per configuration",
            "value": out[DEFAULT_WORKLOAD]["value"], "unit": "TOPS", "higher_is_better": True,
            "data": "synthetic", "nproc": nproc, "cpu_model": model,
            "sample": f"{args.cpu_rows} activation rows and {args.cpu_wrows} weight rows per input, "
                      "each stage scaled to the full sizes",
            "configs": out,
            "one_core_llama3_8b_proj_m2048": {k: cb1[k] for k in ("value", "stages_s",
                                                                  "full_step_s", "cores")}}


def row_vendor(args, torch):
    """The INT8 GEMM of this library against the vendor library's (torch._int_mm,
    which runs hipBLASLt on ROCm: int32 output, no epilogue) on the Llama-2-70B
    MLP shapes, seeded uniform int8 operands; this library's int32 entry point
    is checked bit for bit against it. Context for the GEMM's rate, not a
    stage of the path."""
    import w8a8_smoothquant_int8_amd as sq
    torch.manual_seed(0)
    reps = max(args.steps, 10)

    def timed(f):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    for (M, N, K) in [(8192, 57344, 8192), (8192, 8192, 28672), (8192, 28672, 8192)]:
        X = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        W = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda")
        a = torch.rand(M, device="cuda") * 1e-3
        w = torch.rand(N, device="cuda") * 1e-3
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ops = 2.0 * M * N * K
        rec = {}
        ms = timed(lambda: torch._int_mm(X, W.t()))
        rec["vendor_int32_tops"] = round(ops / ms / 1e9, 1)
        ms = timed(lambda: sq.sq_w8a8_gemm(X, W, a, w, Y))
        rec["sq_bf16_tops"] = round(ops / ms / 1e9, 1)
        if M * N <= 8192 * 28672:
            acc = torch.empty(M, N, dtype=torch.int32, device="cuda")
            ms = timed(lambda: sq.sq_w8a8_gemm_i32(X, W, acc))
            rec["sq_int32_tops"] = round(ops / ms / 1e9, 1)
            rec["int32_equal"] = bool(torch.equal(acc, torch._int_mm(X, W.t())))
            del acc
        out[f"{M}x{N}x{K}"] = rec
        print(f"vendor {M}x{N}x{K}: {rec}", file=sys.stderr, flush=True)
        del X, W, Y
        torch.cuda.empty_cache()
    return {"row": "vendor", "metric": "INT8 GEMM TOPS, this library against torch._int_mm (hipBLASLt)",
            "value": out["8192x57344x8192"]["sq_bf16_tops"], "unit": "TOPS", "higher_is_better": True,
            "data": "seeded uniform int8 operands", "shapes": out}


KERNEL_WORKLOADS = ("tiny_m16_k256_n256", "llama3_8b_proj_m2048", "opt13b_layer_decode_m64",
                    "opt13b_layer_prefill_m4096", "multitenant_lora_m8192", "llama2_70b_mlp_m8192")


def time_rotated(torch, fns, reps):
    """Average ms per call over reps calls cycling through fns (one per input
    copy), after one warm call each: with enough copies the inputs do not stay
    in the 256 MB MALL between their calls (back to back: see time_calls)."""
    return time_calls(torch, fns, reps)


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

    names = KERNEL_WORKLOADS
    if args.kernel_workloads:
        names = tuple(args.kernel_workloads.split(","))
        unknown = [n for n in names if n not in KERNEL_WORKLOADS]
        if unknown:
            raise SystemExit(f"--kernel-workloads: unknown {unknown}; choose from {KERNEL_WORKLOADS}")
    for name in names:
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
            del Wq
            # the GEMMs cycle through enough weight copies that the MALL does not serve repeats
            Wqs = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda")
                   for _ in range(copies(N * K))]
            Xq.copy_(torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda"))
            a.copy_(torch.rand(M, device="cuda") * 1e-2)
            ws_.copy_(torch.rand(N, device="cuda") * 1e-3)
            Y = torch.empty(M, N, dtype=odt, device="cuda")
            ms = time_rotated(torch, [lambda w=w: sq.sq_w8a8_gemm(Xq, w, a, ws_, Y) for w in Wqs], reps)
            g["a5_a6_gemm"] = rec(ms, ops=2.0 * M * N * K)
            g["a5_a6_gemm"]["weight_gbs"] = round(N * K / ms / 1e6, 1)
            # decode-sized shapes can split K across blocks with a workspace (0 bytes elsewhere)
            gws = sq.sq_w8a8_gemm_workspace_bytes(M, N, K)
            if gws:
                wsg = torch.empty(gws, dtype=torch.uint8, device="cuda")
                ms = time_rotated(torch, [lambda w=w: sq.sq_w8a8_gemm_ws(Xq, w, a, ws_, Y, wsg)
                                          for w in Wqs], reps)
                g["a5_a6_gemm_split_k"] = rec(ms, ops=2.0 * M * N * K)
                g["a5_a6_gemm_split_k"]["weight_gbs"] = round(N * K / ms / 1e6, 1)
            r = wl.lora_rank * len(wl.group(inp))
            if r:
                A = (torch.randn(r, K, device="cuda") * 0.01).bfloat16()
                Bb = (torch.randn(N, r, device="cuda") * 0.01).bfloat16()
                T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
                wsp = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
                ms = time_rotated(torch, [lambda x=x: sq.sq_lora_shrink(x, A, T, wsp) for x in Xs], reps)
                g["a7_shrink"] = rec(ms, esz * M * K + 2 * r * K + 2 * M * r, big=big)
                g["a7_shrink"]["rank"] = r
                ms = time_rotated(torch, [lambda w=w: sq.sq_w8a8_gemm_lora(Xq, w, a, ws_, T, Bb, Y)
                                          for w in Wqs], reps)
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
            del Xs, Xc, Xq, Y, Wqs
            torch.cuda.empty_cache()
        out[name] = res
    fracs.sort()
    med = fracs[len(fracs) // 2] if fracs else None
    return {
        "row": "kernels", "metric": "per-kernel rates of the path at every configuration (median "
                                    "HBM fraction of the memory-bound kernels at M >= 4096)",
        "value": round(med, 3) if med is not None else None, "unit": "fraction of 8 TB/s",
        "higher_is_better": True, "data": "synthetic (device-random tensors of each configuration's shapes)",
        "config": {"workloads": list(names), "reps": reps}, "kernels": out,
    }


ROWS = {"f1": row_f1, "f2": row_f2, "f3": row_f3, "f4": row_f4, "kernels": row_kernels,
        "mfma": row_mfma, "lora_window": row_lora_window, "oracle": row_oracle,
        "vendor": row_vendor}


def copy_calibration(args, torch):
    """With --copy-calibration-mib: one device copy of that many MiB, whose
    FETCH_SIZE / WRITE_SIZE counters (known bytes each way) scale the other
    dispatches' counters to bytes."""
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.cpu_baseline_only:
        from synth.workloads import get_workload
        print(json.dumps(cpu_baseline(get_workload(args.workload), args.cpu_rows, args.cpu_wrows)))
        return
    # The oracle baseline runs first, in a child process that never touches
    # the GPU: in a process whose GPU runtime is up, the oracle's BLAS threads
    # share the host cores with the runtime's own threads and ran 10-13x slower.
    cb = None
    if not args.no_cpu_baseline and not args.row:
        import subprocess
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                            "--workload", args.workload, "--cpu-rows", str(args.cpu_rows),
                            "--cpu-wrows", str(args.cpu_wrows)],
                           capture_output=True, text=True, timeout=1800)
        if r.returncode != 0:
            raise SystemExit(f"CPU baseline child failed ({r.returncode}):\n{r.stderr[-2000:]}")
        cb = json.loads(r.stdout.strip().splitlines()[-1])
        print(f"cpu baseline done: {cb['value']:.4g} TOPS", file=sys.stderr, flush=True)
    import torch
    if args.row == "oracle":
        print(json.dumps(ROWS[args.row](args, torch)))
        return
    if args.row:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        copy_calibration(args, torch)
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
    copy_calibration(args, torch)
    st = Streams(torch, groups, max(1, args.streams))
    for _ in range(args.warmup):
        run_step_streams(groups, st, join=False)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, synchronized on both sides and
    # issued back to back. Every group call records its stage events.
    rec = StageRecorder(torch, groups, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step_streams(groups, st, rec, join=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    ops = wl.gemm_ops()

    # Per group (one GEMM launch over the stacked projections) and per projection.
    per_group, per_proj, tile_of = {}, {}, {}
    tot = {"calibrate_fold": 0.0, "quant": 0.0, "shrink": 0.0, "gemm": 0.0, "seg_lora": 0.0}
    for inp, g, _x, _c in groups:
        K = wl.K_of(inp)
        d = rec.stage_ms(inp, g.fused)
        g_ops = 2.0 * wl.M * g.Ntot * K
        lora_ms = d["shrink"] + d["seg_lora"]
        tile_of[inp] = gemm_tile(wl.M, g.Ntot, K, lora=g.fused)
        per_group[inp] = {
            "projections": list(g.rows), "M": wl.M, "N": g.Ntot, "K": K, "tile": tile_of[inp],
            "lora_rank": (g.A_stack.shape[0] if g.fused else
                          (max(s.max_rank for s in g.seg_lora.values()) if g.seg_lora else 0)),
            "ms": {k: round(v, 5) for k, v in d.items() if k != "gemm_launches"},
            "gemm_tops": round(g_ops / d["gemm"] / 1e9, 1),
            "gemm_lora_tops": round(g_ops / (d["gemm"] + lora_ms) / 1e9, 1)}
        for p, (r0, r1) in g.rows.items():
            per_proj[p] = {"input": inp, "M": wl.M, "N": r1 - r0, "K": K,
                           "gemm_tops": per_group[inp]["gemm_tops"],
                           "gemm_lora_tops": per_group[inp]["gemm_lora_tops"]}
        for k in tot:
            tot[k] += d[k]
    gemm_lora_ms = tot["gemm"] + tot["shrink"] + tot["seg_lora"]
    value = ops / (gemm_lora_ms * 1e-3) / 1e12

    # The dominant kernel: the GEMM instantiation (tile configuration) with the
    # most GEMM work per step; its launches in the timed region.
    cfg_ops = {}
    for inp, g, _x, _c in groups:
        cfg_ops[tile_of[inp]] = cfg_ops.get(tile_of[inp], 0.0) + 2.0 * wl.M * g.Ntot * g.K
    dom = max(cfg_ops, key=cfg_ops.get)
    launches, dom_ms, dom_ops = 0, 0.0, 0.0
    dom_inputs = []
    for inp, g, _x, _c in groups:
        if tile_of[inp] != dom:
            continue
        dom_inputs.append(inp)
        ls = rec.stage_ms(inp, g.fused)["gemm_launches"]
        launches += len(ls)
        dom_ms += sum(ls)
        dom_ops += 2.0 * wl.M * g.Ntot * g.K * len(ls)
    avg_launch_ms = dom_ms / launches
    achieved = dom_ops / launches / (avg_launch_ms * 1e-3) / 1e12
    traffic = stored_traffic(dom, wl.name)
    lora_epi = any(groups[i][1].fused for i in range(len(groups)) if groups[i][0] in dom_inputs)

    # The measured matrix-core ceiling beside the paper peak: the MFMA-only
    # probe with random operands, run after the timed region.
    probe_tops, probe_ghz = mfma_probe(torch, 1)

    esz = 4 if wl.dtype == "f32" else 2
    quant_bytes = sum((esz + 1) * wl.M * K + 4 * wl.M for _i, K in wl.inputs)
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
                   "streams": len(st.main), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma",
                     "kernel": f"k_gemm_pipe {dom} tiles" + (", LoRA epilogue" if lora_epi else "")
                               + f" ({', '.join(dom_inputs)})",
                     "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic,
                     "launches_per_step": launches // args.steps,
                     "ops_per_launch": dom_ops / launches,
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "mfma_probe_tops": round(probe_tops, 1),
                     "mfma_probe_clock_ghz": round(probe_ghz, 3),
                     "frac_of_mfma_probe": round(achieved / probe_tops, 4)},
        "value_formula": "sum 2MNK / sum (t_gemm incl. dequant and LoRA expand epilogue + "
                         "t_lora_shrink + t_segmented_lora), HIP events in the timed steps",
        "value_pct_of_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2),
        "full_step_tops": round(ops / (ms_per_step * 1e-3) / 1e12, 2),
        "stages_ms_per_step": {k: round(v, 4) for k, v in tot.items()},
        "quant_gbs": round(quant_bytes / (tot["quant"] * 1e-3) / 1e9, 1),
        "groups": per_group,
        "projections": per_proj,
    }
    if cb is not None:
        cb["value"] = round(cb["value"], 6)
        cb["full_step_tops"] = round(cb["full_step_tops"], 6)
        line["cpu_baseline"] = cb
    print(json.dumps(line))


if __name__ == "__main__":
    main()
