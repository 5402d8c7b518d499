"""Every workload at full size through the call the benchmark times (GPU).

Each input group runs as one sq_linear_group_run call (calibrate, smooth and
fold, quantize, LoRA shrink, GEMM with the dequant and LoRA epilogue; then the
segmented LoRA calls for per-request adapters), at the workload's real
shapes, in the launch configuration bench.py uses. The oracle then recomputes
what it can afford one output at a time:
  - the calibration maxima and the smoothing vector, in full;
  - the weight codes and scales of sampled weight rows, the activation codes
    and scales of sampled activation rows;
  - the outputs at every (row, column) pair of the samples. The samples take
    one row in every tile row and one column in every tile column of the
    tile configuration the library picks for the group's GEMM (at an offset
    inside the tile that changes from tile to tile, so different waves and
    lanes are checked), plus the first and last row and column, each
    projection's edges and the rows holding the largest outliers: every
    output tile has compared elements;
  - for the group's first projection, one whole tile-wide column band over
    all M rows, in chunks of rows.
Properties that hold at any size (|code| <= 127, every nonzero row reaching
127) are checked on the full GPU outputs. The tiny workload is compared in
full.
"""
import numpy as np
import pytest
import torch

import bench
import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import WORKLOADS, get_workload
from w8a8_smoothquant_int8_amd.pipeline import ALL_PHASES, LinearGroup, SegmentedLora

pytestmark = pytest.mark.gpu
F32 = np.float32


def npf(t):
    return t.detach().float().cpu().numpy()


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def lora_ok(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return bool(np.all(np.abs(got - ref) <= 2e-2 * np.abs(ref) + 2e-2 * rms))


def out_np(t, out_dtype):
    t = t.cpu()
    return t.numpy() if out_dtype == "f16" else t.float().numpy()


def build_segmented(wl, proj, seed=0):
    seg = wl.segments(seed)
    ranks = seg["ranks"]
    As, Bs = [], []
    for ad, r in enumerate(ranks):
        a, b = wl.lora(proj, rank=int(r), adapter=ad, seed=seed)
        As.append(a)
        Bs.append(b)
    Ad = [t.cuda() for t in As]
    Bd = [t.cuda() for t in Bs]
    sl = SegmentedLora(
        seg_start=torch.from_numpy(seg["seg_start"]).cuda(),
        seg_adapter=torch.from_numpy(seg["seg_adapter"]).cuda(),
        A=Ad, B=Bd, ranks=torch.from_numpy(ranks).cuda(),
        A_ptrs=sq.pointer_table(Ad, "cuda"), B_ptrs=sq.pointer_table(Bd, "cuda"),
        max_rank=int(ranks.max()))
    return sl, seg, As, Bs


def per_tile(n, t, salt):
    """One index in every tile [i t, min((i + 1) t, n)), at an offset inside the
    tile that moves from tile to tile."""
    out = []
    for i in range(-(-n // t)):
        lo, hi = i * t, min(n, (i + 1) * t)
        out.append(lo + (i * salt + 5) % (hi - lo))
    return out


def tile_samples(M, Ntot, K, rows, lora, extra_rows=()):
    """Sampled rows and columns of a group output: every tile row and tile
    column of the library's tile configuration, plus the edges."""
    tile = bench.gemm_tile(M, Ntot, K, lora=lora)
    BM, BN = bench.tile_dims(tile)
    if tile in ("skinny", "decode", "decode128"):
        BM = 8            # M <= 64: rows of both 32-row MFMA tiles, 8 apart
    # decode blocks: a column in every wave's 32-column MFMA tile
    cstep = 32 if tile in ("decode", "decode128") else BN
    r = set(per_tile(M, BM, 37)) | {0, M - 1} | {int(v) for v in extra_rows if 0 <= v < M}
    c = set(per_tile(Ntot, cstep, 53)) | {0, Ntot - 1}
    for r0, r1 in rows.values():
        c |= {r0, r1 - 1}
    return np.array(sorted(r), np.int64), np.array(sorted(c), np.int64), tile, BN


def ref_outputs(wl, p, rows_m, cols_g, r0, Xn, xq_ref, a_use, Wn, s_ref, host, loras, segs):
    """The oracle's outputs of projection p at rows_m x cols_g (group columns)."""
    wq_p, ws_p = O.fold_and_quantize_weights(Wn[cols_g], s_ref)
    y_ref = O.dequantize(O.int8_gemm(xq_ref, wq_p), a_use, ws_p, wl.out_dtype)
    if p in loras:
        a, b = host[p]
        return O.lora_apply(y_ref, Xn[rows_m], wl.dtype, a, b[cols_g - r0], 1.0, wl.out_dtype), True
    if p in segs:
        seg, As, Bs = host[p]
        y_ref = np.array(y_ref, copy=True)
        gidx = np.searchsorted(seg["seg_start"], rows_m, side="right") - 1
        for i, m in enumerate(rows_m):
            ad = seg["seg_adapter"][gidx[i]]
            if ad >= 0:
                y_ref[i:i + 1] = O.lora_apply(y_ref[i:i + 1], Xn[m:m + 1], wl.dtype, As[ad],
                                              Bs[ad][cols_g - r0], 1.0, wl.out_dtype)
        return y_ref, True
    return y_ref, False


def check_group(wl, inp, seed=0):
    X = wl.x(inp, seed)
    Xc = wl.x_cal(inp, seed)
    W = wl.w_group(inp, seed)
    rows = wl.group_rows(inp)
    loras, segs, host = {}, {}, {}
    for p in rows:
        if wl.lora_rank:
            a, b = wl.lora(p, seed=seed)
            loras[p] = (a.cuda(), b.cuda())
            host[p] = (a.float().numpy(), b.float().numpy())
        elif wl.segmented:
            sl, seg, As, Bs = build_segmented(wl, p, seed)
            segs[p] = sl
            host[p] = (seg, [t.float().numpy() for t in As], [t.float().numpy() for t in Bs])
    Xd, Xcd = X.cuda(), Xc.cuda()
    g = LinearGroup(W.cuda(), rows, wl.alpha, wl.out_dtype, wl.M, lora=loras, seg_lora=segs,
                    modes=wl.act_modes)
    if wl.lora_rank and len(rows) > 1:
        assert g.lora_parts is not None          # the run takes the projections' rank windows
    Xn, Xcn, Wn = X.float().numpy(), Xc.float().numpy(), W.float().numpy()
    act_max = O.calibrate_absmax(Xcn)
    s_ref = O.smoothing_scale(act_max, O.weight_absmax(Wn), wl.alpha)
    Ntot, K = W.shape
    outlier_rows = np.argsort(-np.abs(Xn).max(axis=1))[:4]
    m_rows, cols, tile, BN = tile_samples(wl.M, Ntot, K, rows, g.fused, outlier_rows)
    print(f"[{wl.name}/{inp}] tile {tile}: {len(m_rows)} rows x {len(cols)} columns", flush=True)

    for mode in wl.act_modes:
        g.run(Xd, Xcd, ALL_PHASES, mode=mode)
        torch.cuda.synchronize()
        assert bits_equal(npf(g.act_max), act_max)
        s_gpu = npf(g.s)
        if not bits_equal(s_gpu, s_ref):
            # fp64 pow may land one fp32 ulp apart at a rounding boundary (alpha != 0.5);
            # then the later stages run again on the oracle's s, so the comparison
            # below checks each stage on the oracle's own inputs.
            assert wl.alpha != 0.5
            ulps = np.abs(s_gpu.view(np.int32).astype(np.int64) - s_ref.view(np.int32).astype(np.int64))
            assert ulps.max() <= 1 and np.count_nonzero(ulps) <= 2
            g.s.copy_(torch.from_numpy(s_ref))
            sq.sq_fold_quant_weights(g.W, g.s, g.Wq, g.w_scale)
            sq.sq_static_act_scale(g.act_max, g.s, g.static_scale)
            g.run(Xd, Xcd, sq.SQ_GROUP_FORWARD, mode=mode)
            torch.cuda.synchronize()
        Yg = g.Yg.clone()

        # weight codes and scales of the sampled output columns; properties in full
        wq_ref, wsc_ref = O.fold_and_quantize_weights(Wn[cols], s_ref)
        assert bits_equal(g.Wq[cols].cpu().numpy(), wq_ref)
        assert bits_equal(npf(g.w_scale)[cols], wsc_ref)
        assert int(g.Wq.abs().amax()) <= 127
        assert bool((g.Wq[g.W.abs().amax(dim=1) > 0].abs().amax(dim=1) == 127).all())

        if mode == "dynamic":
            xq_ref, a_ref = O.quantize_per_token(Xn[m_rows], s_ref)
            assert bits_equal(npf(g.a_scale)[m_rows], a_ref)
            a_use = a_ref
            nz = g.Xq.abs().amax(dim=1)
            assert int(nz.max()) <= 127
            assert bool((nz[Xd.abs().amax(dim=1) > 0] == 127).all())
        else:
            a_use = O.static_activation_scale(act_max, s_ref)
            assert npf(g.static_scale)[0] == a_use
            xq_ref, _clipped = O.quantize_per_tensor_static(Xn[m_rows], s_ref, a_use)
        assert bits_equal(g.Xq[m_rows].cpu().numpy(), xq_ref)

        got_all = out_np(Yg, wl.out_dtype)
        for p, (r0, r1) in rows.items():
            cg = cols[(cols >= r0) & (cols < r1)]
            y_ref, lora = ref_outputs(wl, p, m_rows, cg, r0, Xn, xq_ref, a_use, Wn, s_ref, host,
                                      loras, segs)
            got = got_all[np.ix_(m_rows, cg)]
            assert (lora_ok(got, y_ref) if lora else bits_equal(got, y_ref)), (mode, p)

        # one whole tile-wide column band of the first projection, all rows
        p0, (r0, r1) = next(iter(rows.items()))
        b0 = r0 + ((r1 - r0) // 2 // BN) * BN
        band = np.arange(b0, min(b0 + BN, r1), dtype=np.int64)
        for c0 in range(0, wl.M, 2048):
            mr = np.arange(c0, min(c0 + 2048, wl.M), dtype=np.int64)
            if mode == "dynamic":
                xq_b, a_b = O.quantize_per_token(Xn[mr], s_ref)
                assert bits_equal(npf(g.a_scale)[mr], a_b)
            else:
                a_b = a_use
                xq_b, _ = O.quantize_per_tensor_static(Xn[mr], s_ref, a_use)
            assert bits_equal(g.Xq[mr].cpu().numpy(), xq_b)
            y_ref, lora = ref_outputs(wl, p0, mr, band, r0, Xn, xq_b, a_b, Wn, s_ref, host,
                                      loras, segs)
            got = got_all[np.ix_(mr, band)]
            assert (lora_ok(got, y_ref) if lora else bits_equal(got, y_ref)), (mode, p0, c0)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_full_size(name):
    wl = get_workload(name)
    for inp, _K in wl.inputs:
        check_group(wl, inp)
        torch.cuda.empty_cache()


def test_tiny_workload_in_full():
    wl = get_workload("tiny_m16_k256_n256")
    X, Xc, W = wl.x("x"), wl.x_cal("x"), wl.w_group("x")
    a, b = wl.lora("linear")
    g = LinearGroup(W.cuda(), wl.group_rows("x"), wl.alpha, wl.out_dtype, wl.M,
                    lora={"linear": (a.cuda(), b.cuda())})
    g.calibrate(Xc.cuda())
    g.fold()
    Xd = X.cuda()
    g.quantize(Xd)
    g.gemm("linear")
    y = g.Y["linear"].clone()
    g.apply_lora("linear", Xd)
    torch.cuda.synchronize()
    r = O.smoothquant_linear(X.float().numpy(), wl.dtype, W.float().numpy(), Xc.float().numpy(),
                             wl.alpha, wl.out_dtype, lora=(a.float().numpy(), b.float().numpy(), 1.0))
    for k, t in (("act_max", g.act_max), ("s", g.s), ("w_scale", g.w_scale), ("a_scale", g.a_scale)):
        assert bits_equal(npf(t), r[k]), k
    assert bits_equal(g.Wq.cpu().numpy(), r["wq"])
    assert bits_equal(g.Xq.cpu().numpy(), r["xq"])
    assert bits_equal(npf(y), r["y"])
    assert lora_ok(npf(g.Y["linear"]), r["y_lora"])


def test_graph_capture_replays_match_eager():
    """The forward pass (quantize, GEMM, LoRA) captured into a HIP graph and
    replayed several times, with eager work in between, matches the eager run."""
    wl = get_workload("llama3_8b_proj_m2048")
    inp = "attn_in"
    X = wl.x(inp).cuda()
    W = wl.w_group(inp).cuda()
    rows = wl.group_rows(inp)
    loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows}
    g = LinearGroup(W, rows, wl.alpha, wl.out_dtype, wl.M, lora=loras)
    g.calibrate(wl.x_cal(inp).cuda())
    g.fold()
    eager = {p: t.clone() for p, t in g.forward(X).items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.forward(X)                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.forward(X)
    for rep in range(3):
        for t in g.Y.values():
            t.fill_(0)
        tmp = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        graph.replay()
        torch.cuda.synchronize()
        for p in rows:
            assert torch.equal(g.Y[p], eager[p]), (rep, p)
        del tmp
