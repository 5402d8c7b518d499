"""sq_linear_group_run: one native call per input group (GPU).

The call must produce exactly what the single-purpose calls produce in the
same order (calibrate, smooth + fold, quantize, LoRA shrink, GEMM with the
LoRA epilogue): every output is compared bit for bit. The single-purpose path
itself is checked against the oracle in test_gpu_parity.py and
test_gpu_workloads.py.
"""
import pytest
import torch

import bench
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import get_workload
from w8a8_smoothquant_int8_amd.pipeline import ALL_PHASES, LinearGroup

pytestmark = pytest.mark.gpu


def make_group(wl, inp, lora=True, modes=("dynamic",)):
    W = wl.w_group(inp).cuda()
    rows = wl.group_rows(inp)
    loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows} if (lora and wl.lora_rank) else {}
    segs = {p: bench.segmented_lora(wl, p, torch) for p in rows} if (lora and wl.segmented) else {}
    return LinearGroup(W, rows, wl.alpha, wl.out_dtype, wl.M, lora=loras, seg_lora=segs,
                       modes=modes)


def outputs(g, mode="dynamic"):
    a = g.a_scale if mode == "dynamic" else g.static_scale
    return [t.clone() for t in (g.act_max, g.s, g.Wq, g.w_scale, g.Xq, a, g.Yg)]


def separate(g, X, Xc, mode="dynamic"):
    g.calibrate(Xc)
    g.fold()
    g.forward(X, mode)
    torch.cuda.synchronize()
    return outputs(g, mode)


def assert_same(a, b):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), i


@pytest.mark.parametrize("name,inp", [("llama3_8b_proj_m2048", "attn_in"),
                                      ("llama3_8b_proj_m2048", "o_in"),
                                      ("llama3_8b_proj_m2048", "mlp_in"),
                                      ("llama3_8b_proj_m2048", "down_in"),
                                      ("llama2_70b_mlp_m8192", "mlp_in"),
                                      ("llama2_70b_mlp_m8192", "down_in"),
                                      ("multitenant_lora_m8192", "attn_in"),
                                      ("multitenant_lora_m8192", "o_in"),
                                      ("opt13b_layer_decode_m64", "fc2_in")])
def test_group_run_equals_separate_calls(name, inp):
    """Bit for bit: the group call (stacked adapters with their rank windows,
    or segmented adapters after it, or the split-K decode GEMM) against the
    single-purpose calls (full-rank stacked GEMM epilogue, separate GEMM)."""
    wl = get_workload(name)
    g = make_group(wl, inp)
    assert g.fused == bool(wl.lora_rank)
    if wl.lora_rank and len(g.rows) > 1:
        assert g.lora_parts is not None
    X, Xc = wl.x(inp).cuda(), wl.x_cal(inp).cuda()
    ref = separate(g, X, Xc)
    for t in (g.act_max, g.s, g.Wq, g.w_scale, g.Xq, g.a_scale, g.Yg):
        t.zero_()
    g.run(X, Xc)
    torch.cuda.synchronize()
    assert_same(outputs(g), ref)


def test_group_run_static_mode_and_no_lora():
    wl = get_workload("opt13b_layer_prefill_m4096")
    inp = wl.inputs[0][0]
    g = make_group(wl, inp, lora=False, modes=("static",))
    X, Xc = wl.x(inp).cuda(), wl.x_cal(inp).cuda()
    ref = separate(g, X, Xc, mode="static")
    for t in (g.act_max, g.s, g.Wq, g.w_scale, g.Xq, g.static_scale, g.Yg):
        t.zero_()
    g.run(X, Xc, mode="static")
    torch.cuda.synchronize()
    assert_same(outputs(g, "static"), ref)


def test_group_run_phases_one_by_one_and_events():
    wl = get_workload("llama3_8b_proj_m2048")
    g = make_group(wl, "attn_in")
    X, Xc = wl.x("attn_in").cuda(), wl.x_cal("attn_in").cuda()
    g.run(X, Xc)
    torch.cuda.synchronize()
    ref = outputs(g)
    g.Yg.zero_()
    evs = {k: torch.cuda.Event(enable_timing=True) for k in sq.EVENT_FIELDS}
    for e in evs.values():
        e.record()
    for flags in (sq.SQ_GROUP_CALIBRATE, sq.SQ_GROUP_FOLD, sq.SQ_GROUP_FORWARD):
        g.run(X, Xc, flags=flags, events=sq.sq_group_events(**evs))
    torch.cuda.synchronize()
    assert_same(outputs(g), ref)
    # the forward call recorded its events in launch order: quant, shrink, GEMM
    assert evs["begin"].elapsed_time(evs["quant_begin"]) >= 0.0
    assert evs["quant_begin"].elapsed_time(evs["shrink_begin"]) > 0.0
    assert evs["shrink_begin"].elapsed_time(evs["gemm_begin"]) > 0.0
    assert evs["gemm_begin"].elapsed_time(evs["gemm_end"]) > 0.0


def test_group_run_graph_replays_match_eager():
    """The whole step of a group captured into a HIP graph (fills, not
    memsets) and replayed several times, with eager work in between."""
    wl = get_workload("llama3_8b_proj_m2048")
    g = make_group(wl, "mlp_in")
    X, Xc = wl.x("mlp_in").cuda(), wl.x_cal("mlp_in").cuda()
    g.run(X, Xc)
    torch.cuda.synchronize()
    ref = outputs(g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.run(X, Xc, flags=ALL_PHASES)
    for rep in range(3):
        for t in (g.act_max, g.s, g.Wq, g.Xq, g.Yg):
            t.fill_(7)
        tmp = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        graph.replay()
        torch.cuda.synchronize()
        assert_same(outputs(g), ref)
        del tmp
