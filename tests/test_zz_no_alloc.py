"""sq_lora_apply_segmented_noalloc: the segmented LoRA call with the library's
own scratch memory, for callers that cannot allocate (GPU).

Each call is compared bit for bit with sq_lora_apply_segmented on a caller
workspace, on the same inputs. Two calls in a row use the scratch, the second
on a smaller input, so the second finds the first one's contents there; a
third, larger call follows. A shape whose workspace would exceed the
scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to, get_workload

pytestmark = pytest.mark.gpu
F32 = np.float32


def case(seed, M, K, N, ranks, ydt="bf16", xdt="bf16"):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max(2, M // 8), size=4 * M).tolist()
    out, tot = [], 0
    for L in lens:
        if tot + L > M:
            break
        out.append(int(L))
        tot += L
    out.append(M - tot)
    out.insert(1, 0)                          # an empty request
    seg_start = np.concatenate([[0], np.cumsum(out)]).astype(np.int32)
    seg_adapter = rng.integers(0, len(ranks), len(out)).astype(np.int32)
    seg_adapter[rng.random(len(out)) < 0.2] = -1
    x = cast_to(rng.standard_normal((M, K)).astype(F32), xdt).cuda()
    As = [cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16").cuda() for r in ranks]
    Bs = [cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16").cuda() for r in ranks]
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), ydt).cuda()
    return dict(x=x, st=torch.from_numpy(seg_start).cuda(), ad=torch.from_numpy(seg_adapter).cuda(),
                ap=sq.pointer_table(As, "cuda"), bp=sq.pointer_table(Bs, "cuda"),
                rk=torch.from_numpy(np.array(ranks, np.int32)).cuda(), mr=max(ranks), y=y,
                keep=(As, Bs))


def both(c):
    Y_ws, Y_na = c["y"].clone(), c["y"].clone()
    M, K = c["x"].shape
    ws = torch.full((sq.sq_lora_workspace_bytes(M, K, c["mr"]),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    sq.sq_lora_apply_segmented(c["x"], c["st"], c["ad"], c["ap"], c["bp"], c["rk"], c["mr"], Y_ws, ws)
    sq.sq_lora_apply_segmented_noalloc(c["x"], c["st"], c["ad"], c["ap"], c["bp"], c["rk"], c["mr"],
                                       Y_na)
    torch.cuda.synchronize()
    return Y_ws, Y_na


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    wl = get_workload("multitenant_lora_m8192")
    seg = wl.segments(0)
    ranks = [int(r) for r in seg["ranks"]]
    big = case(1, wl.M, 4096, 4096, ranks)
    big["st"] = torch.from_numpy(seg["seg_start"]).cuda()          # the workload's requests
    big["ad"] = torch.from_numpy(seg["seg_adapter"]).cuda()
    assert sq.sq_lora_workspace_bytes(wl.M, 4096, big["mr"]) <= 32 << 20
    calls = [big, case(2, 300, 1024, 208, [8, 24, 64, 16]), case(3, 2048, 4096, 1024, [64, 16],
                                                                   ydt="f32", xdt="f16")]
    for i, c in enumerate(calls):
        Y_ws, Y_na = both(c)
        assert torch.equal(Y_ws.view(torch.uint8), Y_na.view(torch.uint8)), i
        assert not torch.equal(Y_na, c["y"]), i        # the delta was added


def test_noalloc_refuses_shapes_beyond_its_scratch():
    M, K, N, r = 65536, 256, 16, 128
    assert sq.sq_lora_workspace_bytes(M, K, r) > 32 << 20
    x = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(r, K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(N, r, dtype=torch.bfloat16, device="cuda")
    st = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    ad = torch.zeros(1, dtype=torch.int32, device="cuda")
    rk = torch.tensor([r], dtype=torch.int32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_lora_apply_segmented_noalloc(x, st, ad, sq.pointer_table([A], "cuda"),
                                           sq.pointer_table([B], "cuda"), rk, r, y)
    assert e.value.status == sq.SQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not y.any()                             # nothing ran
