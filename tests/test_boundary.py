"""The C-ABI boundary of libsq, without a GPU.

Argument validation runs on the host before any HIP call, so invalid calls can
be checked with fake, never-dereferenced pointer values. Nothing here launches
a kernel.
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from div_cases import near_midpoint_pairs  # noqa: E402
import w8a8_smoothquant_int8_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sq.h")

P = ctypes.c_void_p(0x10000)        # 16-byte aligned fake device pointer
P4 = ctypes.c_void_p(0x10004)       # 4-byte aligned, not 16
NULL = None
S = None                            # stream


@pytest.fixture(scope="module")
def L():
    return sq.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(sq_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sq.SIGNATURES)


def test_status_strings(L):
    for code in range(0, -7, -1):
        assert sq.status_string(code).startswith("SQ_")
    assert "unknown" in sq.status_string(17)


def test_query_support_rejects_null(L):
    assert L.sq_query_support(0, None) == sq.SQ_ERR_INVALID_ARG


def _env_run(code: str, env_extra: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          cwd=ROOT, timeout=120)


def test_arch_gate_forced_unsupported_warns_once():
    code = (
        "import ctypes, w8a8_smoothquant_int8_amd as sq\n"
        "L = sq.lib(); P = ctypes.c_void_p(0x10000)\n"
        "out = ctypes.c_int(7)\n"
        "assert L.sq_query_support(0, ctypes.byref(out)) == 0 and out.value == 0\n"
        "for _ in range(3):\n"
        "    rc = L.sq_quant_per_token(P, sq.SQ_BF16, 4, 64, 64, None, 0, P, P, None)\n"
        "    assert rc == sq.SQ_ERR_UNSUPPORTED_ARCH, rc\n"
        "print('done')\n")
    r = _env_run(code, {"SQ_FORCE_ARCH": "gfx942"})
    assert r.returncode == 0, r.stderr
    assert r.stderr.count("not gfx950") == 1
    assert "done" in r.stdout


def test_arch_gate_forced_supported_query():
    code = ("import ctypes, w8a8_smoothquant_int8_amd as sq\n"
            "out = ctypes.c_int(0)\n"
            "assert sq.lib().sq_query_support(0, ctypes.byref(out)) == 0 and out.value == 1\n")
    r = _env_run(code, {"SQ_FORCE_ARCH": "gfx950"})
    assert r.returncode == 0, r.stderr


# ---------------------------------------------------------------------------
# Validation: each call rejects bad arguments before touching the device.
# ---------------------------------------------------------------------------
def test_calibrate_validation(L):
    f = L.sq_calibrate_absmax
    assert f(NULL, sq.SQ_BF16, 4, 64, 64, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, 7, 4, 64, 64, P, S) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert f(P, sq.SQ_BF16, -1, 64, 64, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, sq.SQ_BF16, 4, 0, 64, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, sq.SQ_BF16, 4, 64, 32, P, S) == sq.SQ_ERR_INVALID_ARG       # ld < K
    assert f(P, sq.SQ_BF16, 4, 40, 48, P, S) == sq.SQ_ERR_MISALIGNED        # K % 16
    assert f(P, sq.SQ_BF16, 4, 64, 72, P, S) == sq.SQ_ERR_MISALIGNED        # ld % 16
    assert f(P4, sq.SQ_BF16, 4, 64, 64, P, S) == sq.SQ_ERR_MISALIGNED
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, sq.SQ_BF16, 4, 65536, 65536, P, S) == sq.SQ_ERR_INVALID_ARG  # K > 32768
    assert f(P, sq.SQ_BF16, 0, 64, 64, P, S) == sq.SQ_OK                    # M = 0: no-op


def test_smooth_validation(L):
    f = L.sq_smooth_scale
    assert f(P, P, sq.SQ_BF16, 8, 64, 64, -0.1, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, P, sq.SQ_BF16, 8, 64, 64, 1.5, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, P, sq.SQ_BF16, 8, 64, 64, float("nan"), P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(NULL, P, sq.SQ_BF16, 8, 64, 64, 0.5, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, P, sq.SQ_BF16, 0, 64, 64, 0.5, P, S) == sq.SQ_ERR_INVALID_ARG   # N >= 1
    g = L.sq_smooth_fold
    assert g(P, P, sq.SQ_BF16, 8, 64, 64, 0.5, P, NULL, P, S) == sq.SQ_ERR_INVALID_ARG
    assert g(P, P, sq.SQ_BF16, 8, 64, 64, 0.5, P, P4, P, S) == sq.SQ_ERR_MISALIGNED
    h = L.sq_fold_quant_weights
    assert h(P, sq.SQ_F16, 8, 64, 64, NULL, NULL, P, S) == sq.SQ_ERR_INVALID_ARG
    assert h(P, sq.SQ_F16, 8, 64, 64, NULL, P4, P, S) == sq.SQ_ERR_MISALIGNED
    assert L.sq_static_act_scale(NULL, NULL, 64, P, S) == sq.SQ_ERR_INVALID_ARG
    assert L.sq_static_act_scale(P, NULL, 0, P, S) == sq.SQ_ERR_INVALID_ARG


def test_quant_validation(L):
    f = L.sq_quant_per_token
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, 5, P, P, S) == sq.SQ_ERR_INVALID_ARG     # mode
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, 0, NULL, P, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, 0, P, NULL, S) == sq.SQ_ERR_INVALID_ARG
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, 0, P4, P, S) == sq.SQ_ERR_MISALIGNED
    assert f(P, sq.SQ_BF16, 0, 64, 64, NULL, 0, P, P, S) == sq.SQ_OK


def test_static_clipped_validation(L):
    f = L.sq_quant_static_clipped
    P8 = ctypes.c_void_p(0x10008)
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, P, P, NULL, S) == sq.SQ_ERR_INVALID_ARG    # counter
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, NULL, P, P, S) == sq.SQ_ERR_INVALID_ARG    # scale
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, P, NULL, P, S) == sq.SQ_ERR_INVALID_ARG    # Xq
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, P, P, P4, S) == sq.SQ_ERR_MISALIGNED       # counter % 8
    assert f(P, sq.SQ_BF16, 4, 64, 64, NULL, P, P4, P, S) == sq.SQ_ERR_MISALIGNED       # Xq % 16
    assert f(P, sq.SQ_BF16, 4, 40, 48, NULL, P, P, P, S) == sq.SQ_ERR_MISALIGNED        # K % 16
    assert f(P, 9, 4, 64, 64, NULL, P, P, P, S) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert f(P, sq.SQ_BF16, 0, 64, 64, NULL, P, P, P8, S) == sq.SQ_OK                   # M == 0


def test_gemm_workspace_rules(L):
    wsb = L.sq_w8a8_gemm_workspace_bytes
    # decode shapes with fewer than 128 column blocks of 64 split K: slices x
    # ceil(N/32) 32-column tiles x 2 row tiles x 4 KB; at most 256 blocks, each
    # slice at least 8 K-tiles
    need = wsb(64, 5120, 20480)
    assert need == 3 * 160 * 2 * 4096                # 80 column blocks: 3 slices
    assert wsb(32, 5120, 20480) == need              # rows pad to two row tiles
    assert wsb(64, 5120, 5120) == 3 * 160 * 2 * 4096     # 40 K-tiles: 3 slices of 14, 14, 12
    assert wsb(64, 1040, 8192) == 8 * 33 * 2 * 4096      # 17 blocks: capped at 64 / 8 slices
    assert wsb(128, 5120, 20480) == 0          # not decode-sized
    assert wsb(64, 8192, 8192) == 0            # 128 column blocks: no split
    assert wsb(64, 20480, 5120) == 0
    assert wsb(64, 5120, 1024) == 0            # 8 K-tiles: too few for two slices
    assert wsb(64, 5120, 8192) > 0
    assert wsb(64, 5120, 2048) == 2 * 160 * 2 * 4096     # 16 K-tiles: 2 slices of 8
    assert wsb(33, 6144, 3072) == 2 * 192 * 2 * 4096     # 96 column blocks: 2 slices
    assert wsb(48, 4096, 8192) == 4 * 128 * 2 * 4096     # 64 column blocks: 4 slices
    assert wsb(64, 5120, 1000) == 0            # K not a multiple of 128
    assert wsb(0, 5120, 20480) == 0 and wsb(-1, 64, 64) == 0
    f = L.sq_w8a8_gemm_ws
    args = lambda **kw: [kw.get(k, v) for k, v in dict(
        xq=P, wq=P, a=P, mode=0, w=P, M=64, N=5120, K=20480, Y=P, yt=sq.SQ_BF16, ldy=5120,
        ws=P, wsb=need, st=S).items()]
    assert f(*args(ws=NULL)) == sq.SQ_ERR_WORKSPACE
    assert f(*args(wsb=need - 1)) == sq.SQ_ERR_WORKSPACE
    assert f(*args(ws=P4)) == sq.SQ_ERR_MISALIGNED
    assert f(*args(xq=NULL)) == sq.SQ_ERR_INVALID_ARG
    assert f(*args(M=0)) == sq.SQ_OK


def test_gemm_validation(L):
    f = L.sq_w8a8_gemm
    args = lambda **kw: [kw.get(k, v) for k, v in dict(
        xq=P, wq=P, a=P, mode=0, w=P, M=4, N=64, K=64, Y=P, yt=sq.SQ_BF16, ldy=64, st=S).items()]
    assert f(*args()) != sq.SQ_ERR_INVALID_ARG
    assert f(*args(xq=NULL)) == sq.SQ_ERR_INVALID_ARG
    assert f(*args(N=40, ldy=48)) == sq.SQ_ERR_MISALIGNED
    assert f(*args(K=40)) == sq.SQ_ERR_MISALIGNED
    assert f(*args(ldy=32)) == sq.SQ_ERR_INVALID_ARG
    assert f(*args(yt=9)) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert f(*args(mode=3)) == sq.SQ_ERR_INVALID_ARG
    assert f(*args(Y=P4)) == sq.SQ_ERR_MISALIGNED
    assert f(*args(M=0)) == sq.SQ_OK
    g = L.sq_w8a8_gemm_i32
    assert g(P, P, 4, 64, 64, NULL, S) == sq.SQ_ERR_INVALID_ARG
    assert g(P, P, 4, 64, 64, P4, S) == sq.SQ_ERR_MISALIGNED


def test_lora_validation(L):
    ws = L.sq_lora_workspace_bytes(64, 256, 16)
    assert ws > 0
    f = L.sq_lora_apply
    ok = [P, sq.SQ_BF16, 64, 256, 256, P, P, 16, 1.0, P, sq.SQ_BF16, 128, 128, P, ws, S]

    def call(**kw):
        a = list(ok)
        for i, k in enumerate(["X", "xt", "M", "K", "ldx", "A", "B", "r", "scale", "Y", "yt", "N",
                               "ldy", "ws", "wsb", "st"]):
            if k in kw:
                a[i] = kw[k]
        return f(*a)
    assert call(r=0) == sq.SQ_ERR_INVALID_ARG
    assert call(r=136) == sq.SQ_ERR_INVALID_ARG
    assert call(r=12) == sq.SQ_ERR_MISALIGNED
    assert call(A=NULL) == sq.SQ_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == sq.SQ_ERR_WORKSPACE
    assert call(ws=NULL) == sq.SQ_ERR_WORKSPACE
    assert call(scale=float("inf")) == sq.SQ_ERR_INVALID_ARG
    assert call(M=0, ws=NULL, wsb=0) == sq.SQ_OK
    g = L.sq_lora_apply_segmented
    seg = [P, sq.SQ_BF16, 64, 256, 256, 4, P, P, 3, P, P, P, 64, 1.0, P, sq.SQ_BF16, 128, 128, P,
           L.sq_lora_workspace_bytes(64, 256, 64), S]
    bad = list(seg); bad[6] = NULL
    assert g(*bad) == sq.SQ_ERR_INVALID_ARG
    bad = list(seg); bad[12] = 136
    assert g(*bad) == sq.SQ_ERR_INVALID_ARG
    bad = list(seg); bad[19] = 16
    assert g(*bad) == sq.SQ_ERR_WORKSPACE
    bad = list(seg); bad[5] = 0
    assert g(*bad) == sq.SQ_OK                      # no segments: no-op
    # the allocation-free variant: same checks, no workspace, its scratch bounds the shape
    h = L.sq_lora_apply_segmented_noalloc
    na = seg[:19] + [S]
    bad = list(na); bad[6] = NULL
    assert h(*bad) == sq.SQ_ERR_INVALID_ARG
    bad = list(na); bad[12] = 136
    assert h(*bad) == sq.SQ_ERR_INVALID_ARG
    bad = list(na); bad[5] = 0
    assert h(*bad) == sq.SQ_OK
    bad = list(na); bad[2], bad[3], bad[4], bad[12] = 65536, 256, 256, 128
    assert L.sq_lora_workspace_bytes(65536, 256, 128) > 32 << 20
    assert h(*bad) == sq.SQ_ERR_WORKSPACE           # refused before anything runs


def test_lora_workspace_grows_with_rank(L):
    # partial sums (S slices of M x r fp32) plus T (M rows of r rounded up to 32
    # ranks, bf16) plus the segmented pair table (16 bytes x (ceil(M / 64) + M))
    tab = 16 * (2048 // 64 + 2048)
    w16 = L.sq_lora_workspace_bytes(2048, 4096, 16)
    w64 = L.sq_lora_workspace_bytes(2048, 4096, 64)
    assert w64 > w16 >= 2048 * 16 * 4 + 2048 * 32 * 2 + tab
    assert (w16 - 2048 * 32 * 2 - tab) % (2048 * 16 * 4) == 0
    assert (w64 - 2048 * 64 * 2 - tab) % (2048 * 64 * 4) == 0
    assert (L.sq_lora_workspace_bytes(65, 256, 8) - 16 * (2 + 65)) % 16 == 0
    assert L.sq_lora_workspace_bytes(0, 4096, 16) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sq, "_lib", None)
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(sq.LibraryNotBuilt):
        sq.lib()


# ---------------------------------------------------------------------------
# Host-side check of the exact-division identity the quant kernels rely on:
# RN32(RN64(x * RN64(1/d))) == RN32(x / d) for fp32 x, d.
# ---------------------------------------------------------------------------
def test_fp64_reciprocal_division_identity():
    rng = np.random.default_rng(0)
    F = np.float32
    n = 400000
    x = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(F)
    d = np.exp(rng.uniform(-20, 20, n)).astype(F)
    # adversarial: x close to (k + 1/2) * d, the ties of the final integer rounding
    k = rng.integers(-127, 127, n) + 0.5
    d2 = np.exp(rng.uniform(-12, 2, n)).astype(F)
    x2 = (k * d2.astype(np.float64)).astype(F)
    x2 = np.nextafter(x2, np.where(rng.random(n) < 0.5, -np.inf, np.inf).astype(F))
    # the hardest quotients: within about 2^-48 of an fp32 rounding midpoint
    x3, d3, _r = near_midpoint_pairs(20000, 1)
    q = x3.astype(np.float64) / d3.astype(np.float64)
    mid = np.abs(q) * 2.0 ** 25
    mid = mid / 2.0 ** np.floor(np.log2(mid) - 24)          # odd multiples of 2^-25 -> odd integers
    assert np.all(np.abs(mid - np.round(mid)) < 2.0 ** -20)  # the construction lands next to a midpoint
    for a, b in ((x, d), (x2, d2), (x3, d3)):
        ref = a / b
        got = (a.astype(np.float64) * (1.0 / b.astype(np.float64))).astype(F)
        assert np.array_equal(got, ref)
    # the near-midpoint cases tell a plain fp32 reciprocal multiply from a division
    approx = x3 * (F(1.0) / d3)
    assert np.mean(approx != x3 / d3) > 0.2


def test_fp64_reciprocal_division_below_the_normal_range():
    """Subnormal quotients (|x / d| < 2^-126), the case the normal-range proof
    leaves out: exact in general, and at most one subnormal ulp off where the
    quotient is exactly a midpoint of the subnormal grid."""
    rng = np.random.default_rng(1)
    F = np.float32
    n = 500000
    x = (rng.standard_normal(n) * np.exp(rng.uniform(np.log(1e-45), np.log(1e-30), n))).astype(F)
    d = np.exp(rng.uniform(np.log(1e-5), np.log(1e5), n)).astype(F)
    assert np.count_nonzero(np.abs(x / d) < 2.0 ** -126) > n // 3
    got = (x.astype(np.float64) * (1.0 / d.astype(np.float64))).astype(F)
    assert np.array_equal(got, x / d)
    # exact midpoints: x = d (2j + 1) 2^-150, representable when d's odd part is small
    d = ((rng.integers(1, 2 ** 12, n) * 2 + 1) * 2.0 ** (rng.integers(0, 30, n) - 20)).astype(F)
    xt = d.astype(np.float64) * (2 * rng.integers(0, 2 ** 10, n) + 1) * 2.0 ** -150
    keep = xt.astype(F).astype(np.float64) == xt
    x, d = xt[keep].astype(F), d[keep]
    ref = x / d
    got = (x.astype(np.float64) * (1.0 / d.astype(np.float64))).astype(F)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() == 1 and np.all(np.abs(ref) < 2.0 ** -126)
    # one fp32 step of x away from each midpoint, the quotient is exact again
    for toward in (np.inf, -np.inf):
        xn = np.nextafter(x, F(toward))
        assert np.array_equal((xn.astype(np.float64) * (1.0 / d.astype(np.float64))).astype(F), xn / d)


def test_code_word_rounding():
    """The quantizers' one-add code: clamp to [-127, 127], add 1.5 * 2^23 in
    fp32 (round half to even), take the low byte as int8. Emulated with numpy
    fp32 arithmetic against clamp(rint(q)) on every half-integer and its fp32
    neighbours in [-140, 140], and on random quotients."""
    F = np.float32
    h = np.arange(-280, 281, dtype=np.float64) / 2.0
    q = np.concatenate([h, np.nextafter(h.astype(F), F(-np.inf)).astype(np.float64),
                        np.nextafter(h.astype(F), F(np.inf)).astype(np.float64),
                        np.random.default_rng(3).uniform(-200, 200, 200000)]).astype(F)
    t = np.minimum(np.maximum(q, F(-127.0)), F(127.0))
    word = (t + F(12582912.0)).view(np.uint32)
    got = (word & 0xFF).astype(np.uint8).view(np.int8)
    ref = np.clip(np.rint(q), -127, 127).astype(np.int8)
    assert np.array_equal(got, ref)


def _group(**over):
    """An sq_linear_group filled with valid fake pointers and shapes."""
    d = sq.SqLinearGroup()
    d.X, d.xt, d.M, d.ldx = 0x10000, sq.SQ_BF16, 64, 256
    d.X_cal, d.M_cal, d.ld_cal = 0x20000, 64, 256
    d.W, d.wt, d.N, d.K, d.ldw = 0x30000, sq.SQ_BF16, 128, 256, 256
    d.alpha, d.mode = 0.5, sq.SQ_ACT_PER_TOKEN_DYNAMIC
    d.act_max, d.s, d.Wq, d.w_scale = 0x40000, 0x41000, 0x50000, 0x60000
    d.Xq, d.a_scale = 0x70000, 0x80000
    d.A, d.B, d.r, d.lora_scale, d.T, d.ldt = 0x90000, 0xA0000, 16, 1.0, 0xB0000, 16
    d.workspace, d.workspace_bytes = 0xC0000, sq.sq_lora_workspace_bytes(64, 256, 16)
    d.Y, d.yt, d.ldy = 0xD0000, sq.SQ_BF16, 128
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _run(L, d, flags=7, events=None):
    return L.sq_linear_group_run(ctypes.byref(d), flags, S,
                                 ctypes.byref(events) if events is not None else None)


@pytest.mark.parametrize("cname,py", [("sq_linear_group", sq.SqLinearGroup),
                                      ("sq_group_events", sq.SqGroupEvents)])
def test_group_struct_layout_matches_header(tmp_path, cname, py):
    """The ctypes mirrors of the C structs have their size and field offsets."""
    fields = [f for f, _ in py._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'  printf(" %zu", offsetof({cname}, {f}));\n' for f in fields)
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n"
                   f'#include "{HEADER}"\n'
                   "int main(void) {\n"
                   f'  printf("%zu", sizeof({cname}));\n'
                   + body +
                   '  printf("\\n");\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(py)
    assert out[1:] == [getattr(py, f).offset for f in fields]


def test_group_validation(L):
    """Every phase's arguments are checked before anything is enqueued."""
    E = sq
    assert L.sq_linear_group_run(None, 7, S, None) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(), flags=0) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(), flags=8) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(mode=5)) == E.SQ_ERR_INVALID_ARG
    # calibrate
    assert _run(L, _group(X_cal=None), flags=1) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(ld_cal=200), flags=1) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(act_max=0x40002), flags=1) == E.SQ_ERR_MISALIGNED
    # fold
    assert _run(L, _group(alpha=1.5), flags=2) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(Wq=0x50004), flags=2) == E.SQ_ERR_MISALIGNED
    assert _run(L, _group(wt=7), flags=2) == E.SQ_ERR_UNSUPPORTED_DTYPE
    assert _run(L, _group(K=250, ldx=250, ldw=250, ld_cal=250), flags=2) == E.SQ_ERR_MISALIGNED
    # forward
    assert _run(L, _group(N=120, ldy=128), flags=4) == E.SQ_ERR_MISALIGNED
    assert _run(L, _group(ldy=64), flags=4) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(r=12), flags=4) == E.SQ_ERR_MISALIGNED
    assert _run(L, _group(r=136), flags=4) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(T=None), flags=4) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _group(workspace_bytes=16), flags=4) == E.SQ_ERR_WORKSPACE
    assert _run(L, _group(yt=9), flags=4) == E.SQ_ERR_UNSUPPORTED_DTYPE
    # a forward-phase error stops the call even when the earlier phases are valid
    assert _run(L, _group(Y=None), flags=7) == E.SQ_ERR_INVALID_ARG
    # no LoRA: A, B, T and the workspace are not needed
    d = _group(r=0, A=None, B=None, T=None, workspace=None, workspace_bytes=0)
    assert _run(L, d, flags=4) in (E.SQ_OK, E.SQ_ERR_UNSUPPORTED_ARCH)


def _parts(d, parts):
    d.lora_parts = len(parts)
    for i, (n, r) in enumerate(parts):
        d.lora_n_end[i], d.lora_r_end[i] = n, r
    return d


def test_group_lora_parts_validation(L):
    """The projection table of stacked adapters: increasing column and rank
    bounds ending at N and r, columns on 16, ranks on 8, at most 4 parts."""
    E = sq
    ok = (E.SQ_OK, E.SQ_ERR_UNSUPPORTED_ARCH)
    assert _run(L, _parts(_group(), [(64, 8), (128, 16)]), flags=4) in ok
    assert _run(L, _parts(_group(), [(128, 16)]), flags=4) in ok          # one part: no table
    assert _run(L, _group(lora_parts=-1), flags=4) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _parts(_group(), [(64, 8), (112, 16)]), flags=4) == E.SQ_ERR_INVALID_ARG  # != N
    assert _run(L, _parts(_group(), [(64, 8), (128, 24)]), flags=4) == E.SQ_ERR_INVALID_ARG  # != r
    assert _run(L, _parts(_group(), [(56, 8), (128, 16)]), flags=4) == E.SQ_ERR_MISALIGNED
    assert _run(L, _parts(_group(), [(64, 4), (128, 16)]), flags=4) == E.SQ_ERR_MISALIGNED
    assert _run(L, _parts(_group(), [(64, 8), (64, 16)]), flags=4) == E.SQ_ERR_INVALID_ARG
    assert _run(L, _parts(_group(), [(64, 8), (128, 8)]), flags=4) == E.SQ_ERR_INVALID_ARG
    d = _parts(_group(), [(32, 8), (64, 16), (96, 16), (128, 16)])
    d.lora_parts = 5
    assert _run(L, d, flags=4) == E.SQ_ERR_INVALID_ARG
    # the table is read only with LoRA
    d = _group(r=0, A=None, B=None, T=None, workspace=None, workspace_bytes=0, lora_parts=9)
    assert _run(L, d, flags=4) in ok


def test_group_events_accepted(L):
    """A group call with an events struct of NULL entries is valid (nothing recorded)."""
    ev = sq.SqGroupEvents()
    assert _run(L, _group(), flags=4, events=ev) in (sq.SQ_OK, sq.SQ_ERR_UNSUPPORTED_ARCH)


def test_alpha_sweep_validation(L):
    f = L.sq_alpha_sweep
    A = (ctypes.c_double * 3)(0.0, 0.5, 1.0)
    BAD = (ctypes.c_double * 2)(0.5, 1.5)
    need = L.sq_alpha_sweep_workspace_bytes(64, 32, 128)
    assert need > 12 * 64 * 32 + 32 * 128 + 64 * 128
    assert L.sq_alpha_sweep_workspace_bytes(0, 32, 128) == 0
    W256 = ctypes.c_void_p(0x100000)

    def call(X=P, xt=sq.SQ_BF16, M=64, K=128, ldx=128, W=P, wt=sq.SQ_BF16, N=32, ldw=128, al=A,
             n=3, mode=0, err=P, rel=NULL, best=NULL, ws=W256, wsb=None):
        return f(X, xt, M, K, ldx, W, wt, N, ldw, al, n, mode, err, rel, best, ws,
                 need if wsb is None else wsb, S)
    assert call(W=NULL) == sq.SQ_ERR_INVALID_ARG
    assert call(N=24) == sq.SQ_ERR_MISALIGNED                      # N % 16
    assert call(ldw=64) == sq.SQ_ERR_INVALID_ARG                   # ldw < K
    assert call(al=None) == sq.SQ_ERR_INVALID_ARG
    assert call(n=0) == sq.SQ_ERR_INVALID_ARG
    assert call(al=BAD, n=2) == sq.SQ_ERR_INVALID_ARG              # alpha outside [0, 1]
    assert call(mode=3) == sq.SQ_ERR_INVALID_ARG
    assert call(err=P4) == sq.SQ_ERR_MISALIGNED
    assert call(rel=P4) == sq.SQ_ERR_MISALIGNED                    # fp64 output
    assert call(best=ctypes.c_void_p(0x10002)) == sq.SQ_ERR_MISALIGNED
    assert call(ws=NULL) == sq.SQ_ERR_WORKSPACE
    assert call(wsb=need - 1) == sq.SQ_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == sq.SQ_ERR_MISALIGNED  # not 256-byte aligned
    assert call(wt=7) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert call(M=0, ws=NULL) == sq.SQ_OK


def test_norm_validation(L):
    f = L.sq_norm_quant

    def call(H=P, ht=sq.SQ_BF16, M=4, K=64, ldh=64, norm=0, g=P, b=NULL, eps=1e-5, mode=0, Xq=P,
             a=P, st=NULL):
        return f(H, ht, M, K, ldh, norm, g, b, ctypes.c_float(eps), mode, Xq, a, st, S)
    assert call(norm=2) == sq.SQ_ERR_INVALID_ARG
    assert call(b=P) == sq.SQ_ERR_INVALID_ARG                      # bias with RMS
    assert call(g=NULL) == sq.SQ_ERR_INVALID_ARG
    assert call(eps=-1.0) == sq.SQ_ERR_INVALID_ARG
    assert call(eps=float("nan")) == sq.SQ_ERR_INVALID_ARG
    assert call(mode=4) == sq.SQ_ERR_INVALID_ARG
    assert call(K=16400, ldh=16400) == sq.SQ_ERR_INVALID_ARG       # beyond 16384 (16-bit)
    assert call(ht=sq.SQ_F32, K=4112, ldh=4112) == sq.SQ_ERR_INVALID_ARG   # beyond 4096 (fp32)
    assert call(g=P4) == sq.SQ_ERR_MISALIGNED
    assert call(norm=1, b=P4) == sq.SQ_ERR_MISALIGNED
    assert call(Xq=P4) == sq.SQ_ERR_MISALIGNED
    assert call(M=0) == sq.SQ_OK
    fold = L.sq_fold_norm_weight
    assert fold(NULL, NULL, sq.SQ_BF16, 64, NULL, P, NULL, S) == sq.SQ_ERR_INVALID_ARG
    assert fold(P, P, sq.SQ_BF16, 64, NULL, P, NULL, S) == sq.SQ_ERR_INVALID_ARG   # beta_out missing
    assert fold(P, NULL, 9, 64, NULL, P, NULL, S) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert fold(P, NULL, sq.SQ_BF16, 0, NULL, P, NULL, S) == sq.SQ_ERR_INVALID_ARG
    assert fold(P, NULL, sq.SQ_F32, 64, NULL, ctypes.c_void_p(0x10002), NULL, S) == sq.SQ_ERR_MISALIGNED


def test_quant_shrink_validation(L):
    f = L.sq_quant_shrink

    def call(X=P, xt=sq.SQ_BF16, M=4, K=64, ldx=64, s=NULL, mode=0, Xq=P, a=P, A=P, r=16, T=P,
             ldt=16):
        return f(X, xt, M, K, ldx, s, mode, Xq, a, A, r, T, ldt, S)
    assert call(xt=sq.SQ_F32) == sq.SQ_ERR_UNSUPPORTED_DTYPE
    assert call(K=8208, ldx=8208) == sq.SQ_ERR_INVALID_ARG       # beyond 8192 (bf16)
    assert call(xt=sq.SQ_F16, K=4112, ldx=4112) == sq.SQ_ERR_INVALID_ARG   # beyond 4096 (fp16)
    assert call(r=0) == sq.SQ_ERR_INVALID_ARG
    assert call(r=12) == sq.SQ_ERR_MISALIGNED
    assert call(r=136, ldt=136) == sq.SQ_ERR_INVALID_ARG
    assert call(A=NULL) == sq.SQ_ERR_INVALID_ARG
    assert call(ldt=8) == sq.SQ_ERR_INVALID_ARG                  # ldt < r
    assert call(ldt=20, r=16) == sq.SQ_ERR_MISALIGNED
    assert call(A=P4) == sq.SQ_ERR_MISALIGNED
    assert call(mode=2) == sq.SQ_ERR_INVALID_ARG
    assert call(M=0) == sq.SQ_OK
