"""Host-only checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every entry point include/int8mm.h declares,
and reject bad arguments on the host with the documented status codes
before anything is enqueued.  Fake non-null device addresses are used where
a pointer must be non-null; every call here fails validation (or is an
empty no-op) before any pointer is touched.
"""

import ctypes
import math
import os
import re

import pytest

import int8_quantized_matmul_col_amd as mm
from int8_quantized_matmul_col_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8mm.h")

FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first
FAKE_WS = 0x7F0000100000  # 256-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from int8_quantized_matmul_col_amd import build
        build.build()
    return mm.load()


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"INT8MM_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    fns = header_functions()
    assert fns == sorted(["int8_weight_ld", "int8_weight_bytes", "int8_prepare_weight", "int8_matmul_workspace_size",
                          "int8_matmul", "int8_linear", "int8_matmul_stages", "int8_matmul_profiled",
                          "int8_column_absmax", "int8mm_strerror", "int8mm_last_hip_error",
                          "int8_matmul_noalloc", "int8_matmul_noalloc_max_workspace",
                          "int8_pack_weight", "int8_outlier_counts"])
    assert set(fns) == set(binding.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_probe_library_loads_and_exports_the_probes(lib):
    """The measurement probes the benchmark loads live in a library of their
    own, outside the matmul ABI."""
    from int8_quantized_matmul_col_amd import build
    assert os.path.exists(build.PROBE_LIB_PATH)
    probes = ctypes.CDLL(build.PROBE_LIB_PATH)
    for name in ("int8mm_probe_mfma_i8", "int8mm_probe_read", "int8mm_probe_read_copies"):
        assert hasattr(probes, name), name
    assert not hasattr(lib, "int8mm_probe_read")


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (INT8MM_\w+) \(?(-?\d+)\)?", src))
    assert int(consts["INT8MM_OK"]) == binding.INT8MM_OK
    assert int(consts["INT8MM_EINVAL"]) == binding.INT8MM_EINVAL
    assert int(consts["INT8MM_ESHAPE"]) == binding.INT8MM_ESHAPE
    assert int(consts["INT8MM_EWORKSPACE"]) == binding.INT8MM_EWORKSPACE
    assert int(consts["INT8MM_EHIP"]) == binding.INT8MM_EHIP
    assert int(consts["INT8MM_ESCRATCH"]) == binding.INT8MM_ESCRATCH
    assert int(consts["INT8MM_MAX_K"]) == binding.INT8MM_MAX_K
    assert int(consts["INT8MM_DECODE_MAX_M"]) == binding.INT8MM_DECODE_MAX_M
    assert int(consts["INT8MM_MAX_COUNT_THRESHOLDS"]) == binding.INT8MM_MAX_COUNT_THRESHOLDS


def test_int32_accumulator_bound():
    # 127^2 * K must fit in int32 exactly up to MAX_K
    assert 127 * 127 * binding.INT8MM_MAX_K < 2 ** 31
    assert 127 * 127 * (binding.INT8MM_MAX_K + 1) >= 2 ** 31


def test_weight_ld(lib):
    assert lib.int8_weight_ld(-1) == -1
    for K, ld in [(0, 0), (1, 64), (63, 64), (64, 64), (65, 128), (4096, 4096), (11008, 11008),
                  (133144, 133184)]:
        assert lib.int8_weight_ld(K) == ld


def test_weight_bytes(lib):
    assert lib.int8_weight_bytes(-1, 8) == -1 and lib.int8_weight_bytes(8, -1) == -1
    assert lib.int8_weight_bytes(8, binding.INT8MM_MAX_K + 1) == -1
    assert lib.int8_weight_bytes(0, 64) == 0
    assert lib.int8_weight_bytes(1, 1) == 256 * 64          # one padded panel
    assert lib.int8_weight_bytes(4096, 4096) == 4096 * 4096
    assert lib.int8_weight_bytes(300, 520) == 512 * 576


def test_untile_matches_documented_layout():
    import torch
    Rp, L = 512, 128
    flat = torch.arange(Rp * L, dtype=torch.int32) % 251
    buf = flat.to(torch.uint8).view(Rp, L)
    rm = binding.untile(buf, 300)
    for (r, b) in [(0, 0), (5, 70), (255, 127), (256, 0), (299, 64), (257, 127)]:
        off = ((r // 256) * (L // 64) + b // 64) * 16384 + (r % 256) * 64 + b % 64
        assert int(rm[r, b]) == int(flat[off]) % 256


def test_workspace_size(lib):
    ws = lib.int8_matmul_workspace_size
    assert ws(-1, 8, 8) == 0 and ws(8, -1, 8) == 0 and ws(8, 8, -1) == 0
    assert ws(8, binding.INT8MM_MAX_K + 1, 8) == 0
    assert ws(8, binding.INT8MM_MAX_K, 8) > 0
    assert ws(0, 0, 0) >= 256
    assert ws(4096, 4096, 4096) % 256 == 0
    # grows with every dimension; holds at least Xq (M*ldk) and, on the
    # prefill path, the worst-case X_O and W_O slices
    assert ws(4096, 4096, 4096) >= 4096 * 4096 * (1 + 2) + 4096 * 4096 * 2
    assert ws(4096, 8192, 4096) > ws(4096, 4096, 4096)
    assert ws(16, 8192, 28672) < ws(17, 8192, 28672)  # decode path needs no W_O copy


def _mm(lib, X=FAKE, M=4, K=8, Wq=FAKE, s=FAKE, N=4, t=6.0, Y=FAKE, ws=FAKE_WS, nbytes=1 << 30):
    return lib.int8_matmul(X, M, K, Wq, s, N, t, Y, ws, nbytes, None)


def test_matmul_rejects_bad_arguments(lib):
    assert _mm(lib, M=-1) == binding.INT8MM_ESHAPE
    assert _mm(lib, K=-1) == binding.INT8MM_ESHAPE
    assert _mm(lib, N=-1) == binding.INT8MM_ESHAPE
    assert _mm(lib, K=binding.INT8MM_MAX_K + 1) == binding.INT8MM_ESHAPE
    assert _mm(lib, t=float("nan")) == binding.INT8MM_EINVAL
    assert _mm(lib, t=-0.5) == binding.INT8MM_EINVAL
    assert _mm(lib, X=None) == binding.INT8MM_EINVAL
    assert _mm(lib, Wq=None) == binding.INT8MM_EINVAL
    assert _mm(lib, s=None) == binding.INT8MM_EINVAL
    assert _mm(lib, Y=None) == binding.INT8MM_EINVAL
    assert _mm(lib, ws=None) == binding.INT8MM_EWORKSPACE
    assert _mm(lib, ws=FAKE_WS + 16) == binding.INT8MM_EWORKSPACE
    need = lib.int8_matmul_workspace_size(4, 8, 4)
    assert _mm(lib, nbytes=need - 1) == binding.INT8MM_EWORKSPACE
    # the panel-tiled weight takes 16-byte accesses
    assert _mm(lib, Wq=FAKE + 8) == binding.INT8MM_EINVAL


def test_element_pointers_must_be_aligned(lib):
    # float16 pointers on odd addresses, float pointers off 4 bytes
    assert _mm(lib, X=FAKE + 1) == binding.INT8MM_EINVAL
    assert _mm(lib, Y=FAKE + 1) == binding.INT8MM_EINVAL
    assert _mm(lib, s=FAKE + 2) == binding.INT8MM_EINVAL
    assert _lin(lib, b=FAKE + 1) == binding.INT8MM_EINVAL
    assert lib.int8_prepare_weight(FAKE + 1, 4, 8, FAKE, FAKE, None) == binding.INT8MM_EINVAL
    assert lib.int8_prepare_weight(FAKE, 4, 8, FAKE, FAKE + 2, None) == binding.INT8MM_EINVAL
    assert lib.int8_column_absmax(FAKE + 1, 4, 8, FAKE, FAKE_WS, 1 << 30, None) == binding.INT8MM_EINVAL
    assert lib.int8_column_absmax(FAKE, 4, 8, FAKE + 1, FAKE_WS, 1 << 30, None) == binding.INT8MM_EINVAL


def test_matmul_empty_is_a_noop(lib):
    # nothing to compute: returns OK without touching any pointer
    assert _mm(lib, M=0, X=FAKE, Y=FAKE) == binding.INT8MM_OK
    assert _mm(lib, N=0) == binding.INT8MM_OK
    assert _mm(lib, M=0, N=0, K=0) == binding.INT8MM_OK


def test_matmul_accepts_infinite_threshold_in_validation(lib):
    # +inf passes the threshold check: the call then fails on the workspace
    assert _mm(lib, t=math.inf, ws=None) == binding.INT8MM_EWORKSPACE


def _lin(lib, X=FAKE, M=4, K=8, Wq=FAKE, s=FAKE, N=4, b=FAKE, t=6.0, Y=FAKE, ws=FAKE_WS,
         nbytes=1 << 30):
    return lib.int8_linear(X, M, K, Wq, s, N, b, t, Y, ws, nbytes, None)


def test_linear_rejects_bad_arguments(lib):
    # the same checks as int8_matmul; a NULL bias is valid (no bias)
    assert _lin(lib, M=-1) == binding.INT8MM_ESHAPE
    assert _lin(lib, K=binding.INT8MM_MAX_K + 1) == binding.INT8MM_ESHAPE
    assert _lin(lib, t=float("nan")) == binding.INT8MM_EINVAL
    assert _lin(lib, X=None) == binding.INT8MM_EINVAL
    assert _lin(lib, s=None) == binding.INT8MM_EINVAL
    assert _lin(lib, Y=None) == binding.INT8MM_EINVAL
    assert _lin(lib, Wq=FAKE + 8) == binding.INT8MM_EINVAL
    assert _lin(lib, b=None, ws=None) == binding.INT8MM_EWORKSPACE
    assert _lin(lib, ws=FAKE_WS + 16) == binding.INT8MM_EWORKSPACE
    assert _lin(lib, M=0) == binding.INT8MM_OK
    assert _lin(lib, N=0, b=None) == binding.INT8MM_OK


def test_column_absmax_rejects_bad_arguments(lib):
    f = lib.int8_column_absmax
    assert f(FAKE, -1, 8, FAKE, FAKE_WS, 1 << 30, None) == binding.INT8MM_ESHAPE
    assert f(FAKE, 4, binding.INT8MM_MAX_K + 1, FAKE, FAKE_WS, 1 << 30, None) == binding.INT8MM_ESHAPE
    assert f(None, 4, 8, FAKE, FAKE_WS, 1 << 30, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 4, 8, None, FAKE_WS, 1 << 30, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 40, 8, FAKE, None, 1 << 30, None) == binding.INT8MM_EWORKSPACE
    assert f(FAKE, 40, 8, FAKE, FAKE_WS + 64, 1 << 30, None) == binding.INT8MM_EWORKSPACE
    need = lib.int8_matmul_workspace_size(40, 8, 0)
    assert f(FAKE, 40, 8, FAKE, FAKE_WS, need - 1, None) == binding.INT8MM_EWORKSPACE
    assert f(None, 4, 0, None, None, 0, None) == binding.INT8MM_OK  # K == 0: nothing to do


def _thr(*ts):
    return (ctypes.c_float * max(len(ts), 1))(*ts)


def test_outlier_counts_rejects_bad_arguments(lib):
    f = lib.int8_outlier_counts
    ok = _thr(0.0, 6.0, math.inf)
    assert f(FAKE, -1, ok, 3, FAKE, None) == binding.INT8MM_ESHAPE
    assert f(FAKE, binding.INT8MM_MAX_K + 1, ok, 3, FAKE, None) == binding.INT8MM_ESHAPE
    assert f(None, 8, ok, 3, FAKE, None) == binding.INT8MM_EINVAL        # no colmax
    assert f(FAKE, 8, None, 3, FAKE, None) == binding.INT8MM_EINVAL      # no thresholds
    assert f(FAKE, 8, ok, 3, None, None) == binding.INT8MM_EINVAL        # no counts
    assert f(FAKE, 8, ok, 0, FAKE, None) == binding.INT8MM_EINVAL        # none asked for
    lim = binding.INT8MM_MAX_COUNT_THRESHOLDS
    many = _thr(*([6.0] * (lim + 1)))
    assert f(FAKE, 8, many, lim + 1, FAKE, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 8, _thr(6.0, math.nan), 2, FAKE, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 8, _thr(-1.0), 1, FAKE, None) == binding.INT8MM_EINVAL
    assert f(FAKE + 1, 8, ok, 3, FAKE, None) == binding.INT8MM_EINVAL    # misaligned colmax
    assert f(FAKE, 8, ok, 3, FAKE + 2, None) == binding.INT8MM_EINVAL    # misaligned counts


def test_stages_rejects_bad_arguments(lib):
    f = lib.int8_matmul_stages
    args = lambda **kw: [kw.get("X", FAKE), kw.get("M", 4), kw.get("K", 8), FAKE, FAKE,
                         kw.get("N", 4), kw.get("t", 6.0)] + [None] * 9 + \
                        [kw.get("ws", FAKE_WS), kw.get("nbytes", 1 << 30), None]
    assert f(*args(M=-3)) == binding.INT8MM_ESHAPE
    assert f(*args(t=float("nan"))) == binding.INT8MM_EINVAL
    assert f(*args(X=None)) == binding.INT8MM_EINVAL
    assert f(*args(ws=None)) == binding.INT8MM_EWORKSPACE
    assert f(*args(M=0)) == binding.INT8MM_OK
    # misaligned panel-tiled stage outputs (Xq, X_O, W_O: argument slots 10, 12, 13)
    for slot in (10, 12, 13):
        a = args()
        a[slot] = FAKE + 4
        assert f(*a) == binding.INT8MM_EINVAL


def test_prepare_weight_rejects_bad_arguments(lib):
    f = lib.int8_prepare_weight
    assert f(FAKE, -1, 8, FAKE, FAKE, None) == binding.INT8MM_ESHAPE
    assert f(FAKE, 4, -1, FAKE, FAKE, None) == binding.INT8MM_ESHAPE
    assert f(FAKE, 4, binding.INT8MM_MAX_K + 1, FAKE, FAKE, None) == binding.INT8MM_ESHAPE
    assert f(None, 4, 8, FAKE, FAKE, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 4, 8, None, FAKE, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 4, 8, FAKE, None, None) == binding.INT8MM_EINVAL
    assert f(FAKE, 4, 8, FAKE + 2, FAKE, None) == binding.INT8MM_EINVAL  # misaligned Wq
    assert f(FAKE, 0, 8, FAKE, FAKE, None) == binding.INT8MM_OK  # empty weight


def test_strerror(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.int8mm_strerror(st)
    assert lib.int8mm_strerror(12345) == b"unknown status"
    assert lib.int8mm_last_hip_error() == b""


def test_binding_raises_on_status(lib):
    with pytest.raises(binding.Int8mmError) as e:
        binding._check("int8_matmul", binding.INT8MM_ESHAPE)
    assert "invalid shape" in str(e.value)
