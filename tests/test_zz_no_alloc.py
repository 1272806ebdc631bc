"""The allocation-free entry point (int8_matmul_noalloc): through the C ABI,
its Y is bit-identical to int8_matmul's on the same inputs (the same
kernels, the workspace being the library's static buffer), on two calls in
a row with the second smaller than the first, on both the decode and the
tile-GEMM paths and the many-outlier form; a shape whose workspace exceeds
the buffer is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest

import workloads
from gpu_cases import to_dev

from int8_quantized_matmul_col_amd import binding


def test_oversized_shape_is_refused_on_the_host():
    lib = binding.load()
    cap = int(lib.int8_matmul_noalloc_max_workspace())
    assert cap == 64 << 20
    # 4096 x 4096 x 4096 needs ~80 MiB of workspace (outlier slices sized for |O| = K)
    assert int(lib.int8_matmul_workspace_size(4096, 4096, 4096)) > cap
    st = lib.int8_matmul_noalloc(None, 4096, 4096, None, None, 4096, 6.0, None, None)
    assert st == binding.INT8MM_ESCRATCH
    assert b"noalloc" in lib.int8mm_strerror(st)
    # a shape check still comes first
    assert lib.int8_matmul_noalloc(None, -1, 4, None, None, 4, 6.0, None, None) == binding.INT8MM_ESHAPE


def _pair(mm, M, K, N, n_out, t, seed):
    import torch
    X, _ = workloads.make_x(M, K, seed, n_out, 8.0, 60.0, "uniform")
    W = workloads.make_w(N, K, seed, 0.02)
    Xd, Wd = to_dev(X), to_dev(W)
    Wq, s = mm.int8_prepare_weight(Wd)
    lib = binding.load()
    stream = torch.cuda.current_stream().cuda_stream
    Y_ref = mm.int8_matmul(Xd, Wq, s, threshold=t)
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    st = lib.int8_matmul_noalloc(Xd.data_ptr(), M, K, Wq.data_ptr(), s.data_ptr(), N,
                                 ctypes.c_float(t), Y.data_ptr(), stream)
    assert st == 0, lib.int8mm_strerror(st)
    torch.cuda.synchronize()
    return Y, Y_ref


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    # tile GEMM (few tiles, each as two halves), then a smaller prefill call
    ((300, 2112, 520, 7, 6.0), (33, 64, 40, 2, 6.0)),
    # many outlier columns (t = 0: every column fp16), then few
    ((96, 320, 96, 4, 0.0), (40, 96, 72, 3, 6.0)),
    # decode, then a smaller decode
    ((16, 4096, 1024, 8, 6.0), (1, 1024, 64, 2, 6.0)),
])
def test_noalloc_matches_int8_matmul_twice(lib, first, second):
    for i, (M, K, N, n_out, t) in enumerate((first, second)):
        print(f"case noalloc call {i}: M={M} K={K} N={N} t={t}", flush=True)
        Y, Y_ref = _pair(lib, M, K, N, n_out, t, seed=M * 131 + K + N + i)
        assert np.array_equal(Y.cpu().numpy().view(np.uint16), Y_ref.cpu().numpy().view(np.uint16))


@pytest.mark.gpu
def test_noalloc_oversized_leaves_output_untouched(lib):
    import torch
    M = K = N = 4096
    Y = torch.zeros((4, 4), dtype=torch.float16, device="cuda")
    st = binding.load().int8_matmul_noalloc(1, M, K, 1, 1, N, ctypes.c_float(6.0),
                                            Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == binding.INT8MM_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y).item() == 0
