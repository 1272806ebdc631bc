"""GPU parity of the biased forward (int8_linear, the 8-bit linear layer) and
of the Int8Linear module against the CPU oracle, element by element."""

import math

import numpy as np
import pytest

import workloads
from gpu_cases import check_prepare, check_y, to_dev
from oracle import int8mm_ref as ref

pytestmark = pytest.mark.gpu


def _bias(N, seed, scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(N) * scale).astype(np.float16)


LINEAR_SHAPES = [
    # (M, K, N, n_out, t, bias scale)
    (1, 1000, 300, 2, 6.0, 0.5),        # decode kernel
    (16, 1024, 1024, 2, 6.0, 0.05),     # decode kernel, one row group per wave
    (5, 3, 7, 1, 0.0, 2.0),             # decode, every column an outlier
    (300, 520, 300, 5, 6.0, 0.5),       # prefill tiles with ragged edges
    (300, 2112, 520, 7, 6.0, 1.0),      # few tiles: each as two 256x128 halves
    (64, 130, 40, 2, 0.0, 0.5),         # many outlier steps (separate fp16 loop)
    (260, 2048, 300, 2, 0.0, 30.0),     # half-tile grid + many outlier steps, large bias
    (96, 320, 96, 4, math.inf, 0.5),    # pure int8
]


@pytest.mark.parametrize("M,K,N,n_out,t,bscale", LINEAR_SHAPES)
def test_linear_parity(lib, M, K, N, n_out, t, bscale):
    print(f"case int8_linear M={M} K={K} N={N} n_out={n_out} t={t} bias={bscale}", flush=True)
    import torch
    seed = M * 7919 + K * 31 + N + 5
    X, _ = workloads.make_x(M, K, seed, n_out, 8.0, 60.0, "uniform")
    W = workloads.make_w(N, K, seed, 0.02)
    b = _bias(N, seed, bscale)
    Wq_d, s_d, Wq_r, s_r = check_prepare(lib, W)
    X_d, b_d = to_dev(X), to_dev(b)
    Y = lib.int8_linear(X_d, Wq_d, s_d, b_d, threshold=t)
    Y0 = lib.int8_matmul(X_d, Wq_d, s_d, threshold=t)
    Yn = lib.int8_linear(X_d, Wq_d, s_d, None, threshold=t)
    torch.cuda.synchronize()
    Y_ref, st = ref.int8_matmul_ref(X, Wq_r, s_r, t, stages=True, bias=b)
    check_y(Y.cpu().numpy(), Y_ref, X, Wq_r, s_r, st["O"].size, bias=b)
    # without a bias the call is int8_matmul, bit for bit
    assert np.array_equal(Yn.cpu().numpy().view(np.uint16), Y0.cpu().numpy().view(np.uint16))


def test_linear_empty_contraction_gives_bias_rows(lib):
    import torch
    for M in (3, 40):  # decode and prefill sizes
        X = torch.empty((M, 0), dtype=torch.float16, device="cuda")
        W = torch.empty((5, 0), dtype=torch.float16, device="cuda")
        Wq, ws = lib.int8_prepare_weight(W)
        b = to_dev(np.array([1.5, -2.0, 0.0, 65504.0, -0.25], np.float16))
        Y = lib.int8_linear(X, Wq, ws, b)
        Y0 = lib.int8_linear(X, Wq, ws, None)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy(), np.tile(b.cpu().numpy(), (M, 1)))
        assert not Y0.cpu().numpy().any()


def test_linear_rejects_bad_bias(lib):
    import torch
    X = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    Wq, ws = lib.int8_prepare_weight(torch.zeros((8, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        lib.int8_linear(X, Wq, ws, torch.zeros(7, dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        lib.int8_linear(X, Wq, ws, torch.zeros(8, dtype=torch.float32, device="cuda"))


def test_int8linear_module_matches_oracle(lib):
    import torch
    M0, M1, K, N = 3, 70, 520, 300
    seed = 4242
    X, _ = workloads.make_x(M0 * M1, K, seed, 3, 8.0, 60.0, "uniform")
    W = workloads.make_w(N, K, seed, 0.02)
    b = _bias(N, seed, 0.5)
    lin = torch.nn.Linear(K, N, bias=True).to(device="cuda", dtype=torch.float16)
    with torch.no_grad():
        lin.weight.copy_(to_dev(W))
        lin.bias.copy_(to_dev(b))
    m = lib.Int8Linear.from_linear(lin, threshold=6.0)
    assert not m.quantized and m.weight is not None
    x = to_dev(X).reshape(M0, M1, K)
    y = m(x)
    torch.cuda.synchronize()
    assert m.quantized and m.weight is None  # the fp16 weight is dropped
    assert y.shape == (M0, M1, N) and y.dtype == torch.float16
    Wq_r, s_r = ref.prepare_weight_ref(W)
    assert np.array_equal(lib.unpack_weight(m.Wq, N, K).cpu().numpy(), Wq_r)
    assert np.array_equal(m.w_scale.cpu().numpy(), s_r)
    Y_ref, st = ref.int8_matmul_ref(X, Wq_r, s_r, 6.0, stages=True, bias=b)
    check_y(y.reshape(M0 * M1, N).cpu().numpy(), Y_ref, X, Wq_r, s_r, st["O"].size, bias=b)
    # a second call reuses the prepared weight and gives the same bits
    y2 = m(x)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16))
    # the prepared layer's state dict loads into a fresh layer as it is
    m3 = lib.Int8Linear(K, N, bias=True, threshold=6.0, device="cuda")
    m3.load_state_dict(m.state_dict())
    y3 = m3(x)
    torch.cuda.synchronize()
    assert m3.quantized and m3.weight is None
    assert np.array_equal(y3.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16))


def test_replace_linear_with_int8_runs(lib):
    import torch
    torch.manual_seed(0)
    net = torch.nn.Sequential()
    net.add_module("up", torch.nn.Linear(512, 1024))
    net.add_module("act", torch.nn.ReLU())
    net.add_module("down", torch.nn.Linear(1024, 512, bias=False))
    net.add_module("lm_head", torch.nn.Linear(512, 64))
    net = net.to(device="cuda", dtype=torch.float16)
    lib.replace_linear_with_int8(net, threshold=6.0, min_in_features=0, skip_modules=("lm_head",))
    assert isinstance(net.up, lib.Int8Linear) and isinstance(net.down, lib.Int8Linear)
    assert isinstance(net.lm_head, torch.nn.Linear) and not isinstance(net.lm_head, lib.Int8Linear)
    x = (torch.randn(2, 33, 512, device="cuda") * 0.5).to(torch.float16)
    y = net(x)
    torch.cuda.synchronize()
    assert y.shape == (2, 33, 64) and torch.isfinite(y).all()
    assert net.up.quantized and net.down.quantized
