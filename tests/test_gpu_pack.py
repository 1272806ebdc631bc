"""int8_pack_weight: an already-quantized weight (int8 codes [N][K] plus one
scale per output channel, the stored form of "PyTorch 2.9 supports
LLM.int8()", section 1) into the library's prepared layout.  Checked byte by
byte against the codes (clamped to [-127, 127], zero padding), against
int8_prepare_weight's own output for the same codes, and end to end: the
decode workload with a pre-quantized 28672 x 8192 weight and fp32
per-channel scales from the oracle, through int8_matmul, against the
oracle."""

import numpy as np
import pytest
import torch

import workloads
from gpu_cases import check_y, run_stages, to_dev
from oracle import int8mm_ref as ref

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 1), (37, 257), (300, 1000), (257, 64), (16, 4096), (5, 17)])
def test_pack_layout_clamp_and_padding(lib, N, K):
    print(f"case pack N={N} K={K}", flush=True)
    rng = np.random.default_rng(N * 1000 + K)
    codes = rng.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    codes[0, 0] = -128
    Wq = lib.int8_pack_weight(to_dev(codes))
    torch.cuda.synchronize()
    t = lib.untile(Wq, Wq.shape[0]).cpu().numpy()
    assert Wq.numel() == lib.int8_weight_bytes(N, K)
    assert np.array_equal(t[:N, :K], np.clip(codes, -127, 127))
    assert not t[:N, K:].any(), "padding columns"
    assert not t[N:].any(), "padding rows"


@pytest.mark.parametrize("N,K", [(300, 1000), (520, 4096)])
def test_pack_of_prepared_codes_is_byte_identical(lib, N, K):
    W = workloads.make_w(N, K, N + K, 0.02)
    Wq_a, s = lib.int8_prepare_weight(to_dev(W))
    codes = lib.unpack_weight(Wq_a, N, K).contiguous()
    Wq_b = lib.int8_pack_weight(codes)
    torch.cuda.synchronize()
    assert torch.equal(Wq_a, Wq_b)
    # and the matmul through the packed weight is the same call
    X, _ = workloads.make_x(64, K, N, 3, 8.0, 60.0, "uniform")
    Xd = to_dev(X)
    Ya = lib.int8_matmul(Xd, Wq_a, s)
    Yb = lib.int8_matmul(Xd, Wq_b, s)
    torch.cuda.synchronize()
    assert torch.equal(Ya.view(torch.int16), Yb.view(torch.int16))


@pytest.mark.slow
def test_decode_with_prequantized_weight(lib):
    # the decode workload as stated: a pre-quantized int8 weight 28672 x 8192
    # with fp32 per-channel scales (here the oracle's quantization of the
    # workload's W), X of 16 rows with 8 outlier columns, threshold 6.0
    case = workloads.config_case("decode16")
    Wq_r, s_r = ref.prepare_weight_ref(case.W)
    Wq = lib.int8_pack_weight(to_dev(Wq_r))
    s = to_dev(s_r.astype(np.float32))
    Y_ref, st, X_d = run_stages(lib, case.X, Wq, s, case.threshold, Wq_r, s_r)
    Y = lib.int8_matmul(X_d, Wq, s, threshold=case.threshold)
    torch.cuda.synchronize()
    check_y(Y.cpu().numpy(), Y_ref, case.X, Wq_r, s_r, st["O"].size)
