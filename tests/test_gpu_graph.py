"""The library enqueues everything on the caller's stream, allocates
nothing and never synchronizes, so a call can be captured in a HIP graph and
replayed.  Each case captures one call (prefill and decode shapes, with and
without a bias), then replays it several times with new activations copied
in eagerly between replays, and checks every replay bit for bit against an
eager call on the same inputs.  Calls on two streams with their own
workspaces run concurrently and give the single-stream results."""

import numpy as np
import pytest

import workloads
from gpu_cases import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,with_bias", [(300, 1024, 512, False), (300, 1024, 512, True),
                                             (300, 2112, 520, True),  # every tile as two halves
                                             (8, 2048, 1024, False), (8, 2048, 1024, True),
                                             # one row: the decode kernel codes X itself
                                             (1, 2048, 1024, False), (1, 2048, 1024, True)])
def test_graph_replay_matches_eager(lib, M, K, N, with_bias):
    import torch
    print(f"case graph M={M} K={K} N={N} bias={with_bias}", flush=True)
    W = workloads.make_w(N, K, 900 + M, 0.02)
    Wq, s = lib.int8_prepare_weight(to_dev(W))
    b = to_dev((np.linspace(-1, 1, N)).astype(np.float16)) if with_bias else None
    xs = [to_dev(workloads.make_x(M, K, 1000 + M + i, 3, 8.0, 60.0, "uniform")[0])
          for i in range(3)]
    X = torch.empty_like(xs[0])
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = lib.workspace_for(M, K, N, X.device)
    torch.cuda.synchronize()

    def call():
        lib.int8_linear(X, Wq, s, b, threshold=6.0, out=Y, workspace=ws)

    X.copy_(xs[0])
    side = torch.cuda.Stream()  # capture off the default stream
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(2):
        for x in xs:
            X.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            got = Y.clone()
            Ye = lib.int8_linear(x, Wq, s, b, threshold=6.0)  # eager, own buffers
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), Ye.view(torch.int16)), (rep, M)


def test_concurrent_calls_on_two_streams(lib):
    # no global mutable state: calls on two streams with their own workspaces
    # overlap freely and each gives the eager single-stream result
    import torch
    print("case two streams", flush=True)
    cases = []
    for i, (M, K, N) in enumerate([(300, 2112, 520), (8, 2048, 1024)]):
        W = workloads.make_w(N, K, 700 + i, 0.02)
        Wq, s = lib.int8_prepare_weight(to_dev(W))
        X = to_dev(workloads.make_x(M, K, 800 + i, 4, 8.0, 60.0, "uniform")[0])
        ref_y = lib.int8_matmul(X, Wq, s, threshold=6.0)
        cases.append((X, Wq, s, ref_y, lib.workspace_for(M, K, N, X.device),
                      torch.empty((M, N), dtype=torch.float16, device="cuda")))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for _ in range(5):
        for (X, Wq, s, _, ws, Y), st in zip(cases, streams):
            with torch.cuda.stream(st):
                lib.int8_matmul(X, Wq, s, threshold=6.0, out=Y, workspace=ws)
    torch.cuda.synchronize()
    for X, Wq, s, ref_y, ws, Y in cases:
        assert torch.equal(Y.view(torch.int16), ref_y.view(torch.int16))
