"""The entry points under HIP graph capture (needs the GPU).

The library neither allocates, synchronises nor clears memory inside a call,
so a sequence of calls can be captured once and replayed. Here relu(A·B)
(bf16, planner's kernel), a transposed-operand call through the caller's
workspace and a row softmax are captured into one graph through torch, then
replayed several times with eager work and synchronisations in between;
every replay must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import datagen
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu


def test_capture_and_replay_matches_eager():
    M, N, K = 512, 768, 384
    a = torch.from_numpy(datagen.normal_f32(1601, M, K, K ** -0.5)).cuda().to(torch.bfloat16)
    b = torch.from_numpy(datagen.normal_f32(1602, K, N, K ** -0.5)).cuda().to(torch.bfloat16)
    at = a.t().contiguous()                           # A stored transposed for the strided call
    x = torch.from_numpy(datagen.normal_f32(1603, 256, 1000, 2.0)).cuda()
    c1 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    need = mm.mmrelu_strided_workspace_size(mm.DTYPE_BF16, mm.ACT_RELU, at.data_ptr(), b.data_ptr(), 0,
                                            c2.data_ptr(), M, N, K, 1, M, N, 1, N, 1)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    wp = (ws.data_ptr() + 255) // 256 * 256

    def work(stream):
        s = stream.cuda_stream
        assert mm.mmrelu_bf16(a.data_ptr(), b.data_ptr(), c1.data_ptr(), M, N, K, K, N, N, s) == mm.MMRELU_OK
        assert mm.mmrelu_strided_bf16(mm.ACT_RELU, at.data_ptr(), b.data_ptr(), 0, c2.data_ptr(), M, N, K, 1, M,
                                      N, 1, N, 1, wp, need, s) == mm.MMRELU_OK
        assert mm.mmrelu_softmax_rows_f32(x.data_ptr(), y.data_ptr(), 256, 1000, 1000, 1000, s) == mm.MMRELU_OK

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(side)                                    # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (c1, c2, y)]
    assert torch.equal(eager[0], eager[1])            # same product, two routes

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(torch.cuda.current_stream())
    for rep in range(4):
        for t in (c1, c2, y):
            t.fill_(float("nan"))                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((c1, c2, y), eager):
            assert torch.equal(got, want), f"replay {rep} differs from the eager result"
