"""Replays of a captured HIP graph of library calls give the eager results.

The short kernels (tall-skinny, decode, the dequant passes) are timed from
graph replays, so their calls are captured here in one graph together with a
split-K GEMM and a split decode (each finished by a fixup kernel) and
replayed three times.  Before
each replay the inputs are rewritten by eager work on the same stream; every
replay's outputs must equal, bit for bit, an eager run of the same calls on
the same inputs (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.float16).cuda()


def test_graph_replays_match_eager():
    # tall-skinny with bias + GELU
    X = _rand((4096, 160), 1, 0.08)
    W = _rand((160, 32), 2, 0.08)
    bias = _rand((32,), 3, 0.1)
    # decode: 4 rows against a 1024 x 1024 weight
    Xd = _rand((4, 1024), 4)
    Wd = _rand((1024, 1024), 5, 0.03)
    # split decode: 48 rows against a 512 x 4096 weight
    Xs = _rand((48, 4096), 8)
    Ws = _rand((512, 4096), 9, 0.02)
    ws_dec = torch.empty(dge.gemm_workspace_size(48, 512, 4096, torch.float16) // 4 + 1,
                         dtype=torch.float32, device="cuda")
    # split-K GEMM: 256 x 512 x 4096 (few tiles, so the schedule splits K)
    A = _rand((256, 4096), 6, 0.02)
    B = _rand((4096, 512), 7, 0.02)
    ws = torch.empty(dge.gemm_workspace_size_splits(256, 512, 4) // 4, dtype=torch.float32,
                     device="cuda")
    # dequant passes
    q6 = torch.from_numpy(inputs.kquant_weights("q6_k", 64, 1024, 7, 20)).cuda()
    q4 = torch.from_numpy(inputs.q4_weights(64, 1024, 4, 21)).cuda()

    def calls(outs):
        dge.gemm_f16(X, W, outs[0], epi="bias_gelu", bias=bias)
        dge.gemm_f16(Xd, Wd, outs[1], trans_b=True)
        dge.gemm_ex(A, B, outs[2], workspace=ws, algo="mfma", splits=4)
        dge.dequant_f16("q6_k", q6, 64, 1024, out=outs[3])
        dge.dequant_q4_f16(q4, 64, 1024, out=outs[4])
        dge.gemm_f16(Xs, Ws, outs[5], trans_b=True, workspace=ws_dec)

    def buffers():
        return [torch.empty((4096, 32), dtype=torch.float16, device="cuda"),
                torch.empty((4, 1024), dtype=torch.float16, device="cuda"),
                torch.empty((256, 512), dtype=torch.float16, device="cuda"),
                torch.empty((64, 1024), dtype=torch.float16, device="cuda"),
                torch.empty((64, 1024), dtype=torch.float16, device="cuda"),
                torch.empty((48, 512), dtype=torch.float16, device="cuda")]

    graph_out, eager_out = buffers(), buffers()
    calls(graph_out)  # first calls outside the capture (device setup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(graph_out)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: new inputs for every call
        X.copy_(_rand((4096, 160), 100 + rep, 0.08))
        Xd.copy_(_rand((4, 1024), 110 + rep))
        A.copy_(_rand((256, 4096), 120 + rep, 0.02))
        q6.copy_(torch.from_numpy(inputs.kquant_weights("q6_k", 64, 1024, 7, 30 + rep)).cuda())
        q4.copy_(torch.from_numpy(inputs.q4_weights(64, 1024, 4, 40 + rep)).cuda())
        Xs.copy_(_rand((48, 4096), 130 + rep))
        for t in graph_out:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        calls(eager_out)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(graph_out, eager_out)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
                "replay %d, call %d differs from the eager run" % (rep, i)
    del g
