"""The run calls under HIP graph capture.

Every run call only enqueues kernels on the caller's stream: no allocation,
no synchronisation, no memset.  So a sequence of them can be captured once
and replayed.  The sequence here covers four paths:
- the ping-pong kernel (which sets its 160 KiB LDS attribute at launch);
- the panel kernel;
- the tile kernel;
- split-K (a batched product plus the reduction).

It is captured with torch's graph API on a capture stream and replayed
several times.  Between replays, eager work on the same buffers clears the
outputs.  Every replay must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import synth
from parity import to_gpu

pytestmark = pytest.mark.gpu


def test_captured_run_calls_replay_like_eager_calls():
    rng = np.random.default_rng(31)
    dev = "cuda"
    # ping-pong: 4096 x 4096 x 1024 (256 work items of 256 x 256)
    A1 = to_gpu(synth.draw(rng, (4096, 1024), "normal", 1.0))
    B1 = to_gpu(synth.draw(rng, (1024, 4096), "normal", 1.0))
    C1 = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    p1 = tg.plan(4096, 4096, 1024, out_dtype=torch.bfloat16)
    assert p1.tile == tg.TILE_PINGPONG
    # panel kernel, forced: 8 score-like products 512 x 2048 x 128, B stored N x K
    A2 = to_gpu(synth.draw(rng, (8, 512, 128), "normal", 1.0))
    B2 = to_gpu(synth.draw(rng, (8, 2048, 128), "normal", 1.0))
    C2 = torch.empty((8, 512, 2048), dtype=torch.float32, device=dev)
    p2 = tg.plan_tile(tg.plan(512, 2048, 128, trans_b=True, batch=8), tg.VARIANT_TILE, tg.TILE_PANEL)
    # tile kernel: 1000^3 with every transpose's A read as stored K x M
    A3 = to_gpu(synth.draw(rng, (1000, 1000), "uniform", -1.0, 1.0))
    B3 = to_gpu(synth.draw(rng, (1000, 1000), "uniform", -1.0, 1.0))
    C3 = torch.empty((1000, 1000), dtype=torch.float32, device=dev)
    p3 = tg.plan(1000, 1000, 1000, trans_a=True)
    # split-K: 256 x 256 x 16384 in 8 parts
    A4 = to_gpu(synth.draw(rng, (256, 16384), "normal", 1.0))
    B4 = to_gpu(synth.draw(rng, (16384, 256), "normal", 1.0))
    C4 = torch.empty((256, 256), dtype=torch.float32, device=dev)
    p4 = tg.plan(256, 256, 16384)
    need = tg.splitk_workspace_bytes(p4, 8)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    outs = (C1, C2, C3, C4)

    def run():
        tg.gemm_run(p1, A1, B1, C1)
        tg.bmm_run(p2, 8, 512 * 128, 2048 * 128, 512 * 2048, A2, B2, C2)
        tg.gemm_run(p3, A3, B3, C3)
        tg.gemm_splitk_run(p4, 8, ws, need, A4, B4, C4)

    run()
    torch.cuda.synchronize()
    eager = [c.clone() for c in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for r in range(3):
        for c in outs:
            c.zero_()  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(outs, eager)):
            assert torch.equal(c, e), f"replay {r}: output {i} differs from the eager run"
