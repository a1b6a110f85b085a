"""The decode step under HIP graph capture: captured once, replayed several
times with eager work (new activations, the same step run eagerly) and
synchronisations between the replays; every replay must equal the eager
result bit for bit.  Covers a split-K shape, whose arrival counters are
re-armed by the kernels themselves (nothing in the captured work clears
memory)."""

import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import inputs
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (4, 512, 12288), (12, 2048, 1024), (24, 1024, 4096)])
def test_graph_replay_matches_eager(gpu_lib, M, N, K):
    say("graph replay", M, N, K)
    wq, ws = bfp8.quantize_weight(inputs.weights_bf16(N, K, workload=700 + M).cuda())
    x = inputs.activations(M, K, workload=700, stream=0).cuda()
    y8 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsq = bfp8.make_workspace(bfp8.OP_QUANT_GEMM_W8A8_BLK128, M, N, K)
    ws16 = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)

    def step():
        bfp8.bfp8_quant_gemm_w8a8_blk128(x, wq, ws, y8, wsq)
        bfp8.bfp8_gemm_w8a16_blk128(x, wq, ws, y16, ws16)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        x.copy_(inputs.activations(M, K, workload=701, stream=rep).cuda())
        ref8 = bfp8.quant_gemm_w8a8(x, wq, ws, out_dtype=torch.float32)
        ref16 = bfp8.gemm_w8a16(x, wq, ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y8.view(torch.int32), ref8.view(torch.int32)), f"replay {rep}: w8a8"
        assert torch.equal(y16.view(torch.int32), ref16.view(torch.int32)), f"replay {rep}: w8a16"
