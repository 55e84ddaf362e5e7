"""HIP graph capture of the hot path (GPU).

Every entry point only launches kernels on the caller's stream: no
allocation, no memset, no host synchronization, and the grouped forms read
their group ends from device memory.  So one training step's casts and its
consumer GEMM capture into a single graph, replayed with one call.  This
test captures forward and backward casts (both layouts), a grouped backward
cast and a GEMM on the forward's rowwise output, then replays the graph for
three input sets, clearing every output in between (eagerly, outside the
graph), and checks each replay bit for bit against the same calls made
eagerly on the same inputs.
"""
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda", 0)
    M, N, K2 = 4096, 2048, 512
    print(f"case: graph capture, {M}x{N} casts and a {M}x{K2}x{N} GEMM", flush=True)
    w13 = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev)
    dh = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gate, up = w13[:, :N], w13[:, N:]
    ends = torch.tensor([1000, 2048, 4096], dtype=torch.int32, device=dev)
    fo = mx.alloc_outputs(M, N, mx.BOTH, dev)
    bo = mx.alloc_outputs(M, 2 * N, mx.BOTH, dev)
    go = mx.alloc_outputs(M, 2 * N, mx.BOTH, dev, 3)
    qw, _, sw, _ = mx.mxfp8_quant_2d(synth.normal_bf16((K2, N), 0.02, seed=9, device=dev), rowwise=True)
    c = torch.empty((M, K2), dtype=torch.float32, device=dev)
    outs = [t for t in (*fo, *bo, *go, c) if t.numel()]

    def step():
        mx.mxfp8_swiglu_fwd(gate, up, rowwise=True, colwise=True, out=fo)
        mx.mxfp8_swiglu_bwd(dh, gate, up, rowwise=True, colwise=True, out=bo)
        mx.mxfp8_gated_bwd_grouped(dh, gate, up, ends, out=go)
        mx.mxfp8_gemm(fo[0], fo[2], qw, sw, out=c)

    def fill(seed):
        w13.copy_(synth.normal_bf16((M, 2 * N), 1.0, seed=seed, device=dev))
        dh.copy_(synth.normal_bf16((M, N), 1.0, seed=seed + 100, device=dev))

    def clear():
        for t in outs:
            t.zero_()

    fill(1)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()  # warm-up launch off the capturing stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for seed in (1, 2, 3):
        fill(seed)
        clear()
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        for _ in range(2):
            clear()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (got, want) in enumerate(zip(outs, ref)):
                assert torch.equal(got, want), f"output {i} differs on replay (seed {seed})"
        assert torch.isfinite(c).all() and c.abs().sum() > 0
