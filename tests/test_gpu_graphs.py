"""Graph capture of the entry points beside the main layer: each is captured once into a HIP graph,
replayed several times with other eager work and synchronisation in between, and every replay must
equal the eager result bit for bit (no launch reads host state or leaves state for the next)."""
import numpy as np
import pytest
import torch

import synth
import weight_only_int4_topk_amd as B
from helpers import cuda_layer, routing_of

pytestmark = pytest.mark.gpu


def _replays(run, out, eager_between, n=3):
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(n):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        eager_between()
        torch.cuda.synchronize()


def test_dense_gemm_graph_replay():
    """Split over K into float32 partials plus the reduce launch (n = 4096 at k = 8192)."""
    d = {k: (v.cuda() if v is not None else None)
         for k, v in synth.make_dense(16, 4096, 8192, 4, "fp16", seed=1).items()}
    need = B.moe_wna16_dense_gemm_workspace_size(16, 4096, 8192, B.QUANT_INT4, torch.float16)
    assert need > 0
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    C = torch.empty((16, 4096), dtype=torch.float16, device="cuda")
    run = lambda: B.moe_wna16_dense_gemm(d["A"], d["B"], d["scales"], d["zeros"], workspace=ws, C=C)
    _replays(run, C, lambda: B.moe_wna16_dense_gemm(d["A"], d["B"], d["scales"], d["zeros"]))


def test_batched_gemm_graph_replay():
    wl = synth.Workload("b", E=4, H=512, I=256, topk=1, Ms=(1,), bits=4)
    lay = cuda_layer(synth.make_layer(wl, seed=2))
    A = (torch.randn((4, 24, 512), device="cuda") * 0.1).half()
    cnt = torch.tensor([24, 0, 9, 17], dtype=torch.int32, device="cuda")
    C = torch.zeros((4, 24, 256), dtype=torch.float16, device="cuda")
    run = lambda: B.moe_wna16_batched_gemm(A, cnt, lay["w13"], lay["w13_scales"], lay["w13_zeros"],
                                           act=1, C=C)
    # rows past each count are never written: compare only the rows that are
    mask = torch.arange(24, device="cuda")[None, :] < cnt[:, None]
    run()
    torch.cuda.synchronize()
    ref = C[mask].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        C.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C[mask].view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        B.moe_wna16_batched_gemm(A, cnt, lay["w13"], lay["w13_scales"], lay["w13_zeros"], act=0)


def test_fused_w8a8_graph_replay():
    wl = synth.Workload("w", E=8, H=512, I=512, topk=2, Ms=(20,), dtype="bf16", bits=8)
    lay = cuda_layer(synth.make_layer(wl, seed=3))
    x = synth.make_x(wl, 20, seed=3).cuda()
    lg = synth.make_logits(wl, 20, seed=3).cuda()
    need = int(B.lib().fused_moe_w8a8_workspace_size(20, 512, 512, 8, 2, 1, 0))
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    out = torch.empty((20, 512), dtype=torch.bfloat16, device="cuda")
    args = (x, lg, 2, routing_of(wl), lay["w13"], lay["w13_scales"], lay["w2"], lay["w2_scales"])
    run = lambda: B.fused_moe_w8a8(*args, workspace=ws, out=out)
    _replays(run, out, lambda: B.fused_moe_w8a8(*args))


def test_fused_act_order_graph_replay():
    """M = 3: routing and align in one launch, the first GEMM split over K into partials, two
    gathers; every launch of the layer inside the graph."""
    wl = synth.Workload("a", E=8, H=1792, I=768, topk=2, Ms=(3,))
    lay = {k: v.cuda() for k, v in synth.make_layer_act_order(wl, seed=4).items()}
    x = synth.make_x(wl, 3, seed=4).cuda()
    lg = synth.make_logits(wl, 3, seed=4).cuda()
    need = int(B.lib().fused_moe_wna16_act_order_workspace_size(3, 1792, 768, 8, 2, 0, 0))
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    out = torch.empty((3, 1792), dtype=torch.float16, device="cuda")
    args = (x, lg, 2, routing_of(wl), lay["w13"], lay["w13_scales"], lay["w13_zeros"],
            lay["w13_perm"], lay["w2"], lay["w2_scales"], lay["w2_zeros"], lay["w2_perm"])
    run = lambda: B.fused_moe_wna16_act_order(*args, workspace=ws, out=out)
    _replays(run, out, lambda: B.fused_moe_wna16_act_order(*args))
