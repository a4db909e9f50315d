"""fused_moe_wna16_noalloc (the layer on the library's static device scratch, for callers that
cannot allocate) against fused_moe_wna16 with a caller-allocated workspace, through the C ABI.

Both run the same kernels, so the outputs must agree bit for bit; the tiny layer is also checked
against the oracle.  Two calls in a row, the second with a smaller batch (the scratch keeps the
first call's contents), and a captured graph replayed with eager work in between."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import assert_layer_close, cuda_layer, oracle_route, routing_of

pytestmark = pytest.mark.gpu


def _args(wl, layer):
    return (routing_of(wl), layer["w13"], layer["w13_scales"], layer["w13_zeros"], layer["w2"],
            layer["w2_scales"], layer["w2_zeros"])


def _both(wl, layer, x, lg):
    M = x.shape[0]
    rt, *w = _args(wl, layer)
    ref = B.fused_moe_wna16(x, lg, wl.topk, rt, *w)                       # workspace entry point
    out = torch.full((M, wl.H), float("nan"), dtype=wl.torch_dtype, device="cuda")
    ti = torch.full((M, wl.topk), -7, dtype=torch.int32, device="cuda")
    tw = torch.full((M, wl.topk), -1.0, dtype=torch.float32, device="cuda")
    B.fused_moe_wna16_noalloc(x, lg, wl.topk, rt, *w, out=out, topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    return ref, out, tw, ti


@pytest.mark.parametrize("name,Ms", [("tiny", (16, 5)), ("mixtral", (64, 4)), ("dsv3_tp8", (64, 1))])
def test_noalloc_matches_workspace_entry_point(name, Ms):
    wl = synth.WORKLOADS[name]
    dev = "cpu" if name == "tiny" else "cuda"
    layer = synth.make_layer(wl, seed=2, device=dev)
    lay = cuda_layer(layer) if dev == "cpu" else layer
    for M in Ms:                                        # the second call is the smaller batch
        print(f"noalloc {name} M={M}", flush=True)
        x = synth.make_x(wl, M, seed=2, device=dev).cuda()
        lg = synth.make_logits(wl, M, seed=2, device=dev).cuda()
        ref, out, tw, ti = _both(wl, lay, x, lg)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name} M={M}"
        ids_ref, w_ref = oracle_route(wl, lg)
        assert np.array_equal(O.to_numpy(ti), ids_ref)
        if name == "tiny":
            want = O.moe_layer(x.cpu(), ids_ref, w_ref, O.ExpertSource(layer, wl.bits))
            assert_layer_close(out, want, f"noalloc tiny M={M}")


def test_noalloc_graph_replay():
    """Captured once, replayed three times with eager layer calls (which reuse the same scratch)
    between the replays; every replay equals the workspace entry point bit for bit."""
    wl = synth.WORKLOADS["tiny"]
    lay = cuda_layer(synth.make_layer(wl, seed=1))
    x = synth.make_x(wl, 16, seed=1).cuda()
    lg = synth.make_logits(wl, 16, seed=1).cuda()
    x2 = synth.make_x(wl, 7, seed=9).cuda()
    lg2 = synth.make_logits(wl, 7, seed=9).cuda()
    rt, *w = _args(wl, lay)
    ref = B.fused_moe_wna16(x, lg, wl.topk, rt, *w)
    out = torch.empty_like(ref)
    B.fused_moe_wna16_noalloc(x, lg, wl.topk, rt, *w, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fused_moe_wna16_noalloc(x, lg, wl.topk, rt, *w, out=out)
    other = torch.empty((7, wl.H), dtype=wl.torch_dtype, device="cuda")
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        B.fused_moe_wna16_noalloc(x2, lg2, wl.topk, rt, *w, out=other)   # eager, same scratch
        torch.cuda.synchronize()


def test_noalloc_refuses_batches_beyond_the_scratch():
    """A batch whose workspace exceeds the static scratch is refused before any launch."""
    wl = synth.WORKLOADS["tiny"]
    M = 8192
    need = B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, wl.E, wl.topk, B.QUANT_INT4,
                                            wl.torch_dtype, 0)
    assert need > B.NOALLOC_SCRATCH_BYTES
    lay = cuda_layer(synth.make_layer(wl, seed=0))
    x = torch.zeros((M, wl.H), dtype=wl.torch_dtype, device="cuda")
    lg = torch.zeros((M, wl.E), dtype=torch.float32, device="cuda")
    out = torch.empty((M, wl.H), dtype=wl.torch_dtype, device="cuda")
    rt, *w = _args(wl, lay)
    with pytest.raises(B.MoeError) as ei:
        B.fused_moe_wna16_noalloc(x, lg, wl.topk, rt, *w, out=out)
    assert ei.value.status == -4 and "static scratch" in str(ei.value)
