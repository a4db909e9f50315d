"""The dot-product paths of the layer (uint4, block_m left to the library).  One token: one dot
product per weight row in two launches (routing inside the first, SiLU(gate) * up; the second
product with the top-k combine).  A few tokens (2 to 4, I <= 512): routing, then the same two
launches with the slots grouped by expert in every workgroup.  Against the oracle, every element, with the tolerance of the
other layer tests; the shapes cover each groups-per-lane variant of the launches, quantisation
groups that do not fill a wavefront, one expert taking every token, and the fallback to the grouped
GEMMs where the staged activations exceed LDS."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from tests.helpers import (assert_layer_close, assert_weights_close, cuda_layer, fused_vs_oracle,
                           oracle_route, routing_of, run_fused)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

CASES = {
    "tiny_fp16": W["tiny"].with_(block_m=0),
    "tiny_bf16": W["tiny"].with_(block_m=0, dtype="bf16"),
    "sigmoid_groups_bf16": synth.Workload("sg1", E=64, H=512, I=256, topk=8, Ms=(1,), dtype="bf16",
                                          score="sigmoid", num_groups=8, topk_groups=4, scale=2.5),
    "softmax_bias": synth.Workload("sb1", E=64, H=768, I=512, topk=8, Ms=(1,), logit_bias=True),
    "no_renorm": synth.Workload("nr1", E=32, H=512, I=256, topk=4, Ms=(1,), renormalize=False),
    "one_expert": synth.Workload("d11", E=1, H=512, I=512, topk=1, Ms=(1,)),
    "all_experts": synth.Workload("ae1", E=4, H=256, I=256, topk=4, Ms=(1,)),
    "topk3": synth.Workload("k31", E=16, H=1024, I=768, topk=3, Ms=(1,), dtype="bf16"),
    # 14 and 10 groups per row: lanes without a group in both launches
    "odd_groups_fp16": synth.Workload("og1", E=16, H=1792, I=1280, topk=4, Ms=(1,)),
    "odd_groups_bf16": synth.Workload("og2", E=16, H=1792, I=1280, topk=4, Ms=(1,), dtype="bf16"),
    # 96 groups per first-launch row over 32 lanes: four steps of one group per lane, the last empty
    "wide_h": synth.Workload("wh1", E=4, H=12288, I=512, topk=2, Ms=(1,), dtype="bf16"),
    # 256 groups per first-launch row over 32 lanes: eight steps
    "widest_h": synth.Workload("wh2", E=2, H=32768, I=256, topk=1, Ms=(1,)),
    # 66 and 112 groups per second-launch row over 64 lanes: two steps of one group per lane, the
    # second step partly empty with 66
    "two_steps_ragged_i": synth.Workload("ti1", E=8, H=512, I=8448, topk=2, Ms=(1,)),
    "two_steps_i_bf16": synth.Workload("ti2", E=8, H=256, I=14336, topk=2, Ms=(1,), dtype="bf16"),
    # 256 groups per second-launch row over 64 lanes: four steps of one group per lane; with
    # topk 2 the staged intermediate rows take 128 KiB of LDS
    "widest_i": synth.Workload("wi1", E=2, H=256, I=32768, topk=2, Ms=(1,), dtype="bf16"),
    # the same with topk 4 exceeds LDS: the grouped GEMMs run instead
    "widest_i_fallback": synth.Workload("wi2", E=4, H=256, I=32768, topk=4, Ms=(1,)),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("seed", [0, 1])
def test_single_token_vs_oracle(name, seed):
    wl = CASES[name]
    want = B.PATH_GROUPED if name == "widest_i_fallback" else B.PATH_ONE_TOKEN
    assert B.fused_moe_wna16_path(1, wl.H, wl.I, wl.E, wl.topk) == want
    print(f"single token {name} seed={seed}", flush=True)
    fused_vs_oracle(wl, 1, seed=seed)


@pytest.mark.parametrize("name", ["tiny_fp16", "sigmoid_groups_bf16", "odd_groups_fp16"])
def test_single_token_grouped_gemm_path(name):
    """An explicit block_m keeps one token on the grouped GEMMs: both paths against the oracle."""
    fused_vs_oracle(CASES[name], 1, seed=3, block_m=16)


ROUTINGS = [("softmax", 64, 6, 1, 1), ("softmax", 60, 4, 1, 1), ("softmax", 8, 2, 1, 1),
            ("sigmoid", 96, 5, 6, 3), ("sigmoid", 256, 8, 8, 4), ("sigmoid", 8, 8, 1, 1),
            ("sigmoid", 64, 32, 64, 40), ("sigmoid", 20, 3, 1, 1)]


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("score,E,k,ng,tg", ROUTINGS)
@pytest.mark.parametrize("logits", ["normal", "ties", "neg_inf"])
def test_single_token_routing(score, E, k, ng, tg, renorm, logits):
    """The first launch routes the token itself: ids bit for bit and weights as the oracle's, for
    each rule, with ties (logits on a grid of 0.5, equal values go to the lower id) and with -inf
    logits (a quarter of the experts), and the layer output with them."""
    wl = synth.Workload("r1", E=E, H=256, I=256, topk=k, Ms=(1,), score=score,
                        renormalize=bool(renorm), num_groups=ng, topk_groups=tg, scale=1.5)
    layer = synth.make_layer(wl, seed=5)
    x = synth.make_x(wl, 1, seed=5)
    lg = synth.make_logits(wl, 1, seed=5)
    if logits == "ties":
        lg = torch.round(lg * 2) / 2
    elif logits == "neg_inf":
        lg[0, 1::4] = -float("inf")
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), cuda_layer(layer))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    assert_weights_close(tw, w_ref)
    ref = O.moe_layer(x, ids_ref, w_ref, O.ExpertSource(layer, 4))
    assert_layer_close(out, ref, f"one token, {score} E={E} topk={k}")


def test_single_token_zero_activations_give_zero():
    """x = 0: every group's dot product and activation sum are exactly zero, so is the output."""
    wl = CASES["odd_groups_bf16"]
    layer = cuda_layer(synth.make_layer(wl, seed=2))
    x = torch.zeros((1, wl.H), dtype=wl.torch_dtype, device="cuda")
    lg = synth.make_logits(wl, 1, seed=2).cuda()
    out, _, _ = run_fused(wl, x, lg, layer)
    assert (out.float() == 0).all()


def test_single_token_fp16_tiny_activations():
    """fp16 activations of order 2e-5 (many subnormal) against weights N(0, 5^2): the dot products
    take the activations as they are, so the output matches the oracle to the usual tolerance
    relative to its largest element."""
    wl = synth.Workload("ta1", E=4, H=512, I=512, topk=2, Ms=(1,), x_std=2e-5, w_std=5.0)
    layer = synth.make_layer(wl, seed=3)
    x = synth.make_x(wl, 1, seed=3)
    lg = synth.make_logits(wl, 1, seed=3)
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), cuda_layer(layer))
    ids_ref, w_ref = oracle_route(wl, lg)
    ref = O.moe_layer(x, ids_ref, w_ref, O.ExpertSource(layer, 4))
    sc = 1.0 / np.abs(ref).max()
    assert_layer_close(O.to_numpy(out).astype(np.float64) * sc, np.asarray(ref) * sc,
                       "tiny activations, one token")


# one step per lane in both launches; two steps of the second launch; four of the first
@pytest.mark.parametrize("name", ["sigmoid_groups_bf16", "two_steps_i_bf16", "wide_h"])
def test_single_token_deterministic_and_graph_replay(name):
    wl = CASES[name]
    layer = cuda_layer(synth.make_layer(wl, seed=1))
    x = synth.make_x(wl, 1, seed=1).cuda()
    lg = synth.make_logits(wl, 1, seed=1).cuda()
    out1, _, _ = run_fused(wl, x, lg, layer)
    out2, _, _ = run_fused(wl, x, lg, layer)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    ws = torch.empty((B.fused_moe_wna16_workspace_size(1, wl.H, wl.I, wl.E, wl.topk, B.QUANT_INT4,
                                                       wl.torch_dtype, 0),), dtype=torch.uint8,
                     device="cuda")
    gout = torch.empty_like(out1)
    run = lambda: B.fused_moe_wna16(x, lg, wl.topk, routing_of(wl), layer["w13"],
                                    layer["w13_scales"], layer["w13_zeros"], layer["w2"],
                                    layer["w2_scales"], layer["w2_zeros"], block_m=0,
                                    workspace=ws, out=gout)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        gout.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout.view(torch.int16), out1.view(torch.int16)), f"replay {i}"
        run_fused(wl, x, lg, layer)  # eager work between replays


# ------------------------------------------------------------------------------------------------
# a few tokens
# ------------------------------------------------------------------------------------------------
FEW = {
    # many experts, narrow I (a tensor-parallel share): 32 slots over 64 experts
    "tp_like_fp16": synth.Workload("f1", E=64, H=1024, I=256, topk=8, Ms=(4,), score="sigmoid",
                                   num_groups=8, topk_groups=4, scale=2.5),
    "tp_like_bf16": synth.Workload("f2", E=64, H=1024, I=256, topk=8, Ms=(3,), dtype="bf16",
                                   score="sigmoid", num_groups=8, topk_groups=4, scale=2.5),
    # 14 groups per first-launch row (half the lanes of each half-wavefront idle), two slots each
    "softmax_top2": synth.Workload("f3", E=8, H=1792, I=512, topk=2, Ms=(2,)),
    # 48 groups per first-launch row: the whole wavefront on one row at a time
    "wide_h_bf16": synth.Workload("f4", E=16, H=6144, I=512, topk=4, Ms=(4,), dtype="bf16"),
    # 64 groups per first-launch row, two second-launch groups per row
    "widest_h": synth.Workload("f5", E=16, H=8192, I=256, topk=4, Ms=(3,)),
    # 128 slots: top-32 of 64 experts for 4 tokens
    "many_slots": synth.Workload("f7", E=64, H=512, I=256, topk=32, Ms=(4,), dtype="bf16"),
    # the most tokens the path takes: 5 tokens, 40 slots over 64 experts
    "tp_like_m5": synth.Workload("f8", E=64, H=1024, I=256, topk=8, Ms=(5,), score="sigmoid",
                                 num_groups=8, topk_groups=4, scale=2.5),
}


@pytest.mark.parametrize("name", sorted(FEW))
@pytest.mark.parametrize("seed", [0, 1])
def test_few_tokens_vs_oracle(name, seed):
    wl = FEW[name]
    assert B.fused_moe_wna16_path(wl.Ms[0], wl.H, wl.I, wl.E, wl.topk) == B.PATH_FEW_TOKENS
    print(f"few tokens {name} M={wl.Ms[0]} seed={seed}", flush=True)
    fused_vs_oracle(wl, wl.Ms[0], seed=seed)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [4, 5])
def test_few_tokens_hot_expert(dtype, M):
    """Every token's first choice is expert 3: one expert's rows meet every token's rows (five is
    the most a workgroup stages) in both launches."""
    wl = synth.Workload("fh", E=32, H=1024, I=512, topk=2, Ms=(M,), dtype=dtype)
    assert B.fused_moe_wna16_path(M, wl.H, wl.I, wl.E, wl.topk) == B.PATH_FEW_TOKENS
    layer = synth.make_layer(wl, seed=8)
    x = synth.make_x(wl, M, seed=8)
    lg = synth.make_logits(wl, M, seed=8)
    lg[:, 3] += 50.0
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), cuda_layer(layer))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert (ids_ref[:, 0] == 3).all()
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    ref = O.moe_layer(x, ids_ref, w_ref, O.ExpertSource(layer, 4))
    assert_layer_close(out, ref, f"few tokens, hot expert, {dtype}")


def test_few_tokens_deterministic_and_graph_replay():
    wl = FEW["tp_like_fp16"]
    M = 4
    layer = cuda_layer(synth.make_layer(wl, seed=1))
    x = synth.make_x(wl, M, seed=1).cuda()
    lg = synth.make_logits(wl, M, seed=1).cuda()
    out1, _, _ = run_fused(wl, x, lg, layer)
    out2, _, _ = run_fused(wl, x, lg, layer)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    ws = torch.empty((B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, wl.E, wl.topk, B.QUANT_INT4,
                                                       wl.torch_dtype, 0),), dtype=torch.uint8,
                     device="cuda")
    gout = torch.empty_like(out1)
    run = lambda: B.fused_moe_wna16(x, lg, wl.topk, routing_of(wl), layer["w13"],
                                    layer["w13_scales"], layer["w13_zeros"], layer["w2"],
                                    layer["w2_scales"], layer["w2_zeros"], block_m=0,
                                    workspace=ws, out=gout)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        gout.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout.view(torch.int16), out1.view(torch.int16)), f"replay {i}"
        run_fused(wl, x, lg, layer)  # eager work between replays
