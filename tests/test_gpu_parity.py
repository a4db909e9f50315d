"""Parity of the HIP path (through the C ABI) with the CPU oracle on an MI355X.

Bit-exact: routing ids, align outputs, decoded weights.  Layer outputs: |gpu - ref| <= 1e-2 +
1e-2*|ref| per element plus relative L2 <= 1e-2.  Small cases compare every element and span several
tiles with ragged tails; full-size layers (drawn on the GPU) compare sampled tokens."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from tests.helpers import (ORACLE_WORKERS, assert_align_exact, assert_layer_close,
                           assert_weights_close, cuda_layer, expert_subset, fused_vs_oracle,
                           oracle_route, routing_of, run_fused, spaced_rows)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen2", "dsv3_tp8", "dsv3_prefill_int4"])
@pytest.mark.parametrize("seed", [0, 1])
def test_routing_ids_exact(name, seed):
    wl = W[name]
    M = max(wl.Ms) if max(wl.Ms) <= 1024 else 1024
    lg = synth.make_logits(wl, M, seed=seed)
    tw, ti = B.moe_topk_softmax(lg.cuda(), wl.topk, routing_of(wl))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    assert_weights_close(tw, w_ref)


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("score,E,k,ng,tg", [("softmax", 64, 6, 1, 1), ("sigmoid", 96, 5, 6, 3),
                                              ("sigmoid", 1024, 8, 8, 4), ("sigmoid", 8, 8, 1, 1)])
def test_routing_variants(score, E, k, ng, tg, renorm):
    wl = synth.Workload("r", E=E, H=256, I=256, topk=k, Ms=(77,), score=score, renormalize=bool(renorm),
                        num_groups=ng, topk_groups=tg, scale=1.5)
    lg = synth.make_logits(wl, 77, seed=3)
    tw, ti = B.moe_topk_softmax(lg.cuda(), k, routing_of(wl))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    assert_weights_close(tw, w_ref)


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("score,E,k,ng,tg", [("softmax", 64, 6, 1, 1), ("softmax", 200, 8, 1, 1),
                                              ("sigmoid", 96, 5, 6, 3), ("sigmoid", 256, 8, 8, 4),
                                              ("sigmoid", 64, 32, 64, 40)])
@pytest.mark.parametrize("logits", ["ties", "neg_inf"])
@pytest.mark.parametrize("M", [33, 1024, 1025])
def test_routing_ties_and_neg_inf(score, E, k, ng, tg, renorm, logits, M):
    """64 to 256 experts up to 1024 tokens take the one-workgroup-per-token ranking launch, 1025
    tokens the one-wavefront-per-token launch: the same ids bit for bit and the oracle's weights,
    with ties (logits on a grid of 0.5: equal scores go to the lower id) and with -inf logits (a
    quarter of the experts of every token)."""
    wl = synth.Workload("rt", E=E, H=256, I=256, topk=k, Ms=(M,), score=score,
                        renormalize=bool(renorm), num_groups=ng, topk_groups=tg, scale=1.5)
    lg = synth.make_logits(wl, M, seed=7)
    if logits == "ties":
        lg = torch.round(lg * 2) / 2
    else:
        lg[:, 1::4] = -float("inf")
    tw, ti = B.moe_topk_softmax(lg.cuda(), k, routing_of(wl))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    assert_weights_close(tw, w_ref)


# ------------------------------------------------------------------------------------------------
# align
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,k,E,bm", [(16, 2, 8, 16), (1, 8, 256, 16), (64, 8, 256, 16),
                                      (256, 8, 256, 16), (512, 8, 64, 32), (4096, 8, 256, 128),
                                      (1023, 2, 8, 64), (333, 3, 1024, 16), (5, 1, 1, 16)])
def test_align_exact(M, k, E, bm):
    rng = np.random.default_rng(M + E + bm)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), E, bm)
    r_st, r_ex, r_T = O.align_block_size(ids, E, bm)
    assert int(npost.item()) == r_T
    assert np.array_equal(O.to_numpy(st), r_st)
    assert np.array_equal(O.to_numpy(ex), r_ex)


@pytest.mark.parametrize("numel,E,bm,foreign", [(64, 256, 16, False), (65, 256, 16, False),
                                                  (32, 1024, 64, False), (6, 8, 128, False),
                                                  (64, 64, 32, False), (1, 256, 16, False),
                                                  (40, 16, 16, True), (64, 3, 16, True)])
def test_align_small_batches(numel, E, bm, foreign):
    """Up to 64 slots one wavefront aligns alone (65 takes the workgroup path): stable order,
    experts repeated many times, ids of other shards (negative or >= E) left out."""
    rng = np.random.default_rng(numel * 7 + E + bm)
    ids = rng.integers(0, E, size=numel).astype(np.int32)
    if E <= 16:
        ids[: numel // 2] = E - 1                          # one expert takes many slots
    if foreign:
        ids[::5] = -1
        ids[1::7] = E + 3
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), E, bm)
    r_st, r_ex, r_T = O.align_block_size(ids, E, bm)
    assert int(npost.item()) == r_T
    assert np.array_equal(O.to_numpy(st), r_st)
    assert np.array_equal(O.to_numpy(ex), r_ex)


def test_align_skewed_and_foreign_ids():
    """All slots on one expert (many blocks), and ids outside [0, E) (not listed)."""
    ids = np.full((300, 2), 5, np.int32)
    ids[::7, 1] = -1
    ids[::11, 0] = 64
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), 64, 16)
    r_st, r_ex, r_T = O.align_block_size(ids, 64, 16)
    assert int(npost.item()) == r_T
    assert np.array_equal(O.to_numpy(st), r_st)
    assert np.array_equal(O.to_numpy(ex), r_ex)


@pytest.mark.parametrize("E,k,M,bm,hot", [(64, 8, 1024, 16, False), (256, 8, 4096, 64, False),
                                         (256, 8, 4096, 256, True), (32, 2, 8192, 32, True)])
def test_fused_layer_align_many_slots_exact(E, k, M, bm, hot):
    """From 8192 slots on, the fused layer aligns with two launches over many workgroups (its
    counts in the layer's workspace).  Its sorted ids, block expert ids and padded total, read back
    from the workspace (laid out as routing weights, ids, sorted ids, block expert ids, total, each
    at a 256-byte boundary), equal the oracle's bit for bit; with a hot expert (every token's first
    choice) one expert's slots span many workgroups' chunks."""
    wl = synth.Workload("am", E=E, H=256, I=256, topk=k, Ms=(M,))
    layer = cuda_layer(synth.make_layer(wl, seed=11))
    x = synth.make_x(wl, M, seed=11).cuda()
    lg = synth.make_logits(wl, M, seed=11)
    if hot:
        lg[:, 1] += 50.0
    lg = lg.cuda()
    S = M * k
    up = lambda v: (v + 255) // 256 * 256
    cap = B.moe_align_capacity(S, E, bm)
    need = B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, E, k, B.QUANT_INT4, wl.torch_dtype, bm)
    ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")
    B.fused_moe_wna16(x, lg, k, routing_of(wl), layer["w13"], layer["w13_scales"],
                      layer["w13_zeros"], layer["w2"], layer["w2_scales"], layer["w2_zeros"],
                      block_m=bm, workspace=ws)
    torch.cuda.synchronize()
    o_ids = up(S * 4)
    o_sorted = o_ids + up(S * 4)
    o_eids = o_sorted + up(cap * 4)
    nblk = (cap + bm - 1) // bm
    o_T = o_eids + up(nblk * 4)
    words = lambda o, n: ws[o:o + 4 * n].view(torch.int32).cpu().numpy()
    ids = words(o_ids, S).reshape(M, k)
    ids_ref, _ = oracle_route(wl, lg)
    assert np.array_equal(ids, ids_ref)
    r_st, r_ex, r_T = O.align_block_size(ids_ref, E, bm, capacity=cap)
    assert int(words(o_T, 1)[0]) == r_T
    assert np.array_equal(words(o_sorted, cap), r_st)
    assert np.array_equal(words(o_eids, nblk), r_ex)


def test_align_golden(golden):
    g = golden("align_example.txt")
    ids = np.array([int(v) for v in g["topk_ids"][0].split()], np.int32)
    E = int(g["C.E"][0])
    bm = int(g["C.block_m"][0])
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), E, bm)
    assert O.to_numpy(st).tolist() == [int(v) for v in g["C.sorted_token_ids"][0].split()]
    assert O.to_numpy(ex).tolist() == [int(v) for v in g["C.expert_ids"][0].split()]
    assert int(npost.item()) == int(g["C.num_tokens_post_padded"][0])


# ------------------------------------------------------------------------------------------------
# decoded weights (identity probe) and the grouped GEMM
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dt,bits", [("fp16", 4), ("bf16", 4), ("fp16", 8), ("bf16", 8)])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_dequant_identity_probe(dt, bits, bm):
    """One-hot activation rows routed to one expert with weight 1: GEMM row k is the decoded
    column k of that expert, which must equal the oracle's correctly rounded (q - z) * s exactly.
    Every kernel variant: BLOCK_M 16 (biased codes, bias and zero point removed by a second
    MFMA), 32 (fp16 uint4: the half-precision subtraction (1024+q) - (1024+z); int8 and bf16:
    biased codes), 64 and 128 (exact decoded weights; bf16 and int8 activations straight into
    LDS)."""
    wl = synth.Workload("p", E=3, H=512, I=256, topk=1, Ms=(1,), dtype=dt, bits=bits)
    layer = synth.make_layer(wl, seed=5)
    lay = cuda_layer(layer)
    K = wl.H
    eye = torch.eye(K, dtype=wl.torch_dtype, device="cuda")
    for e in range(wl.E):
        ids = torch.full((K, 1), e, dtype=torch.int32, device="cuda")
        st, ex, npost = B.moe_align_block_size(ids, wl.E, bm)
        C = B.moe_wna16_gemm(eye, 1, lay["w13"], lay["w13_scales"], lay["w13_zeros"], st, ex,
                             npost, bm, K)
        src = O.ExpertSource(layer, bits)
        ref_bits = O.dequant_bits(src.w13(e), dt)          # [2I, K]
        got = C.view(torch.int16).cpu().numpy().view(np.uint16).T   # [N, K]
        assert np.array_equal(got, ref_bits), f"expert {e}"


@pytest.mark.parametrize("dt,bits", [("fp16", 4), ("bf16", 4), ("bf16", 8)])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("act,weighted", [(1, False), (0, True), (0, False)])
def test_grouped_gemm_vs_oracle(dt, bits, bm, act, weighted):
    # block_m 32 without SiLU runs the 8-wavefront workgroup (N = 512 divides its 256 columns), as
    # do block_m 64 and 128 with bf16 activations or int8 weights (SiLU: 512 gate columns)
    wl = synth.Workload("g", E=6, H=512, I=512, topk=3, Ms=(45,), dtype=dt, bits=bits)
    layer = synth.make_layer(wl, seed=8)
    lay = cuda_layer(layer)
    M = 45
    x = synth.make_x(wl, M, seed=8)
    lg = synth.make_logits(wl, M, seed=8)
    ids, w = oracle_route(wl, lg)
    ns = M * wl.topk
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    tw = torch.from_numpy(w.astype(np.float32)).cuda() if weighted else None
    src = O.ExpertSource(layer, bits)
    if act:
        C = B.moe_wna16_gemm(x.cuda(), wl.topk, lay["w13"], lay["w13_scales"], lay["w13_zeros"],
                             st, ex, npost, bm, ns, topk_weights=tw, act=1)
        ref = O.grouped_gemm(x, wl.topk, src.w13, *O.align_block_size(ids, wl.E, bm), bm, ns,
                             topk_weights=w if weighted else None, act=1)
    else:
        A = (torch.randn(ns, wl.I, generator=torch.Generator().manual_seed(9)) * 0.3).to(wl.torch_dtype)
        C = B.moe_wna16_gemm(A.cuda(), 1, lay["w2"], lay["w2_scales"], lay["w2_zeros"], st, ex,
                             npost, bm, ns, topk_weights=tw, act=0)
        ref = O.grouped_gemm(A, 1, src.w2, *O.align_block_size(ids, wl.E, bm), bm, ns,
                             topk_weights=w if weighted else None, act=0)
    torch.cuda.synchronize()
    refm = np.stack([ref[s] for s in range(ns)])
    assert_layer_close(C, refm, f"gemm act={act}")


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("weighted", [False, True])
def test_grouped_gemm_silu_wide_experts(dt, weighted):
    """block_m 32 with SiLU(gate) * up for wide experts (I = 8192): the first GEMM's eight-wavefront
    workgroup (128 gate columns), every slot and column against the oracle."""
    wl = synth.Workload("w", E=3, H=256, I=8192, topk=2, Ms=(40,), dtype=dt)
    layer = synth.make_layer(wl, seed=12)
    lay = cuda_layer(layer)
    M, bm = 40, 32
    x = synth.make_x(wl, M, seed=12)
    lg = synth.make_logits(wl, M, seed=12)
    ids, w = oracle_route(wl, lg)
    ns = M * wl.topk
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    tw = torch.from_numpy(w.astype(np.float32)).cuda() if weighted else None
    C = B.moe_wna16_gemm(x.cuda(), wl.topk, lay["w13"], lay["w13_scales"], lay["w13_zeros"], st, ex,
                         npost, bm, ns, topk_weights=tw, act=1)
    ref = O.grouped_gemm(x, wl.topk, O.ExpertSource(layer, 4).w13, *O.align_block_size(ids, wl.E, bm),
                         bm, ns, topk_weights=w if weighted else None, act=1)
    torch.cuda.synchronize()
    assert_layer_close(C, np.stack([ref[s] for s in range(ns)]), "gemm silu wide experts")


# ------------------------------------------------------------------------------------------------
# the fused layer
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fused_tiny_layer(seed):
    out, ids, rel = fused_vs_oracle(W["tiny"], 16, seed=seed)
    assert rel < 5e-3


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_fused_tiny_block_sizes(bm):
    fused_vs_oracle(W["tiny"], 16, seed=0, block_m=bm)


SMALL = {
    "tiny_bf16": W["tiny"].with_(dtype="bf16"),
    "tiny_int8_fp16": W["tiny"].with_(bits=8),
    "tiny_int8_bf16": W["tiny"].with_(bits=8, dtype="bf16"),
    "sigmoid_groups": synth.Workload("sg", E=64, H=512, I=256, topk=8, Ms=(37,), score="sigmoid",
                                     num_groups=8, topk_groups=4, scale=2.5),
    "softmax_bias": synth.Workload("sb", E=64, H=768, I=512, topk=8, Ms=(50,), logit_bias=True),
    "prefill_bf16_int4": synth.Workload("pi4", E=16, H=1024, I=512, topk=4, Ms=(300,), dtype="bf16"),
    "prefill_bf16_int8": synth.Workload("pi8", E=16, H=1024, I=512, topk=4, Ms=(300,), dtype="bf16",
                                        bits=8),
    "no_renorm": synth.Workload("nr", E=32, H=512, I=256, topk=4, Ms=(40,), renormalize=False),
    "dense_single_expert": synth.Workload("d1", E=1, H=512, I=512, topk=1, Ms=(33,)),
    "all_experts": synth.Workload("ae", E=4, H=256, I=256, topk=4, Ms=(21,)),
    # few workgroups: the first GEMM is split over K (14 k-blocks into 2 x 7, the second split
    # starting on an odd k-block) and SiLU(gate) * up runs after the float32 partials are summed
    # (BLOCK_M 16 given: with the library's choice three tokens take the few-token path)
    "split_odd_start": synth.Workload("so", E=8, H=1792, I=768, topk=2, Ms=(3,), block_m=16),
    # BLOCK_M 64 (scales and zero points through the two-slot ring): zero-point rows of an odd
    # number of bytes (K / 256 = 7 and 5, so rows start on odd bytes and the 2-byte words the
    # kernel reads straddle rows), and the second GEMM split over K into 2 x 5 k-blocks, the second
    # split starting on an odd k-block (the other nibble of its zero-point bytes)
    "prefill_odd_rows_bf16": synth.Workload("pob", E=16, H=1792, I=1280, topk=4, Ms=(300,),
                                            dtype="bf16"),
    "prefill_odd_rows_fp16": synth.Workload("pof", E=16, H=1792, I=1280, topk=4, Ms=(300,)),
    # K = I = 256 with enough second-GEMM workgroups: each streams two column chunks in turn
    # against one staged activation tile (16 chunks, ~126 blocks)
    "column_groups": synth.Workload("cg", E=128, H=4096, I=256, topk=8, Ms=(64,), score="sigmoid",
                                    num_groups=8, topk_groups=4, scale=2.5),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_fused_small_variants(name):
    wl = SMALL[name]
    fused_vs_oracle(wl, wl.Ms[0], seed=4)


@pytest.mark.parametrize("name", ["prefill_bf16_int4", "prefill_bf16_int8", "prefill_odd_rows_bf16",
                                  "prefill_odd_rows_fp16", "tiny_int8_fp16"])
def test_fused_block_m_256(name):
    """256-row blocks (eight 32-row tiles, one column tile per wavefront; with SiLU the mixed
    gate/up tile): blocks holding 1 to 8 listed row tiles, odd zero-point rows, fp16 and bf16."""
    wl = SMALL[name]
    fused_vs_oracle(wl, wl.Ms[0], seed=4, block_m=256)


@pytest.mark.parametrize("dtype,bits", [("bf16", 4), ("bf16", 8), ("fp16", 4)])
def test_fused_block_m_256_hot_expert(dtype, bits):
    """One expert takes every token's first choice: 600 slots in blocks of 256 (two full blocks
    of eight row tiles and a tail of three), the other experts partly filled blocks."""
    wl = synth.Workload("hot256", E=8, H=1024, I=512, topk=2, Ms=(600,), dtype=dtype, bits=bits)
    layer = synth.make_layer(wl, seed=7)
    x = synth.make_x(wl, 600, seed=7)
    lg = synth.make_logits(wl, 600, seed=7)
    lg[:, 5] += 50.0
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), cuda_layer(layer), block_m=256)
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    assert_align_exact(ids_ref, wl.E, 256)
    ref = O.moe_layer(x, ids_ref, w_ref, O.ExpertSource(layer, bits))
    assert_layer_close(out, ref, f"hot expert, block_m 256, {dtype} int{bits}")


def test_fused_one_hot_expert_load():
    """Every token's first choice is the same expert (one expert with many blocks)."""
    wl = synth.Workload("hot", E=8, H=512, I=256, topk=2, Ms=(200,))
    layer = synth.make_layer(wl, seed=6)
    x = synth.make_x(wl, 200, seed=6)
    lg = synth.make_logits(wl, 200, seed=6)
    lg[:, 3] += 50.0
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), cuda_layer(layer))
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref)
    ref = O.moe_layer(x, ids_ref, w_ref, O.ExpertSource(layer, 4))
    assert_layer_close(out, ref, "hot expert")


def test_fused_single_token():
    fused_vs_oracle(W["tiny"], 1, seed=2)


def test_fused_deterministic_and_graph_replay():
    wl = W["tiny"]
    layer = cuda_layer(synth.make_layer(wl, seed=1))
    x = synth.make_x(wl, 16, seed=1).cuda()
    lg = synth.make_logits(wl, 16, seed=1).cuda()
    out1, _, _ = run_fused(wl, x, lg, layer)
    out2, _, _ = run_fused(wl, x, lg, layer)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    # capture into a graph and replay it, with eager work between replays
    M = 16
    ws = torch.empty((B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, wl.E, wl.topk, B.QUANT_INT4,
                                                       wl.torch_dtype, 16),), dtype=torch.uint8,
                     device="cuda")
    gout = torch.empty_like(out1)
    run = lambda: B.fused_moe_wna16(x, lg, wl.topk, routing_of(wl), layer["w13"],
                                    layer["w13_scales"], layer["w13_zeros"], layer["w2"],
                                    layer["w2_scales"], layer["w2_zeros"], block_m=16,
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


def test_fused_empty_batch():
    wl = W["tiny"]
    layer = cuda_layer(synth.make_layer(wl, seed=0))
    x = torch.empty((0, wl.H), dtype=torch.float16, device="cuda")
    lg = torch.empty((0, wl.E), dtype=torch.float32, device="cuda")
    out = B.fused_moe_wna16(x, lg, wl.topk, routing_of(wl), layer["w13"], layer["w13_scales"],
                            layer["w13_zeros"], layer["w2"], layer["w2_scales"], layer["w2_zeros"],
                            workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, wl.H)


# ------------------------------------------------------------------------------------------------
# full-size layers (drawn on the GPU), sampled tokens against the oracle
# ------------------------------------------------------------------------------------------------
# Every M of the Mixtral-, Qwen2- and DeepSeek-V3 TP-share workloads, so each plan the library
# picks at full size runs once: one token on the dot-product path, a few tokens of the TP share on
# the grouped dot-product path, and the grouped GEMMs with BLOCK_M 16/32/64, the first GEMM
# unsplit, split to ~512 workgroups and split towards one round, 8-wavefront workgroups; the
# grouped GEMMs also at the sizes the dot-product paths take (BLOCK_M 16 given).  Every token
# against the oracle; align of the full routing result at the BLOCK_M the grouped GEMMs ran.
FULL = [("mixtral", 64, 0), ("mixtral", 16, 0), ("mixtral", 4, 0), ("mixtral", 1, 0),
        ("mixtral", 1, 16), ("qwen2", 512, 0), ("qwen2", 128, 0), ("qwen2", 16, 0), ("qwen2", 1, 0),
        ("qwen2", 1, 16), ("dsv3_tp8", 256, 0), ("dsv3_tp8", 64, 0), ("dsv3_tp8", 16, 0),
        ("dsv3_tp8", 16, 16), ("dsv3_tp8", 4, 0), ("dsv3_tp8", 1, 0), ("dsv3_tp8", 1, 16)]


@pytest.mark.parametrize("name,M,bm", FULL)
def test_fused_full_size_all_tokens(name, M, bm):
    wl = W[name]
    print(f"full size {name} M={M} block_m={bm}", flush=True)
    out, ids, rel = fused_vs_oracle(wl, M, seed=0, device="cuda", block_m=bm)
    assert_align_exact(ids, wl.E, bm or B.moe_pick_block_m(M, wl.E, wl.topk, wl.bits, wl.torch_dtype))


@pytest.mark.parametrize("name", ["dsv3_prefill_int4", "dsv3_prefill_int8"])
def test_fused_prefill_full_size_spaced_tokens(name):
    """DeepSeek-V3 full-expert prefill (256 experts, H 7168, I 2048, bf16, grouped sigmoid top-8)
    at M = 4096 and 1024, in the launch configuration the bench times (the library's BLOCK_M):
    every token's routing exact, align exact at that BLOCK_M, and 256 evenly spaced tokens of each
    batch (first and last included) against the oracle.  The smaller batch is the leading rows of
    the larger one, so one decoding of each expert serves both."""
    wl = W[name]
    layer = synth.make_layer(wl, seed=0, device="cuda")
    Mbig = 4096
    x = synth.make_x(wl, Mbig, seed=0, device="cuda")
    lg = synth.make_logits(wl, Mbig, seed=0, device="cuda")
    ids_all, w_all = oracle_route(wl, lg)
    outs, rows = {}, {}
    for M in (4096, 1024):
        bm = B.moe_pick_block_m(M, wl.E, wl.topk, wl.bits, wl.torch_dtype)
        print(f"prefill {name} M={M} block_m={bm}", flush=True)
        out, tw, ti = run_fused(wl, x[:M].contiguous(), lg[:M].contiguous(), layer)
        assert np.array_equal(O.to_numpy(ti), ids_all[:M]), "topk ids differ"
        assert_weights_close(tw, w_all[:M])
        assert_align_exact(ids_all[:M], wl.E, bm)
        outs[M], rows[M] = O.to_numpy(out), spaced_rows(M)
    union = np.union1d(rows[4096], rows[1024])
    experts = sorted(set(ids_all[union].reshape(-1).tolist()))
    src = O.ExpertSource(expert_subset(layer, experts), wl.bits, experts)
    del layer
    ref, _ = O.moe_layer_rows(x.cpu(), ids_all, w_all, src, union, workers=ORACLE_WORKERS)
    pos = {int(r): i for i, r in enumerate(union)}
    for M in (4096, 1024):
        r = rows[M]
        assert_layer_close(outs[M][r], ref[[pos[int(v)] for v in r]], f"{name} M={M}")


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_grouped_gemm_fp16_tiny_activations(bm):
    """fp16 activations far below 2^-10 (N(0, (2e-5)^2)): the uint4 kernels store the activations
    met by the 16x high-nibble pairs divided by 16, which is subnormal there and drops up to 4 low
    bits.  The GEMM alone (no SiLU, whose fp16 rows would underflow at this scale), weights drawn
    N(0, 5^2) so the outputs stay normal fp16 numbers, against the oracle at every BLOCK_M."""
    wl = synth.Workload("tinyact", E=4, H=512, I=512, topk=2, Ms=(40,), x_std=2e-5, w_std=5.0)
    layer = synth.make_layer(wl, seed=3)
    lay = cuda_layer(layer)
    M = 40
    ns = M * wl.topk
    A = synth.make_x(wl.with_(H=wl.I), ns, seed=3)          # [slots, I] activations of w2
    assert float(A.float().abs().max()) < 2.0**-10
    ids, _ = oracle_route(wl, synth.make_logits(wl, M, seed=3))
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    C = B.moe_wna16_gemm(A.cuda(), 1, lay["w2"], lay["w2_scales"], lay["w2_zeros"], st, ex, npost,
                         bm, ns, act=0)
    torch.cuda.synchronize()
    ref = O.grouped_gemm(A, 1, O.ExpertSource(layer, 4).w2, *O.align_block_size(ids, wl.E, bm), bm,
                         ns)
    refm = np.stack([ref[s] for s in range(ns)])
    assert np.abs(refm).max() > 2.0**-14 * 4                  # normal fp16 outputs
    sc = 1.0 / np.abs(refm).max()                             # make the elementwise bound bite
    assert_layer_close(O.to_numpy(C).astype(np.float64) * sc, refm * sc, f"tiny activations bm={bm}")


@pytest.mark.parametrize("bm", [16, 32])
def test_grouped_gemm_longest_k(bm):
    """K = 35,840, the longest K the 16- and 32-row kernels accept (their scales and zero points for
    the whole K range staged in LDS beside the activation tiles, at the 160 KiB limit)."""
    wl = synth.Workload("lk", E=2, H=35840, I=256, topk=1, Ms=(20,), dtype="fp16", bits=4)
    layer = synth.make_layer(wl, seed=13)
    lay = cuda_layer(layer)
    M = 20
    x = synth.make_x(wl, M, seed=13)
    ids = (np.arange(M) % 2).astype(np.int32)[:, None]
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    C = B.moe_wna16_gemm(x.cuda(), 1, lay["w13"], lay["w13_scales"], lay["w13_zeros"], st, ex,
                         npost, bm, M, act=1)
    torch.cuda.synchronize()
    src = O.ExpertSource(layer, 4)
    ref = O.grouped_gemm(x, 1, src.w13, *O.align_block_size(ids, wl.E, bm), bm, M, act=1)
    assert_layer_close(C, np.stack([ref[s] for s in range(M)]), f"K=35840 bm={bm}")


def test_fused_zero_activations_give_zero():
    """x = 0: every product is exactly zero, so the layer output is exactly zero (also after the
    SiLU, whose value at 0 is 0, and the float32 combine)."""
    wl = W["tiny"]
    layer = cuda_layer(synth.make_layer(wl, seed=2))
    x = torch.zeros((16, wl.H), dtype=torch.float16, device="cuda")
    lg = synth.make_logits(wl, 16, seed=2).cuda()
    out, _, _ = run_fused(wl, x, lg, layer)
    assert (out.float() == 0).all()


def test_fused_largest_batch_sampled():
    """The largest batch the layer accepts at the DeepSeek-V3 prefill shape: M = 65535 keeps the
    intermediate rows (M * topk * I * 2 bytes) under 2 GiB, one token more is refused.  The second
    GEMM's float32 rows then hold 3.8e9 values (15 GB), so their offsets and the combine's pass
    2^32 bytes.  256 evenly spaced tokens (first and last included) against the oracle, routing
    included."""
    wl = W["dsv3_prefill_int4"]
    M = 65535
    assert M * wl.topk * wl.I * 2 < 2**31 <= (M + 1) * wl.topk * wl.I * 2
    layer = synth.make_layer(wl, seed=0, device="cuda")
    x = synth.make_x(wl, M, seed=0, device="cuda")
    lg = synth.make_logits(wl, M, seed=0, device="cuda")
    print(f"fused largest batch M={M}", flush=True)
    out, tw, ti = run_fused(wl, x, lg, layer)
    rows = spaced_rows(M)
    ids_ref, w_ref = oracle_route(wl, lg[rows])          # routing is per token
    assert np.array_equal(O.to_numpy(ti)[rows], ids_ref), "topk ids differ"
    assert_weights_close(tw[rows], w_ref)
    experts = sorted(set(ids_ref.reshape(-1).tolist()))
    src = O.ExpertSource(expert_subset(layer, experts), wl.bits, experts)
    del layer
    ref, _ = O.moe_layer_rows(x[rows].cpu(), ids_ref, w_ref, src, np.arange(len(rows)),
                              workers=ORACLE_WORKERS)
    assert_layer_close(O.to_numpy(out)[rows], ref, f"dsv3 prefill M={M}")
    assert torch.isfinite(out[-4096:].float()).all()
