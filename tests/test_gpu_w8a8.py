"""w8a8 (per-token int8 activations, per-channel int8 weights) on the GPU vs the CPU oracle.

The GEMM is fed the oracle's own activation codes and scales (the quantiser is checked bit-exactly on
its own), so every input of the comparison comes from the oracle or the seeded generators."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import assert_layer_close, cuda_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("rows,K", [(1, 256), (7, 4096), (130, 768)])
def test_quant_int8_rows_exact(dt, rows, K):
    """Codes and scales equal the oracle's bit for bit (both decide in float32), including a row of
    zeros and a row whose maximum sits on a rounding tie."""
    wl = synth.Workload("q", E=1, H=K, I=256, topk=1, Ms=(rows,), dtype=dt)
    x = synth.make_x(wl, rows, seed=rows + K)
    x[0] = 0
    if rows > 2:
        x[2, :] = x[2, :] * 0 + 0.25
        x[2, 1] = 127 * 0.25 / 127 * 0.5                 # exactly half a step: a tie
    q, s = B.moe_quant_int8_rows(x.cuda())
    torch.cuda.synchronize()
    rq, rs = O.quant_int8_rows(x)
    assert np.array_equal(s.cpu().numpy(), rs), "scales differ"
    assert np.array_equal(q.cpu().numpy(), rq), "codes differ"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("bm", [16, 64, 128, 256])
def test_w8a8_layout_probe_bit_exact(dt, bm):
    """Activation codes one-hot at column k with scale 1, routed to one expert: row k of the output
    is column k of that expert's int8 weights times their channel scales, which must equal the
    correctly rounded q * s bit for bit.  A wrong pairing of A and B bytes in the matrix-core
    operands would mix columns."""
    wl = synth.Workload("p8", E=2, H=512, I=256, topk=1, Ms=(1,), dtype=dt, bits=8)
    layer = synth.make_layer(wl, seed=6)
    lay = cuda_layer(layer)
    K = wl.H
    A = torch.eye(K, dtype=torch.int8, device="cuda")
    sa = torch.ones((K,), dtype=torch.float32, device="cuda")
    for e in range(wl.E):
        ids = torch.full((K, 1), e, dtype=torch.int32, device="cuda")
        st, ex, npost = B.moe_align_block_size(ids, wl.E, bm)
        C = B.moe_w8a8_gemm(A, sa, 1, lay["w13"], lay["w13_scales"], st, ex, npost, bm, K,
                            wl.torch_dtype)
        torch.cuda.synchronize()
        ref = O.dequant_bits(O.dequant_int8(O.to_numpy(layer["w13"][e]),
                                            O.to_numpy(layer["w13_scales"][e])), dt)   # [N, K]
        got = C.view(torch.int16).cpu().numpy().view(np.uint16).T
        assert np.array_equal(got, ref), f"expert {e}"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("act,weighted", [(1, False), (0, True)])
def test_w8a8_gemm_vs_oracle(dt, bm, act, weighted):
    wl = synth.Workload("g8", E=6, H=768, I=512, topk=3, Ms=(45,), dtype=dt, bits=8)
    layer = synth.make_layer(wl, seed=9)
    lay = cuda_layer(layer)
    M = 45
    x = synth.make_x(wl, M, seed=9)
    lg = synth.make_logits(wl, M, seed=9)
    ids, w = O.route(O.to_numpy(lg), wl.topk)
    ns = M * wl.topk
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    tw = torch.from_numpy(w.astype(np.float32)).cuda() if weighted else None
    if act:
        Aq, sa = O.quant_int8_rows(x)
        div, name = wl.topk, "w13"
    else:
        h = (torch.randn(ns, wl.I, generator=torch.Generator().manual_seed(10)) * 0.3)
        Aq, sa = O.quant_int8_rows(h)
        div, name = 1, "w2"
    C = B.moe_w8a8_gemm(torch.from_numpy(Aq).cuda(), torch.from_numpy(sa).cuda(), div, lay[name],
                        lay[name + "_scales"], st, ex, npost, bm, ns, wl.torch_dtype,
                        topk_weights=tw, act=act)
    torch.cuda.synchronize()
    ref = O.w8a8_grouped_gemm(Aq, sa, div,
                              lambda e: (O.to_numpy(layer[name][e]), O.to_numpy(layer[name + "_scales"][e])),
                              *O.align_block_size(ids, wl.E, bm), bm, ns,
                              topk_weights=w if weighted else None, act=act)
    assert_layer_close(C, np.stack([ref[s] for s in range(ns)]), f"w8a8 act={act} bm={bm}")


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("act,weighted", [(1, False), (0, True)])
def test_w8a8_gemm_256_rows_hot_experts(dt, act, weighted):
    """256-row blocks with every count of filled 32-row tiles: expert 0 takes 300 slots (a full
    block and a block of 44 rows), expert 1 takes 170 (six tiles, the last partial), expert 2 takes
    the remaining 230 (eight tiles, the last partial); with the SiLU epilogue each wavefront's column
    tile mixes 16 gate and the 16 matching up rows."""
    wl = synth.Workload("h8", E=3, H=512, I=256, topk=1, Ms=(700,), dtype=dt, bits=8)
    layer = synth.make_layer(wl, seed=11)
    lay = cuda_layer(layer)
    M = 700
    ids = np.concatenate([np.zeros(300), np.ones(170), np.full(230, 2)]).astype(np.int32)
    ids = ids[np.random.default_rng(3).permutation(M)].reshape(M, 1)
    w = np.random.default_rng(4).uniform(0.1, 1.0, size=(M, 1)).astype(np.float32)
    bm = 256
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, bm)
    tw = torch.from_numpy(w).cuda() if weighted else None
    if act:
        x = synth.make_x(wl, M, seed=12)
        Aq, sa = O.quant_int8_rows(x)
        name = "w13"
    else:
        h = (torch.randn(M, wl.I, generator=torch.Generator().manual_seed(13)) * 0.3)
        Aq, sa = O.quant_int8_rows(h)
        name = "w2"
    C = B.moe_w8a8_gemm(torch.from_numpy(Aq).cuda(), torch.from_numpy(sa).cuda(), 1, lay[name],
                        lay[name + "_scales"], st, ex, npost, bm, M, wl.torch_dtype,
                        topk_weights=tw, act=act)
    torch.cuda.synchronize()
    ref = O.w8a8_grouped_gemm(Aq, sa, 1,
                              lambda e: (O.to_numpy(layer[name][e]), O.to_numpy(layer[name + "_scales"][e])),
                              *O.align_block_size(ids, wl.E, bm), bm, M,
                              topk_weights=w if weighted else None, act=act)
    assert_layer_close(C, np.stack([ref[s] for s in range(M)]), f"w8a8 256 rows act={act}")


def test_w8a8_mixtral_shape_sampled():
    """Mixtral-shaped experts (8 x [28672, 4096] int8, fp16) at M = 64, first GEMM with SiLU, every
    slot of the batch checked on 512 sampled output columns."""
    wl = synth.WORKLOADS["mixtral"].with_(bits=8)
    layer = synth.make_layer(wl, seed=0, device="cuda")
    M = 64
    x = synth.make_x(wl, M, seed=0)
    lg = synth.make_logits(wl, M, seed=0)
    ids, _ = O.route(O.to_numpy(lg), wl.topk)
    Aq, sa = O.quant_int8_rows(x)
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(ids).cuda(), wl.E, 32)
    C = B.moe_w8a8_gemm(torch.from_numpy(Aq).cuda(), torch.from_numpy(sa).cuda(), wl.topk,
                        layer["w13"], layer["w13_scales"], st, ex, npost, 32, M * wl.topk,
                        wl.torch_dtype, act=1)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(1).choice(wl.I, size=512, replace=False))
    rows = np.concatenate([cols, wl.I + cols])
    sub = lambda e: (O.to_numpy(layer["w13"][e])[rows], O.to_numpy(layer["w13_scales"][e])[rows])
    ref = O.w8a8_grouped_gemm(Aq, sa, wl.topk, sub, *O.align_block_size(ids, wl.E, 32), 32,
                              M * wl.topk, act=1)
    got = O.to_numpy(C)[:, cols]
    assert_layer_close(got, np.stack([ref[s] for s in range(M * wl.topk)]), "w8a8 mixtral")
