"""The fused w8a8 layer (int8 experts, per-token int8 activations) on the GPU vs the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import (ORACLE_WORKERS, assert_align_exact, assert_layer_close, cuda_layer,
                     oracle_route, routing_of, spaced_rows)

pytestmark = pytest.mark.gpu

SMALL = {
    "softmax_fp16": synth.Workload("a", E=8, H=512, I=512, topk=2, Ms=(33,), dtype="fp16", bits=8),
    "softmax_bf16": synth.Workload("b", E=8, H=768, I=256, topk=2, Ms=(70,), dtype="bf16", bits=8),
    "sigmoid_groups_bf16": synth.Workload("c", E=64, H=512, I=256, topk=8, Ms=(20,), score="sigmoid",
                                          num_groups=8, topk_groups=4, scale=2.5, dtype="bf16",
                                          bits=8),
    "single_token": synth.Workload("d", E=16, H=1024, I=512, topk=4, Ms=(1,), bits=8),
}


def _run(wl, M, seed, device="cpu", block_m=0):
    layer = synth.make_layer(wl, seed=seed, device=device)
    x = synth.make_x(wl, M, seed=seed, device=device)
    lg = synth.make_logits(wl, M, seed=seed, device=device)
    lay = cuda_layer(layer) if device == "cpu" else layer
    ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
    out = B.fused_moe_w8a8(x.cuda(), lg.cuda(), wl.topk, routing_of(wl), lay["w13"],
                           lay["w13_scales"], lay["w2"], lay["w2_scales"], block_m=block_m,
                           topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    ids, w = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids)
    return out, x, ids, w, lay


@pytest.mark.parametrize("name", sorted(SMALL))
def test_fused_w8a8_vs_oracle(name):
    wl = SMALL[name]
    M = wl.Ms[0]
    out, x, ids, w, lay = _run(wl, M, seed=5)
    print(f"fused w8a8 {name} M={M}", flush=True)
    ref = O.moe_layer_w8a8_rows(x, ids, w, {k: v.cpu() for k, v in lay.items() if v is not None},
                                wl.dtype)
    assert_layer_close(out, ref, f"w8a8 {name}")


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_fused_w8a8_block_sizes_deterministic(bm):
    wl = SMALL["softmax_fp16"]
    out1, x, ids, w, lay = _run(wl, 33, seed=6, block_m=bm)
    out2, *_ = _run(wl, 33, seed=6, block_m=bm)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    ref = O.moe_layer_w8a8_rows(x, ids, w, {k: v.cpu() for k, v in lay.items() if v is not None},
                                wl.dtype)
    assert_layer_close(out1, ref, f"w8a8 bm={bm}")


def _expert_rows(lay, ids, rows):
    """The experts the listed tokens use, copied to the host, and ids renumbered to match."""
    experts = sorted(set(ids[rows].reshape(-1).tolist()))
    idx = torch.tensor(experts, dtype=torch.long, device="cuda")
    sub = {k: v.index_select(0, idx).cpu() for k, v in lay.items() if v is not None}
    remap = np.full(int(ids.max()) + 1, -1, np.int64)
    remap[experts] = np.arange(len(experts))
    ids_sub = np.where(np.isin(ids, experts), remap[np.clip(ids, 0, None)], 0)
    return sub, ids_sub


def test_fused_w8a8_mixtral_shape_all_tokens():
    """Mixtral-shaped int8 experts at M = 16 on the GPU; every token against the oracle (the
    experts copied to the host)."""
    wl = synth.WORKLOADS["mixtral"].with_(bits=8)
    M = 16
    out, x, ids, w, lay = _run(wl, M, seed=0, device="cuda")
    rows = np.arange(M)
    sub, ids_sub = _expert_rows(lay, ids, rows)
    ref = O.moe_layer_w8a8_rows(x.cpu(), ids_sub, w, sub, wl.dtype, rows=rows,
                                workers=ORACLE_WORKERS)
    assert_layer_close(O.to_numpy(out)[rows], ref, "w8a8 mixtral")


def test_fused_w8a8_dsv3_full_size_spaced_tokens():
    """DeepSeek-V3-shaped int8 experts (256 x H 7168 x I 2048, bf16, grouped sigmoid top-8) at the
    batch sizes the bench times, M = 4096 and 1024, with the library's block size (256 rows at 4096
    tokens, 64 at 1024): every token's routing exact, align exact at that block size, and 256 evenly
    spaced tokens of each batch (first and last included) against the oracle.  The smaller batch is
    the leading rows of the larger one, so the experts are copied and decoded once."""
    wl = synth.WORKLOADS["dsv3_prefill_int8"]
    lay = synth.make_layer(wl, seed=0, device="cuda")
    x = synth.make_x(wl, 4096, seed=0, device="cuda")
    lg = synth.make_logits(wl, 4096, seed=0, device="cuda")
    ids, w = oracle_route(wl, lg)
    outs, rows = {}, {}
    for M in (4096, 1024):
        bm = B.moe_pick_block_m(M, wl.E, wl.topk, 8, wl.torch_dtype)
        assert bm == (64 if M == 1024 else 256)
        print(f"fused w8a8 dsv3 full size M={M} block_m={bm}", flush=True)
        ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
        tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
        out = B.fused_moe_w8a8(x[:M].contiguous(), lg[:M].contiguous(), wl.topk, routing_of(wl),
                               lay["w13"], lay["w13_scales"], lay["w2"], lay["w2_scales"],
                               topk_weights=tw, topk_ids=ti)
        torch.cuda.synchronize()
        assert np.array_equal(O.to_numpy(ti), ids[:M])
        assert_align_exact(ids[:M], wl.E, bm)
        outs[M], rows[M] = O.to_numpy(out), spaced_rows(M)
    union = np.union1d(rows[4096], rows[1024])
    sub, ids_sub = _expert_rows(lay, ids, union)
    del lay
    ref = O.moe_layer_w8a8_rows(x.cpu(), ids_sub, w, sub, wl.dtype, rows=union,
                                workers=ORACLE_WORKERS)
    pos = {int(r): i for i, r in enumerate(union)}
    for M in (4096, 1024):
        r = rows[M]
        assert_layer_close(outs[M][r], ref[[pos[int(v)] for v in r]], f"w8a8 dsv3 M={M}")


def test_fused_w8a8_largest_batch_sampled():
    """The largest batch the w8a8 layer accepts at the DeepSeek-V3 int8 shape: M = 131071 keeps the
    second GEMM's int8 activations (M * topk * I bytes) under 2 GiB, one token more is refused.
    Its float32 rows then take 30 GB and the combine reads them past 2^34 bytes.  256
    evenly spaced tokens (first and last included) against the oracle, their routing exact."""
    wl = synth.WORKLOADS["dsv3_prefill_int8"]
    M = 131071
    assert M * wl.topk * wl.I < 2**31 <= (M + 1) * wl.topk * wl.I
    lay = synth.make_layer(wl, seed=0, device="cuda")
    x = synth.make_x(wl, M, seed=0, device="cuda")
    lg = synth.make_logits(wl, M, seed=0, device="cuda")
    ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
    print(f"fused w8a8 largest batch M={M}", flush=True)
    out = B.fused_moe_w8a8(x, lg, wl.topk, routing_of(wl), lay["w13"], lay["w13_scales"],
                           lay["w2"], lay["w2_scales"], topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    rows = spaced_rows(M)
    ids, w = oracle_route(wl, lg[rows])                   # routing is per token
    assert np.array_equal(O.to_numpy(ti)[rows], ids)
    sub, ids_sub = _expert_rows(lay, ids, np.arange(len(rows)))
    del lay
    ref = O.moe_layer_w8a8_rows(x[rows].cpu(), ids_sub, w, sub, wl.dtype, workers=ORACLE_WORKERS)
    assert_layer_close(O.to_numpy(out)[rows], ref, f"w8a8 dsv3 M={M}")
    assert torch.isfinite(out[-4096:].float()).all()
