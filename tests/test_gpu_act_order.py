"""The fused layer with GPTQ act-order uint4 experts on the GPU vs the CPU oracle.

The library reads the sorted storage (columns in group order plus each expert's permutation); the
oracle reads the GPTQ form (codes in the original column order plus the group index of every
column), rebuilt here from the seeded layer, and decodes with oracle.dequant_uint4_gidx."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import ORACLE_WORKERS, assert_layer_close, oracle_route, routing_of, spaced_rows

pytestmark = pytest.mark.gpu


class GidxSource:
    """float64 weights of each expert in the original column order, from the GPTQ form."""

    def __init__(self, layer, experts):
        self.layer = {k: O.to_numpy(v) for k, v in layer.items()}
        self.index = {int(e): i for i, e in enumerate(experts)}

    def _deq(self, name, e):
        i = self.index[int(e)]
        q_sorted = O.unpack_uint4(self.layer[name][i])
        perm = self.layer[name + "_perm"][i].astype(np.int64)
        q = np.empty_like(q_sorted)
        q[:, perm] = q_sorted                                 # column perm[j] holds sorted column j
        g_idx = np.empty(perm.shape[0], np.int64)
        g_idx[perm] = np.arange(perm.shape[0]) // 128
        packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        return O.dequant_uint4_gidx(packed, self.layer[name + "_scales"][i],
                                    self.layer[name + "_zeros"][i], g_idx)

    def w13(self, e):
        return self._deq("w13", e)

    def w2(self, e):
        return self._deq("w2", e)


SMALL = {
    "softmax_fp16": synth.Workload("a", E=8, H=512, I=512, topk=2, Ms=(33,)),
    "softmax_bf16": synth.Workload("b", E=16, H=768, I=512, topk=4, Ms=(50,), dtype="bf16"),
    "sigmoid_groups": synth.Workload("c", E=64, H=512, I=256, topk=8, Ms=(20,), score="sigmoid",
                                     num_groups=8, topk_groups=4, scale=2.5),
    "single_token": synth.Workload("d", E=8, H=1792, I=768, topk=2, Ms=(1,)),
    # one token, more experts and slots, and a wider first-GEMM K
    "single_token_sigmoid_bf16": synth.Workload("e", E=64, H=2048, I=512, topk=8, Ms=(1,),
                                                dtype="bf16", score="sigmoid", num_groups=8,
                                                topk_groups=4, scale=2.5),
    "single_token_two_steps": synth.Workload("f", E=16, H=6144, I=768, topk=4, Ms=(1,)),
}


def _run(wl, M, seed, device="cpu", rows=None):
    layer = synth.make_layer_act_order(wl, seed=seed, device=device)
    x = synth.make_x(wl, M, seed=seed, device=device)
    lg = synth.make_logits(wl, M, seed=seed, device=device)
    lay = {k: v.cuda() for k, v in layer.items()}
    ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
    out = B.fused_moe_wna16_act_order(x.cuda(), lg.cuda(), wl.topk, routing_of(wl), lay["w13"],
                                      lay["w13_scales"], lay["w13_zeros"], lay["w13_perm"],
                                      lay["w2"], lay["w2_scales"], lay["w2_zeros"], lay["w2_perm"],
                                      topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    ids, w = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    experts = sorted(set(ids[rows].reshape(-1).tolist()))
    idx = torch.tensor(experts, dtype=torch.long, device=lay["w13"].device)
    sub = {k: v.index_select(0, idx).cpu() for k, v in lay.items()}
    ref, _ = O.moe_layer_rows(x.cpu(), ids, w, GidxSource(sub, experts), rows,
                              workers=ORACLE_WORKERS)
    return out, ref, rows


@pytest.mark.parametrize("name", sorted(SMALL))
def test_act_order_layer_vs_oracle(name):
    wl = SMALL[name]
    out, ref, rows = _run(wl, wl.Ms[0], seed=3)
    print(f"act-order {name}", flush=True)
    assert_layer_close(O.to_numpy(out)[rows], ref, f"act-order {name}")


def test_act_order_deterministic():
    wl = SMALL["softmax_fp16"]
    a, _, _ = _run(wl, 33, seed=4)
    b, _, _ = _run(wl, 33, seed=4)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_act_order_mixtral_shape_all_tokens():
    wl = synth.WORKLOADS["mixtral"]
    out, ref, rows = _run(wl, 16, seed=0, device="cuda")
    assert_layer_close(O.to_numpy(out)[rows], ref, "act-order mixtral")


def test_act_order_mixtral_shape_one_token():
    wl = synth.WORKLOADS["mixtral"]
    out, ref, rows = _run(wl, 1, seed=0, device="cuda")
    assert_layer_close(O.to_numpy(out)[rows], ref, "act-order mixtral, one token")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_act_order_one_token_matches_grouped_with_entries_out_of_range(dtype):
    """Permutation entries outside [0, H) / [0, I) read as zero whatever the block size: the
    library's choice (block_m 0) against 16-row blocks on the same inputs."""
    wl = SMALL["single_token"].with_(dtype=dtype)
    lay = synth.make_layer_act_order(wl, seed=5, device="cuda")
    lay["w13_perm"][:, 5] = wl.H
    lay["w13_perm"][1, 200] = -1
    lay["w2_perm"][:, 7] = wl.I + 3
    x = synth.make_x(wl, 1, seed=5, device="cuda")
    lg = synth.make_logits(wl, 1, seed=5, device="cuda")
    outs = [B.fused_moe_wna16_act_order(x, lg, wl.topk, routing_of(wl), lay["w13"],
                                        lay["w13_scales"], lay["w13_zeros"], lay["w13_perm"],
                                        lay["w2"], lay["w2_scales"], lay["w2_zeros"],
                                        lay["w2_perm"], block_m=bm) for bm in (0, 16)]
    torch.cuda.synchronize()
    assert_layer_close(outs[0], O.to_numpy(outs[1]), f"act-order, two block sizes, {dtype}")


def test_act_order_largest_batch_sampled():
    """The largest batch the act-order layer accepts at the DeepSeek-V3 prefill shape: M = 18724
    keeps the first GEMM's gathered rows (M * topk * H * 2 bytes) under 2 GiB, one token more is
    refused.  256 evenly spaced tokens, the last one's gathered rows ending just below 2^31 bytes,
    against the oracle, their routing exact."""
    wl = synth.WORKLOADS["dsv3_prefill_int4"]
    M = 18724
    assert M * wl.topk * wl.H * 2 < 2**31 <= (M + 1) * wl.topk * wl.H * 2
    lay = synth.make_layer_act_order(wl, seed=0, device="cuda")
    x = synth.make_x(wl, M, seed=0, device="cuda")
    lg = synth.make_logits(wl, M, seed=0, device="cuda")
    ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
    print(f"act-order largest batch M={M}", flush=True)
    out = B.fused_moe_wna16_act_order(x, lg, wl.topk, routing_of(wl), lay["w13"],
                                      lay["w13_scales"], lay["w13_zeros"], lay["w13_perm"],
                                      lay["w2"], lay["w2_scales"], lay["w2_zeros"], lay["w2_perm"],
                                      topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    rows = spaced_rows(M)
    assert rows[-1] == M - 1
    ids, w = oracle_route(wl, lg[rows])                   # routing is per token
    assert np.array_equal(O.to_numpy(ti)[rows], ids)
    experts = sorted(set(ids.reshape(-1).tolist()))
    idx = torch.tensor(experts, dtype=torch.long, device="cuda")
    sub = {k: v.index_select(0, idx).cpu() for k, v in lay.items()}
    del lay
    ref, _ = O.moe_layer_rows(x[rows].cpu(), ids, w, GidxSource(sub, experts),
                              np.arange(len(rows)), workers=ORACLE_WORKERS)
    assert_layer_close(O.to_numpy(out)[rows], ref, f"act-order dsv3 M={M}")
