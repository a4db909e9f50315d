"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import os

import numpy as np
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B

# layer-output tolerance: |gpu - ref| <= ATOL + RTOL*|ref| per element, and a relative L2 gate that
# the elementwise bound alone would not enforce for small-magnitude outputs
ATOL, RTOL, REL_L2 = 1e-2, 1e-2, 1e-2

# threads for the oracle's per-expert work at full size
ORACLE_WORKERS = max(1, min(8, os.cpu_count() or 1))


def spaced_rows(M, n=256):
    """n evenly spaced token rows of a batch of M (all of them when M <= n), first and last kept."""
    if M <= n:
        return np.arange(M)
    return np.unique(np.round(np.linspace(0, M - 1, n)).astype(np.int64))


def routing_of(wl):
    return B.routing(wl.score, wl.renormalize, wl.num_groups, wl.topk_groups, wl.scale)


def oracle_route(wl, logits):
    return O.route(O.to_numpy(logits), wl.topk, wl.score, wl.renormalize, wl.num_groups,
                   wl.topk_groups, wl.scale)


def assert_layer_close(gpu, ref, what=""):
    g = O.to_numpy(gpu).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, max err {err.max()}"
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e}"
    return rel


def assert_weights_close(gpu_w, ref_w):
    g = O.to_numpy(gpu_w).astype(np.float64)
    np.testing.assert_allclose(g, ref_w, rtol=2e-6, atol=1e-7)


def cuda_layer(layer):
    return {k: (v.cuda() if v is not None else None) for k, v in layer.items()}


def run_fused(wl, x, logits, layer, block_m=None):
    M = x.shape[0]
    tw = torch.empty((M, wl.topk), dtype=torch.float32, device="cuda")
    ti = torch.empty((M, wl.topk), dtype=torch.int32, device="cuda")
    out = B.fused_moe_wna16(x, logits, wl.topk, routing_of(wl), layer["w13"], layer["w13_scales"],
                            layer["w13_zeros"], layer["w2"], layer["w2_scales"],
                            layer["w2_zeros"], block_m=wl.block_m if block_m is None else block_m,
                            topk_weights=tw, topk_ids=ti)
    torch.cuda.synchronize()
    return out, tw, ti


def expert_subset(layer, experts):
    """Copy the listed experts' stored weights to the host (for the oracle)."""
    idx = torch.tensor(list(experts), dtype=torch.long, device=layer["w13"].device)
    return {k: (v.index_select(0, idx).cpu() if v is not None else None) for k, v in layer.items()}


def fused_vs_oracle(wl, M, seed=0, device="cpu", rows=None, block_m=None, layer=None):
    """Run the fused layer on the GPU and compare with the oracle (all rows, or the listed rows).

    Inputs are drawn on `device` (cpu: bytes identical everywhere; cuda: for full-size layers)."""
    if layer is None:
        layer = synth.make_layer(wl, seed=seed, device=device)
    x = synth.make_x(wl, M, seed=seed, device=device)
    lg = synth.make_logits(wl, M, seed=seed, device=device)
    lay_gpu = cuda_layer(layer) if device == "cpu" else layer
    out, tw, ti = run_fused(wl, x.cuda(), lg.cuda(), lay_gpu, block_m)
    ids_ref, w_ref = oracle_route(wl, lg)
    assert np.array_equal(O.to_numpy(ti), ids_ref), "topk ids differ"
    assert_weights_close(tw, w_ref)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    experts = sorted(set(ids_ref[rows].reshape(-1).tolist()))
    src = O.ExpertSource(expert_subset(lay_gpu, experts), wl.bits, experts)
    ref, _ = O.moe_layer_rows(x.cpu(), ids_ref, w_ref, src, rows, workers=ORACLE_WORKERS)
    rel = assert_layer_close(O.to_numpy(out)[rows], ref, f"{wl.name} M={M} seed={seed}")
    return out, ids_ref, rel


def assert_align_exact(ids, E, bm):
    """moe_align_block_size on the GPU against the oracle, all three outputs bit for bit."""
    st, ex, npost = B.moe_align_block_size(torch.from_numpy(np.ascontiguousarray(ids)).cuda(), E, bm)
    r_st, r_ex, r_T = O.align_block_size(ids, E, bm)
    assert int(npost.item()) == r_T, f"T {int(npost.item())} != {r_T}"
    assert np.array_equal(O.to_numpy(st), r_st), "sorted_token_ids differ"
    assert np.array_equal(O.to_numpy(ex), r_ex), "expert_ids differ"
