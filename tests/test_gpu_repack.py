"""moe_repack_uint4 (GPTQ / AWQ checkpoint storage -> canonical storage) on the GPU against the
oracle, bit for bit, and checkpoints fed through the layer after repacking.

The checkpoints are synthetic: codes, zero points and scales drawn from a seeded generator and
packed here by the stated layouts (tests/golden/gptq_awq_layout.txt pins that packing by hand)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import assert_layer_close, cuda_layer, oracle_route, routing_of

pytestmark = pytest.mark.gpu


def _pack_words(vals):
    v = np.asarray(vals, dtype=np.int64)
    w = np.zeros(v.shape[:-1], np.int64)
    for i in range(8):
        w |= v[..., i] << (4 * i)
    return w.astype(np.uint32).view(np.int32)


def _checkpoint(fmt, E, N, K, dt, seed, act_order=False):
    """Random checkpoint of E experts: q [E, K, N], z [E, G, N], s [E, G, N], g_idx [E, K] or None,
    and the packed tensors (qweight, qzeros, scales, g_idx) as the checkpoint ships them."""
    rng = np.random.default_rng(seed)
    G = K // 128
    q = rng.integers(0, 16, size=(E, K, N))
    z = rng.integers(0, 16, size=(E, G, N))
    s = torch.tensor(rng.uniform(0.002, 0.02, size=(E, G, N))).to(dt)
    g_idx = None
    if act_order:
        g_idx = np.empty((E, K), np.int64)
        for e in range(E):
            order = rng.permutation(K)
            g_idx[e, order] = np.arange(K) // 128          # every group exactly 128 columns
    if fmt == B.FORMAT_GPTQ:
        qw = _pack_words(q.reshape(E, K // 8, 8, N).transpose(0, 1, 3, 2))
    else:
        qw = _pack_words(q.reshape(E, K, N // 8, 8)[..., list(O.AWQ_PACK_ORDER)])
    zo = list(range(8)) if fmt == B.FORMAT_GPTQ else list(O.AWQ_PACK_ORDER)
    qz = _pack_words(z.reshape(E, G, N // 8, 8)[..., zo])
    dev = dict(qweight=torch.from_numpy(qw).cuda(), qzeros=torch.from_numpy(qz).cuda(),
               scales=s.cuda(), g_idx=None if g_idx is None else torch.from_numpy(g_idx.astype(np.int32)).cuda())
    return q, z, s, g_idx, dev


@pytest.mark.parametrize("fmt,act_order", [(0, False), (1, False), (0, True)])
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_repack_vs_oracle(fmt, act_order, dt):
    """E 3, N 200 (not a multiple of the 64-row tile), K 768: every output byte against the oracle's
    unpacking and canonical storage (which the hand-worked golden fixture pins)."""
    E, N, K = 3, 200, 768
    q, z, s, g_idx, dev = _checkpoint(fmt, E, N, K, dt, seed=7 + fmt, act_order=act_order)
    out = B.moe_repack_uint4(fmt, dev["qweight"], dev["qzeros"], dev["scales"], g_idx=dev["g_idx"])
    torch.cuda.synchronize()
    unpack = O.unpack_gptq if fmt == 0 else O.unpack_awq
    for e in range(E):
        uq, uz = unpack(dev["qweight"][e].cpu(), dev["qzeros"][e].cpu())
        np.testing.assert_array_equal(uq, q[e])           # the test's packing is the stated one
        Bo, so, zo, perm = O.canonical_from_checkpoint(uq, uz, s[e], None if g_idx is None else g_idx[e])
        assert np.array_equal(O.to_numpy(out[0][e]), Bo), f"codes, expert {e}"
        assert torch.equal(out[1][e].cpu(), s[e].T.contiguous()), f"scales, expert {e}"
        assert np.array_equal(O.to_numpy(out[2][e]), zo), f"zeros, expert {e}"
        if act_order:
            assert np.array_equal(O.to_numpy(out[3][e]), perm), f"perm, expert {e}"


def test_repack_counts_invalid_groups():
    """g_idx with 129 columns in group 0 and 127 in group 1: the 129th column of group 0 is left
    out, group 1 is padded with K, and *invalid counts both."""
    E, N, K = 1, 64, 256
    q, z, s, _, dev = _checkpoint(0, E, N, K, torch.float16, seed=3)
    g = np.zeros((1, K), np.int32)
    g[0, 129:] = 1                                        # group 0: columns 0..128, group 1: 127
    inv = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, _, _, perm = B.moe_repack_uint4(0, dev["qweight"], dev["qzeros"], dev["scales"],
                                       g_idx=torch.from_numpy(g).cuda(), invalid=inv)
    torch.cuda.synchronize()
    p = O.to_numpy(perm)[0]
    assert p[:128].tolist() == list(range(128))
    assert p[128:255].tolist() == list(range(129, 256)) and p[255] == K
    assert int(inv.item()) == 2


class CheckpointSource:
    """float64 weights of each expert straight from a checkpoint's codes (original column order):
    w[n, k] = (q[k, n] - z[g(k), n]) * s[g(k), n], with g(k) = g_idx[k] or k // 128."""

    def __init__(self, parts):
        self.parts = parts                                # name -> (q, z, s, g_idx)

    def _w(self, name, e):
        q, z, s, g = self.parts[name]
        K = q.shape[1]
        gk = np.arange(K) // 128 if g is None else g[e]
        s64 = O.to_numpy(s[e]).astype(np.float64)
        return ((q[e].astype(np.float64) - z[e][gk, :]) * s64[gk, :]).T

    def w13(self, e):
        return self._w("w13", e)

    def w2(self, e):
        return self._w("w2", e)


@pytest.mark.parametrize("fmt,act_order", [(0, True), (1, False)])
def test_checkpoint_through_the_layer(fmt, act_order):
    """A GPTQ act-order checkpoint through fused_moe_wna16_act_order, and an AWQ checkpoint through
    fused_moe_wna16, after repacking on the GPU, against the oracle decoding the checkpoint."""
    wl = synth.Workload("ck", E=8, H=512, I=256, topk=2, Ms=(24,), dtype="fp16")
    M = 24
    dt = torch.float16
    q13, z13, s13, g13, d13 = _checkpoint(fmt, wl.E, 2 * wl.I, wl.H, dt, seed=11, act_order=act_order)
    q2, z2, s2, g2, d2 = _checkpoint(fmt, wl.E, wl.H, wl.I, dt, seed=12, act_order=act_order)
    r13 = B.moe_repack_uint4(fmt, d13["qweight"], d13["qzeros"], d13["scales"], g_idx=d13["g_idx"])
    r2 = B.moe_repack_uint4(fmt, d2["qweight"], d2["qzeros"], d2["scales"], g_idx=d2["g_idx"])
    x = (torch.randn(M, wl.H, generator=torch.Generator().manual_seed(5)) * 0.5).to(dt)
    lg = synth.make_logits(wl, M, seed=5)
    rt = routing_of(wl)
    if act_order:
        out = B.fused_moe_wna16_act_order(x.cuda(), lg.cuda(), wl.topk, rt, r13[0], r13[1], r13[2],
                                          r13[3], r2[0], r2[1], r2[2], r2[3])
    else:
        out = B.fused_moe_wna16(x.cuda(), lg.cuda(), wl.topk, rt, r13[0], r13[1], r13[2], r2[0],
                                r2[1], r2[2])
    torch.cuda.synchronize()
    ids, w = oracle_route(wl, lg)
    src = CheckpointSource({"w13": (q13, z13, s13, g13), "w2": (q2, z2, s2, g2)})
    ref = O.moe_layer(x, ids, w, src)
    assert_layer_close(out, ref, f"checkpoint fmt={fmt} act_order={act_order}")
