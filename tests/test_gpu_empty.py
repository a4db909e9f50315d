"""Empty batches through every entry point: nothing is computed, every call succeeds, and the
one device-side result an empty batch has (the padded total T = 0 of the align step) is written."""
import pytest
import torch

import weight_only_int4_topk_amd as B

pytestmark = pytest.mark.gpu

E, H, I, TOPK = 8, 256, 256, 2


def test_routing_empty():
    lg = torch.empty((0, E), dtype=torch.float32, device="cuda")
    tw, ti = B.moe_topk_softmax(lg, TOPK, B.routing())
    assert tw.shape == (0, TOPK) and ti.shape == (0, TOPK)


@pytest.mark.parametrize("bm", [16, 128])
def test_align_empty_writes_zero_total(bm):
    ids = torch.empty((0,), dtype=torch.int32, device="cuda")
    assert B.moe_align_capacity(0, E, bm) == 0
    st, ex, npost = B.moe_align_block_size(ids, E, bm)   # capacity 0: empty id buffers
    torch.cuda.synchronize()
    assert st.numel() == 0 and ex.numel() == 0
    assert int(npost.item()) == 0


def test_align_empty_with_spare_capacity():
    """A capacity larger than needed is filled with sentinels (value numel = 0) and -1 blocks."""
    ids = torch.empty((0,), dtype=torch.int32, device="cuda")
    st, ex, npost = B.moe_align_block_size(ids, E, 16, capacity=48)
    torch.cuda.synchronize()
    assert int(npost.item()) == 0
    assert st.shape == (48,) and bool((st == 0).all())
    assert ex.shape == (3,) and bool((ex == -1).all())


def test_grouped_gemms_empty():
    ids = torch.empty((0,), dtype=torch.int32, device="cuda")
    st, ex, npost = B.moe_align_block_size(ids, E, 16)
    A = torch.empty((0, H), dtype=torch.float16, device="cuda")
    w = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    s = torch.ones((E, 2 * I, H // 128), dtype=torch.float16, device="cuda")
    z = torch.zeros((E, 2 * I, H // 256), dtype=torch.uint8, device="cuda")
    C = B.moe_wna16_gemm(A, TOPK, w, s, z, st, ex, npost, 16, 0, act=1)
    assert C.shape == (0, I)
    q, sc = B.moe_quant_int8_rows(A)
    assert q.shape == (0, H) and sc.shape == (0,)
    w8 = torch.zeros((E, 2 * I, H), dtype=torch.int8, device="cuda")
    s8 = torch.ones((E, 2 * I), dtype=torch.float16, device="cuda")
    C8 = B.moe_w8a8_gemm(q, sc, TOPK, w8, s8, st, ex, npost, 16, 0, torch.float16, act=1)
    assert C8.shape == (0, I)
    torch.cuda.synchronize()


def test_fused_layers_empty():
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, E), dtype=torch.float32, device="cuda")
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.int8, device="cuda")
    s13 = torch.ones((E, 2 * I), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((E, H, I), dtype=torch.int8, device="cuda")
    s2 = torch.ones((E, H), dtype=torch.bfloat16, device="cuda")
    out = B.fused_moe_w8a8(x, lg, TOPK, B.routing(), w13, s13, w2, s2)
    assert out.shape == (0, H)
    u13 = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    g13 = torch.ones((E, 2 * I, H // 128), dtype=torch.bfloat16, device="cuda")
    z13 = torch.zeros((E, 2 * I, H // 256), dtype=torch.uint8, device="cuda")
    p13 = torch.arange(H, dtype=torch.int32, device="cuda").repeat(E, 1)
    u2 = torch.zeros((E, H, I // 2), dtype=torch.uint8, device="cuda")
    g2 = torch.ones((E, H, I // 128), dtype=torch.bfloat16, device="cuda")
    z2 = torch.zeros((E, H, I // 256), dtype=torch.uint8, device="cuda")
    p2 = torch.arange(I, dtype=torch.int32, device="cuda").repeat(E, 1)
    out = B.fused_moe_wna16_act_order(x, lg, TOPK, B.routing(), u13, g13, z13, p13, u2, g2, z2,
                                      p2)
    assert out.shape == (0, H)
    torch.cuda.synchronize()
