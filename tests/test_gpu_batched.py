"""Grouped GEMM over batched-experts activations (A [E, T, K], per-expert row counts on the device)
on the GPU vs the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import assert_layer_close, cuda_layer

pytestmark = pytest.mark.gpu

SENTINEL = 0x7C01  # a NaN pattern in fp16 and a normal bf16 value: never produced by the kernel


def _case(E, T, K, N, bits, dt, counts, act, block_m=0, seed=0):
    wl = synth.Workload("b", E=E, H=K, I=N // 2, topk=1, Ms=(1,), dtype=dt, bits=bits)
    layer = synth.make_layer(wl, seed=seed)
    lay = cuda_layer(layer)
    A = (torch.randn((E, T, K), generator=torch.Generator().manual_seed(seed + 1)) * 0.1).to(
        wl.torch_dtype)
    cnt = torch.tensor(counts, dtype=torch.int32)
    n_out = N // 2 if act else N
    C = torch.full((E, T, n_out), SENTINEL, dtype=torch.int16).view(wl.torch_dtype).cuda()
    B.moe_wna16_batched_gemm(A.cuda(), cnt.cuda(), lay["w13"], lay["w13_scales"], lay["w13_zeros"],
                             act=act, block_m=block_m, C=C)
    torch.cuda.synchronize()
    src = O.ExpertSource(layer, bits)
    ref = O.batched_gemm(A, cnt.numpy(), src.w13, act=act)
    got = C.cpu()
    print(f"batched E={E} T={T} K={K} N={N} bits={bits} {dt} act={act} bm={block_m}", flush=True)
    if ref:
        keys = sorted(ref)
        assert_layer_close(torch.stack([got[e, r] for e, r in keys]),
                           np.stack([ref[k] for k in keys]), "batched rows")
    raw = got.view(torch.int16).numpy()
    for e in range(E):
        n = int(min(max(counts[e], 0), T))
        assert (raw[e, n:] == np.int16(SENTINEL)).all(), f"expert {e}: rows past its count written"


@pytest.mark.parametrize("bits,dt", [(4, "fp16"), (4, "bf16"), (8, "fp16"), (8, "bf16")])
@pytest.mark.parametrize("act", [0, 1])
def test_batched_vs_oracle(bits, dt, act):
    """Counts of 0, a full batch, more than the batch (clamped), negative (0) and ragged."""
    _case(E=6, T=40, K=512, N=512, bits=bits, dt=dt, counts=[40, 0, 17, 55, -3, 1], act=act)


@pytest.mark.parametrize("T,block_m", [(7, 0), (16, 0), (100, 0), (40, 16), (40, 64)])
def test_batched_block_sizes(T, block_m):
    rng = np.random.default_rng(T + block_m)
    counts = rng.integers(0, T + 1, size=5).tolist()
    counts[0] = T
    _case(E=5, T=T, K=768, N=1536, bits=4, dt="fp16", counts=counts, act=1, block_m=block_m, seed=2)


def test_batched_expert_parallel_share_sampled():
    """DeepSeek-V3 expert shape (H 7168, I 2048, uint4 g128, bf16) on an expert-parallel share of 8
    local experts with 64-token batches; every row checked for 2 of the experts."""
    E, T, K, N = 8, 64, 7168, 4096
    wl = synth.Workload("ep", E=E, H=K, I=N // 2, topk=1, Ms=(1,), dtype="bf16", bits=4)
    layer = synth.make_layer(wl, seed=3, device="cuda")
    A = (torch.randn((E, T, K), generator=torch.Generator(device="cuda").manual_seed(4),
                     device="cuda") * 0.1).to(torch.bfloat16)
    counts = [64, 3, 0, 50, 64, 1, 33, 64]
    C = B.moe_wna16_batched_gemm(A, torch.tensor(counts, dtype=torch.int32, device="cuda"),
                                 layer["w13"], layer["w13_scales"], layer["w13_zeros"], act=1)
    torch.cuda.synchronize()
    for e in (0, 3):
        sub = {k: (v[e:e + 1].cpu() if v is not None else None) for k, v in layer.items()}
        src = O.ExpertSource(sub, 4)
        ref = O.batched_gemm(A[e:e + 1].cpu(), np.array([counts[e]]), src.w13, act=1)
        keys = sorted(ref)
        assert_layer_close(torch.stack([C[e, r].cpu() for _, r in keys]),
                           np.stack([ref[k] for k in keys]), f"expert {e}")


def test_batched_output_past_4_gib():
    """The output is addressed with 64 bits: 80 experts x 4096 tokens through a DeepSeek-V3 w2
    (K 2048 -> N 7168, uint4, bf16) give a 4.7 GB C (A stays at 1.3 GB, under its 2 GiB bound); the
    last 8 rows of the first and the last expert, the latter past 2^32 bytes, against the oracle."""
    E, T, K, N = 80, 4096, 2048, 7168
    assert E * T * N * 2 > 2**32 and E * T * K * 2 < 2**31
    wl = synth.Workload("ep_big", E=E, H=N, I=K, topk=1, Ms=(1,), dtype="bf16", bits=4)
    layer = synth.make_layer(wl, seed=7, device="cuda")
    A = (torch.randn((E, T, K), generator=torch.Generator(device="cuda").manual_seed(8),
                     device="cuda") * 0.1).to(torch.bfloat16)
    counts = torch.full((E,), T, dtype=torch.int32, device="cuda")
    print("batched gemm with a 4.7 GB output", flush=True)
    C = B.moe_wna16_batched_gemm(A, counts, layer["w2"], layer["w2_scales"], layer["w2_zeros"],
                                 act=0)
    torch.cuda.synchronize()
    for e in (0, E - 1):
        sub = {k: (v[e:e + 1].cpu() if v is not None else None) for k, v in layer.items()}
        src = O.ExpertSource(sub, 4)
        ref = O.batched_gemm(A[e:e + 1, T - 8:].cpu(), np.array([8]), src.w2, act=0)
        keys = sorted(ref)
        assert_layer_close(torch.stack([C[e, T - 8 + r].cpu() for _, r in keys]),
                           np.stack([ref[k] for k in keys]), f"expert {e}")
