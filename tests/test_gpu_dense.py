"""Dense weight-only GEMM (one weight matrix, every row routed) on the GPU vs the CPU oracle.

The shapes include the small-n GEMM benchmark of "[Kernel] optimize performance of gptq marlin kernel
when n is small" (m 16, k 8192, n 128 ... 32768), where K is split across workgroups."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_int4_topk_amd as B
from helpers import assert_layer_close

pytestmark = pytest.mark.gpu


def _run(d, dev=True):
    t = {k: (v.cuda() if v is not None else None) for k, v in d.items()} if dev else d
    C = B.moe_wna16_dense_gemm(t["A"], t["B"], t["scales"], t["zeros"])
    torch.cuda.synchronize()
    return C, t


def _oracle(d, cols=None):
    if cols is None:
        return O.dense_gemm(d["A"], d["B"], d["scales"], d["zeros"])
    z = None if d["zeros"] is None else O.to_numpy(d["zeros"])[cols]
    return O.dense_gemm(d["A"], O.to_numpy(d["B"])[cols], O.to_numpy(d["scales"])[cols], z)


@pytest.mark.parametrize("bits,dt", [(4, "fp16"), (4, "bf16"), (8, "fp16"), (8, "bf16")])
@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (7, 384, 1024), (16, 256, 8192),
                                   (33, 640, 512), (100, 128, 2048)])
def test_dense_vs_oracle(bits, dt, M, N, K):
    """Several column tiles and row blocks with ragged tails (M not a multiple of the block, N not
    of the four-tile workgroup), split and unsplit K."""
    d = synth.make_dense(M, N, K, bits, dt, seed=M + N)
    C, _ = _run(d)
    print(f"dense M={M} N={N} K={K} bits={bits} {dt}", flush=True)
    assert_layer_close(C, _oracle(d), f"dense M={M} N={N} K={K} bits={bits} {dt}")


@pytest.mark.parametrize("bits,dt", [(4, "fp16"), (4, "bf16"), (8, "bf16")])
def test_dense_identity_probe_bit_exact(bits, dt):
    """One-hot rows: row i of C is the decoded column k_i, which must equal the oracle's correctly
    rounded (q - z) * s bit for bit, also where K is split (the other splits add exact zeros)."""
    N, K = 256, 8192
    d = synth.make_dense(1, N, K, bits, dt, seed=3)
    ks = [0, 1, 127, 128, 4095, 4096, 8190, 8191] + list(range(1000, 1016))
    A = torch.zeros((len(ks), K), dtype=d["A"].dtype)
    A[torch.arange(len(ks)), torch.tensor(ks)] = 1
    d["A"] = A
    C, _ = _run(d)
    if bits == 4:
        W = O.dequant_uint4(O.to_numpy(d["B"]), O.to_numpy(d["scales"]), O.to_numpy(d["zeros"]))
    else:
        W = O.dequant_int8(O.to_numpy(d["B"]), O.to_numpy(d["scales"]))
    ref = O.dequant_bits(W[:, ks], dt).T
    got = C.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("n", [128, 1024, 4096, 32768])
def test_dense_benchmark_shapes_sampled(n):
    """m 16, k 8192 at the benchmark's n: every row, 256 sampled columns (the oracle decodes only
    those weight rows), plus bitwise determinism across two calls."""
    d = synth.make_dense(16, n, 8192, 4, "fp16", seed=0, device="cuda")
    C1, t = _run(d, dev=False)
    C2, _ = _run(d, dev=False)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), "not deterministic"
    cols = np.sort(np.random.default_rng(n).choice(n, size=min(n, 256), replace=False))
    host = {k: (v.cpu() if v is not None else None) for k, v in t.items()}
    print(f"dense benchmark shape n={n}", flush=True)
    assert_layer_close(O.to_numpy(C1)[:, cols], _oracle(host, cols), f"dense 16x8192x{n}")


def test_dense_empty_batch():
    d = synth.make_dense(1, 128, 256, 4, "fp16")
    t = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    C = B.moe_wna16_dense_gemm(t["A"][:0], t["B"], t["scales"], t["zeros"])
    torch.cuda.synchronize()
    assert C.shape == (0, 128)
