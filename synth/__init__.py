"""Seeded synthetic inputs for the fused mixture-of-experts layer.

This module is shared by the tests, the smoke check and the benchmark.  It holds no step of the
layer itself (no routing, grouping, dequantisation, GEMM, activation or combine).  It only

* describes the workloads (expert count, hidden and intermediate sizes, top-k, routing rule),
* draws weights, activations and router logits from seeded generators, and
* stores the drawn weights in the packed formats the layer consumes, the way a GPTQ/AWQ
  checkpoint arrives (uint4 with per-group-of-128 scales and integer zero points, or int8 with
  one symmetric scale per output channel).

Storage formats (row-major, little-endian):

int4  qweight uint8 [E, N, K/2]   byte j of a row holds k = 2j in bits 0-3 and k = 2j+1 in bits 4-7
      scales  fp16|bf16 [E, N, K/128]
      zeros   uint8 [E, N, K/256]   byte j holds the zero of group 2j (bits 0-3) and 2j+1 (bits 4-7)
int8  qweight int8 [E, N, K]
      scales  fp16|bf16 [E, N]

Every tensor is drawn with torch on the requested device: on the CPU the bytes are identical on
every machine; on a GPU the same seed gives a different (but again reproducible) draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch

GROUP = 128

_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One synthetic MoE layer shape and its routing rule."""

    name: str
    E: int
    H: int
    I: int
    topk: int
    Ms: tuple
    dtype: str = "fp16"          # activations, outputs and scales
    bits: int = 4                # 4: uint4 g128 asymmetric, 8: int8 per-channel symmetric
    score: str = "softmax"       # "softmax" or "sigmoid"
    renormalize: bool = True
    num_groups: int = 1
    topk_groups: int = 1
    scale: float = 1.0           # routed scaling factor
    logit_bias: bool = False     # add a per-expert N(0,1) bias to the logits (skewed loads)
    block_m: int = 0             # 0: let the library choose
    w_std: float = 0.02
    x_std: float = 0.1
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", E=8, H=256, I=512, topk=2, Ms=(16,), block_m=16,
                     notes="8 experts, hidden 256, intermediate 512, top-2, 16 tokens, BLOCK_M 16"),
    "mixtral": Workload("mixtral", E=8, H=4096, I=14336, topk=2, Ms=(1, 4, 16, 64),
                        notes="Mixtral-8x7B-shaped, int4 g128 asymmetric, top-2 softmax"),
    "qwen2": Workload("qwen2", E=64, H=3584, I=2560, topk=8, Ms=(1, 16, 128, 512), logit_bias=True,
                      notes="Qwen2-57B-A14B-shaped, top-8 softmax, per-expert logit bias"),
    "dsv3_tp8": Workload("dsv3_tp8", E=256, H=7168, I=256, topk=8, Ms=(1, 16, 64, 256),
                         score="sigmoid", num_groups=8, topk_groups=4, scale=2.5,
                         notes="DeepSeek-V3-shaped, one GPU's TP=8 share of the expert intermediate"),
    "dsv3_prefill_int4": Workload("dsv3_prefill_int4", E=256, H=7168, I=2048, topk=8, Ms=(1024, 4096),
                                  dtype="bf16", score="sigmoid", num_groups=8, topk_groups=4, scale=2.5,
                                  notes="DeepSeek-V3-shaped full expert, bf16, int4 g128"),
    "dsv3_prefill_int8": Workload("dsv3_prefill_int8", E=256, H=7168, I=2048, topk=8, Ms=(1024, 4096),
                                  dtype="bf16", bits=8, score="sigmoid", num_groups=8, topk_groups=4,
                                  scale=2.5, notes="DeepSeek-V3-shaped full expert, bf16, int8 per channel"),
}


# ----------------------------------------------------------------------------------------------
# seeded streams
# ----------------------------------------------------------------------------------------------
_TAGS = {"w13": 1, "w2": 2, "x": 3, "logits": 4, "bias": 5, "dense_w": 6, "dense_x": 7,
         "perm13": 8, "perm2": 9}


def stream_seed(seed: int, tag: str, idx: int = 0) -> int:
    """Independent seed for (run seed, tensor tag, expert index)."""
    v = (seed * 1_000_003 + _TAGS[tag]) * 1_000_003 + idx
    return v % (2**62)


def _gen(seed: int, tag: str, idx: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(stream_seed(seed, tag, idx))
    return g


def _randn(shape, seed, tag, idx, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, tag, idx, device), device=device,
                       dtype=torch.float32)


# ----------------------------------------------------------------------------------------------
# storage encoders (checkpoint format; the layer only ever decodes)
# ----------------------------------------------------------------------------------------------
def _round_up_to(v64: torch.Tensor, dtype) -> torch.Tensor:
    """Smallest value of `dtype` that is >= v64 (v64 > 0, finite)."""
    c = v64.to(torch.float32).to(dtype)  # any rounding lands within one ulp of v64
    bits = c.view(torch.int16)
    below = c.double() < v64
    c = torch.where(below, (bits + 1).view(dtype), c)
    bits = c.view(torch.int16)
    prev = (bits - 1).view(dtype)
    c = torch.where(prev.double() >= v64, prev, c)
    return c


def encode_uint4_g128(w: torch.Tensor, scale_dtype):
    """Asymmetric min/max uint4 encoding of w [N, K] in groups of 128 along K.

    Per group, in float64: lo/hi = min/max, s = (hi - lo)/15 rounded up to the scale dtype,
    z = clamp(rint(-lo/s), 0, 15), q = clamp(rint(w/s) + z, 0, 15) (rint = round half to even).
    Returns (qweight uint8 [N, K/2], scales [N, K/128], zeros uint8 [N, K/256]).
    """
    N, K = w.shape
    assert K % (2 * GROUP) == 0, "K must be a multiple of 256 so zeros pack two per byte"
    wg = w.double().reshape(N, K // GROUP, GROUP)
    lo = wg.amin(-1)
    hi = wg.amax(-1)
    assert bool((hi > lo).all()), "degenerate group (all weights equal)"
    s = _round_up_to((hi - lo) / 15.0, scale_dtype)
    sd = s.double()
    z = torch.clamp(torch.round(-lo / sd), 0, 15)
    q = torch.clamp(torch.round(wg / sd[..., None]) + z[..., None], 0, 15)
    q = q.to(torch.uint8).reshape(N, K)
    qpacked = q[:, 0::2] | (q[:, 1::2] << 4)
    zq = z.to(torch.uint8)
    zpacked = zq[:, 0::2] | (zq[:, 1::2] << 4)
    return qpacked.contiguous(), s.contiguous(), zpacked.contiguous()


def encode_int8_channel(w: torch.Tensor, scale_dtype):
    """Symmetric int8 encoding of w [N, K], one scale per output row.

    s = max|w| / 127 rounded up to the scale dtype; q = clamp(rint(w/s), -127, 127).
    Returns (qweight int8 [N, K], scales [N]).
    """
    w64 = w.double()
    amax = w64.abs().amax(-1)
    assert bool((amax > 0).all())
    s = _round_up_to(amax / 127.0, scale_dtype)
    q = torch.clamp(torch.round(w64 / s.double()[:, None]), -127, 127).to(torch.int8)
    return q.contiguous(), s.contiguous()


# ----------------------------------------------------------------------------------------------
# layer tensors
# ----------------------------------------------------------------------------------------------
def expert_weights_fp32(wl: Workload, e: int, seed: int = 0, device="cpu"):
    """The unquantised draws of expert e: w13 [2I, H] (gate rows then up rows) and w2 [H, I]."""
    w13 = _randn((2 * wl.I, wl.H), seed, "w13", e, device) * wl.w_std
    w2 = _randn((wl.H, wl.I), seed, "w2", e, device) * wl.w_std
    return w13, w2


def make_layer(wl: Workload, seed: int = 0, device="cpu", experts=None) -> dict:
    """Quantised expert weights for all experts (or only the listed ones, stacked in that order).

    Returns a dict with keys w13, w13_scales, w13_zeros, w2, w2_scales, w2_zeros
    (zeros are None for int8).
    """
    ids = range(wl.E) if experts is None else list(experts)
    dt = wl.torch_dtype
    parts = {k: [] for k in ("w13", "w13_scales", "w13_zeros", "w2", "w2_scales", "w2_zeros")}
    for e in ids:
        w13, w2 = expert_weights_fp32(wl, e, seed, device)
        for name, w in (("w13", w13), ("w2", w2)):
            if wl.bits == 4:
                q, s, z = encode_uint4_g128(w, dt)
                parts[name].append(q)
                parts[name + "_scales"].append(s)
                parts[name + "_zeros"].append(z)
            else:
                q, s = encode_int8_channel(w, dt)
                parts[name].append(q)
                parts[name + "_scales"].append(s)
        del w13, w2
    out = {k: (torch.stack(v) if v else None) for k, v in parts.items()}
    return out


def make_x(wl: Workload, M: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Activations [M, H]: N(0, x_std^2) drawn in fp32, rounded to the activation dtype.

    Smaller M takes the leading rows of the same draw."""
    mmax = max(max(wl.Ms), M)
    x = _randn((mmax, wl.H), seed, "x", 0, device) * wl.x_std
    return x[:M].to(wl.torch_dtype).contiguous()


def make_logits(wl: Workload, M: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router logits [M, E] fp32: N(0,1), plus a per-expert N(0,1) bias when the workload asks."""
    mmax = max(max(wl.Ms), M)
    lg = _randn((mmax, wl.E), seed, "logits", 0, device)[:M]
    if wl.logit_bias:
        lg = lg + _randn((wl.E,), seed, "bias", 0, device)[None, :]
    return lg.contiguous()


def weight_bytes_per_expert(wl: Workload) -> int:
    """Packed weight + scale + zero bytes of one expert (w13 and w2)."""
    def one(N, K):
        if wl.bits == 4:
            return N * K // 2 + 2 * N * (K // GROUP) + N * (K // (2 * GROUP))
        return N * K + 2 * N
    return one(2 * wl.I, wl.H) + one(wl.H, wl.I)


def w13_bytes_per_expert(wl: Workload) -> int:
    N, K = 2 * wl.I, wl.H
    if wl.bits == 4:
        return N * K // 2 + 2 * N * (K // GROUP) + N * (K // (2 * GROUP))
    return N * K + 2 * N


# ----------------------------------------------------------------------------------------------
# dense GEMM inputs (one weight matrix): the small-n benchmark's shapes, m 16, k 8192, n 128..32768
# ----------------------------------------------------------------------------------------------
def make_dense(M: int, N: int, K: int, bits: int = 4, dtype: str = "fp16", seed: int = 0,
               device="cpu") -> dict:
    """A [M, K] = N(0, 0.1^2) rounded to dtype (the benchmark's activations, randn / 10); weights
    N(0, 0.02^2) [N, K] encoded as the layer's experts (uint4 g128 asymmetric, or int8 per row)."""
    dt = _DT[dtype]
    A = (_randn((M, K), seed, "dense_x", 0, device) * 0.1).to(dt)
    w = _randn((N, K), seed, "dense_w", 0, device) * 0.02
    if bits == 4:
        qw, sc, zp = encode_uint4_g128(w, dt)
    else:
        qw, sc = encode_int8_channel(w, dt)
        zp = None
    return {"A": A, "B": qw, "scales": sc, "zeros": zp}


# ----------------------------------------------------------------------------------------------
# act-order layers: every expert's input columns grouped by a seeded random permutation
# ----------------------------------------------------------------------------------------------
def make_layer_act_order(wl: Workload, seed: int = 0, device="cpu") -> dict:
    """uint4 g128 experts whose quantisation groups are sets of 128 input columns in any order (GPTQ
    act-order), in the sorted storage the layer reads: for expert e, perm[e] lists the original
    input columns in group order (group g = perm[e][128g : 128g + 128]), and the codes, scales and
    zero points are those of the drawn weights with their columns taken in that order.
    Adds w13_perm int32 [E, H] and w2_perm int32 [E, I] to the usual tensors."""
    assert wl.bits == 4
    dt = wl.torch_dtype
    out = {k: [] for k in ("w13", "w13_scales", "w13_zeros", "w2", "w2_scales", "w2_zeros",
                           "w13_perm", "w2_perm")}
    for e in range(wl.E):
        w13, w2 = expert_weights_fp32(wl, e, seed, device)
        for name, w, tag in (("w13", w13, "perm13"), ("w2", w2, "perm2")):
            g = _gen(seed, tag, e, device)
            perm = torch.randperm(w.shape[1], generator=g, device=device)
            q, s, z = encode_uint4_g128(w[:, perm], dt)
            out[name].append(q)
            out[name + "_scales"].append(s)
            out[name + "_zeros"].append(z)
            out[name + "_perm"].append(perm.to(torch.int32))
    return {k: torch.stack(v).contiguous() for k, v in out.items()}

