"""Plain CPU oracle of the fused MoE layer with weight-only quantised experts (w4a16 / w8a16).

TEST INFRASTRUCTURE ONLY (imported by tests, the smoke check and the benchmark's CPU baseline).
It shares no code with the GPU library and is deliberately slow: numpy, float64 for the layer
arithmetic, Python loops where the definition is a loop.

What it computes, and where each step is defined:

* Storage decoding of the expert weights.  "[Kernel] add triton fused moe kernel for gptq/awq"
  (review thread: the kernel takes its own weight format that accepts GPTQ/AWQ checkpoints) and
  "[Kernel] optimize performance of gptq marlin kernel when n is small" (benchmark script: uint4,
  group size 128, integer zero point, has_zp=True, is_zp_float=False) fix the encoding family:
  w = (q - z) * s per group of 128 along K.  The int8 variant is symmetric with one scale per output
  channel and no zero point (the int8 MoE backend listing, make_int8_moe_quant_config: w8a16 config
  with w1_zp = w2_zp = None; _humming_int8_weight_schema: symmetric, strategy "channel").
  Nibble order and zero packing are not on the pages; the reading used is low nibble = even k.
* Routing.  The pages describe none; the workloads fix it: softmax top-k (renormalised), or
  DeepSeek-V3-style sigmoid scores with group-limited selection and a routed scaling factor.
* moe_align_block_size.  Named in the first PR's notes (shared-memory version for large expert
  counts, usable under CUDA graphs); its output format is not printed, the reading used is the
  plainest one (stable grouping by expert, each group padded to BLOCK_M with a sentinel).
* The expert FFN out[m] = sum_j w[m,j] * W2[e_mj] (SiLU(W1[e_mj] x_m) * W3[e_mj] x_m), with W1/W3 the
  gate/up halves of w13 (rows [0,I) and [I,2I)); the pages name the one-launch grouped GEMM that
  computes it (first PR, description).

Every reading the pages leave open is listed with its justification in the design notes.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GROUP = 128

__all__ = [
    "GROUP", "unpack_uint4", "dequant_uint4", "dequant_int8", "dequant_bits",
    "exp_f32_spec", "sigmoid_f32_spec", "route_softmax", "route_sigmoid_grouped", "route",
    "align_capacity", "align_block_size", "silu", "ExpertSource", "moe_layer", "moe_layer_rows",
    "grouped_gemm", "dense_gemm", "batched_gemm", "quant_int8_rows", "w8a8_grouped_gemm",
    "round_to_dtype", "moe_layer_w8a8_rows", "dequant_uint4_gidx", "to_numpy",
    "AWQ_PACK_ORDER", "unpack_gptq", "unpack_awq", "canonical_from_checkpoint",
]


def to_numpy(t):
    """torch tensor (any device, any dtype incl. bfloat16) -> numpy; bf16 arrives as float32."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        return np.asarray(t)
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy()
    return np.asarray(t)


# ================================================================================================
# storage decoding
# ================================================================================================
def unpack_uint4(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> uint8 [..., 2n]: element 2j is bits 0-3 of byte j, element 2j+1 bits 4-7."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant_uint4(qweight, scales, zeros) -> np.ndarray:
    """Exact dequantised weights (q - z) * s as float64 [N, K] for one expert.

    qweight uint8 [N, K/2], scales float [N, K/128], zeros uint8 [N, K/256]."""
    q = unpack_uint4(qweight).astype(np.float64)
    z = unpack_uint4(zeros).astype(np.float64)
    s = np.asarray(scales, dtype=np.float64)
    N, K = q.shape
    ng = K // GROUP
    assert s.shape == (N, ng) and z.shape == (N, ng), (s.shape, z.shape, (N, ng))
    return ((q.reshape(N, ng, GROUP) - z[..., None]) * s[..., None]).reshape(N, K)


def dequant_int8(qweight, scales) -> np.ndarray:
    """Exact dequantised weights q * s as float64 [N, K]; qweight int8 [N, K], scales [N]."""
    q = np.asarray(qweight, dtype=np.int8).astype(np.float64)
    s = np.asarray(scales, dtype=np.float64)
    return q * s[:, None]


def dequant_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round exact dequantised values to the activation dtype (round to nearest even).

    Returns the uint16 bit patterns.  The exact value (q - z) * s has at most 18 significant bits, so
    it is exact in float32 and one rounding from there is the correct rounding."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x64, dtype=np.float64))
    if dtype == "fp16":
        return x32.astype(np.float16).view(np.uint16)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ================================================================================================
# routing
# ================================================================================================
# e^x in float32, specified operation by operation so that any two IEEE-754 implementations that
# follow it produce the same bits: clamp x to [-80, 80]; n = rint(x * log2(e)); Cody-Waite two-part
# reduction r = (x - n*C1) - n*C2 with C1 = 355/512 and C2 = ln2 - C1 (rounded to float32); degree-7
# Taylor polynomial of e^r in Horner form with coefficients 1/i! rounded to float32; scale by 2^n.
# Every step is one float32 operation rounded to nearest even, in exactly this order, never fused.
_LOG2E = np.float32(1.4426950408889634)
_C1 = np.float32(355.0 / 512.0)
_C2 = np.float32(math.log(2.0) - 355.0 / 512.0)
_INV_FACT = [np.float32(1.0 / math.factorial(i)) for i in range(8)]


def exp_f32_spec(x) -> np.ndarray:
    x = np.clip(np.asarray(x, dtype=np.float32), np.float32(-80.0), np.float32(80.0))
    n = np.rint(x * _LOG2E)
    r = (x - n * _C1) - n * _C2
    p = _INV_FACT[7]
    for i in range(6, -1, -1):
        p = p * r + _INV_FACT[i]      # separate multiply then add (numpy never fuses)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def sigmoid_f32_spec(x) -> np.ndarray:
    """1 / (1 + e^-x) in float32 with the exp above and a correctly rounded division."""
    e = exp_f32_spec(-np.asarray(x, dtype=np.float32))
    return (np.float32(1.0) / (np.float32(1.0) + e)).astype(np.float32)


def route_softmax(logits, topk: int, renormalize: bool = True, scale: float = 1.0):
    """Softmax top-k.  ids: the k largest logits, descending, ties to the lower expert id (softmax is
    monotone, so ranking logits ranks probabilities without rounding).  weights (float64): the
    softmax probabilities of the chosen experts, divided by their sum when renormalising, times the
    routed scaling factor."""
    lg = np.asarray(logits, dtype=np.float32)
    M, E = lg.shape
    ids = np.zeros((M, topk), np.int32)
    w = np.zeros((M, topk), np.float64)
    for m in range(M):
        row = lg[m]
        order = sorted(range(E), key=lambda e: (-float(row[e]), e))[:topk]
        l64 = row.astype(np.float64)
        p = np.exp(l64 - l64.max())
        p /= p.sum()
        sel = p[order]
        if renormalize:
            sel = sel / sel.sum()
        ids[m] = order
        w[m] = sel * scale
    return ids, w


def route_sigmoid_grouped(logits, topk: int, num_groups: int, topk_groups: int,
                          renormalize: bool = True, scale: float = 1.0):
    """DeepSeek-V3-style group-limited routing on sigmoid scores.

    1. sigma = sigmoid_f32_spec(logit) per expert (float32: these values decide which ids win).
    2. Experts form num_groups contiguous groups; a group's score is the float32 sum of its two
       largest sigma (its single sigma if the group has one expert).
    3. Keep the topk_groups best groups (descending score, ties to the lower group id).
    4. ids = the topk largest sigma inside kept groups (descending, ties to the lower expert id).
    5. weights = sigma of the chosen experts / their sum (if renormalising) * scale, in float64.
    """
    lg = np.asarray(logits, dtype=np.float32)
    M, E = lg.shape
    assert E % num_groups == 0
    gs = E // num_groups
    sig = sigmoid_f32_spec(lg)
    ids = np.zeros((M, topk), np.int32)
    w = np.zeros((M, topk), np.float64)
    for m in range(M):
        s = sig[m]
        gscore = []
        for g in range(num_groups):
            members = sorted((float(v) for v in s[g * gs:(g + 1) * gs]), reverse=True)
            if gs >= 2:
                gscore.append(np.float32(members[0]) + np.float32(members[1]))
            else:
                gscore.append(np.float32(members[0]))
        kept = set(sorted(range(num_groups), key=lambda g: (-float(gscore[g]), g))[:topk_groups])
        cand = [e for e in range(E) if e // gs in kept]
        sel = sorted(cand, key=lambda e: (-float(s[e]), e))[:topk]
        v = s[sel].astype(np.float64)
        if renormalize:
            v = v / v.sum()
        ids[m] = sel
        w[m] = v * scale
    return ids, w


def route(logits, topk, score="softmax", renormalize=True, num_groups=1, topk_groups=1, scale=1.0):
    if score == "softmax":
        assert num_groups == 1
        return route_softmax(logits, topk, renormalize, scale)
    return route_sigmoid_grouped(logits, topk, num_groups, topk_groups, renormalize, scale)


# ================================================================================================
# moe_align_block_size
# ================================================================================================
def align_capacity(numel: int, E: int, block_m: int) -> int:
    """Largest possible padded length: every non-empty expert adds at most block_m - 1 padding."""
    return numel + min(E, numel) * (block_m - 1)


def align_block_size(topk_ids, E: int, block_m: int, capacity: int | None = None):
    """Group token-slots by expert and pad each group to a multiple of block_m.

    Slot s = m * topk + j.  For experts in ascending order, the slots routed to expert e are listed
    in ascending slot order, followed by sentinel entries (value numel) up to the next multiple of
    block_m; an expert with no slots takes no space.  Entries from the padded total T up to the
    capacity are sentinels too.  expert_ids[b] is the expert of block b (entries b*block_m ...), or -1
    for blocks at or beyond T.  Ids outside [0, E) are not listed.
    Returns (sorted_token_ids int32 [cap], expert_ids int32 [ceil(cap/block_m)], T).
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    numel = flat.size
    cap = align_capacity(numel, E, block_m) if capacity is None else capacity
    sorted_ids = np.full(cap, numel, dtype=np.int32)
    expert_ids = np.full(-(-cap // block_m), -1, dtype=np.int32)
    pos = 0
    for e in range(E):
        slots = np.nonzero(flat == e)[0]
        if slots.size == 0:
            continue
        padded = -(-slots.size // block_m) * block_m
        sorted_ids[pos:pos + slots.size] = slots
        expert_ids[pos // block_m:(pos + padded) // block_m] = e
        pos += padded
    return sorted_ids, expert_ids, pos


# ================================================================================================
# expert FFN and the layer
# ================================================================================================
def silu(v):
    return v / (1.0 + np.exp(-v))


class ExpertSource:
    """Serves exact float64 dequantised weights of one expert at a time.

    `layer` maps w13, w13_scales, w13_zeros, w2, w2_scales, w2_zeros to arrays indexed by the
    position in `experts` (default: position = expert id)."""

    def __init__(self, layer: dict, bits: int, experts=None):
        self.layer = {k: (to_numpy(v) if v is not None else None) for k, v in layer.items()}
        self.bits = bits
        self.index = None if experts is None else {int(e): i for i, e in enumerate(experts)}

    def _i(self, e):
        return int(e) if self.index is None else self.index[int(e)]

    def _deq(self, name, i):
        L = self.layer
        if self.bits == 4:
            return dequant_uint4(L[name][i], L[name + "_scales"][i], L[name + "_zeros"][i])
        return dequant_int8(L[name][i], L[name + "_scales"][i])

    def w13(self, e):
        return self._deq("w13", self._i(e))

    def w2(self, e):
        return self._deq("w2", self._i(e))


def _per_expert(experts, fn, workers):
    """[fn(e) for e in experts], on `workers` threads when > 1 (each call is independent; numpy
    releases the interpreter lock inside its array operations).  The threads then run the BLAS
    products single-threaded, so they do not compete with BLAS's own threads."""
    if workers <= 1:
        return [fn(e) for e in experts]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    with ThreadPoolExecutor(max_workers=workers) as ex:
        if threadpool_limits is None:
            return list(ex.map(fn, experts))
        with threadpool_limits(1):
            return list(ex.map(fn, experts))


def moe_layer_rows(x, topk_ids, topk_weights, src: ExpertSource, rows=None, workers: int = 1):
    """out[m] = sum_j w[m,j] * W2[e] (SiLU(gate_e x_m) * up_e x_m) for the token rows `rows`.

    Float64 throughout; the per-slot results are summed over j in ascending order.  The experts
    are independent, so `workers` > 1 evaluates them on that many threads (same arithmetic).
    Returns (out float64 [len(rows), H], per-slot y float64 [len(rows), topk, H])."""
    x64 = np.asarray(to_numpy(x), dtype=np.float64)
    ids = np.asarray(to_numpy(topk_ids), dtype=np.int64)
    wts = np.asarray(to_numpy(topk_weights), dtype=np.float64)
    rows = np.arange(ids.shape[0]) if rows is None else np.asarray(rows)
    k = ids.shape[1]
    sub = ids[rows]

    def expert(e):
        W13 = src.w13(e)
        W2 = src.w2(e)
        I = W13.shape[0] // 2
        rr, jj = np.nonzero(sub == e)
        h = x64[rows[rr]] @ W13.T                 # each row is one token's product with expert e
        a = silu(h[:, :I]) * h[:, I:]
        return rr, jj, a @ W2.T

    y = None
    for rr, jj, ye in _per_expert(sorted(set(sub.reshape(-1).tolist())), expert, workers):
        if y is None:
            y = np.zeros((len(rows), k, ye.shape[1]), np.float64)
        y[rr, jj] = ye
    out = np.zeros((len(rows), y.shape[2]), np.float64)
    for j in range(k):
        out += wts[rows, j][:, None] * y[:, j]
    return out, y


def moe_layer(x, topk_ids, topk_weights, src: ExpertSource):
    return moe_layer_rows(x, topk_ids, topk_weights, src)[0]


def grouped_gemm(A, a_row_div: int, weight_of, sorted_token_ids, expert_ids, num_tokens_post_padded,
                 block_m: int, num_slots: int, topk_weights=None, act: int = 0):
    """The grouped GEMM over align output, as a definition.

    For every listed slot s at position p < T: e = expert_ids[p // block_m],
    h = A[s // a_row_div] @ W[e]^T (float64); with act == 1, c = SiLU(h[:N/2]) * h[N/2:], else c = h;
    times topk_weights[s] if given.  Returns ({slot: row float64}) for the listed slots."""
    A64 = np.asarray(to_numpy(A), dtype=np.float64)
    st = np.asarray(sorted_token_ids)
    ex = np.asarray(expert_ids)
    tw = None if topk_weights is None else np.asarray(to_numpy(topk_weights), np.float64).reshape(-1)
    out = {}
    cache = {}
    for p in range(int(num_tokens_post_padded)):
        s = int(st[p])
        if s >= num_slots:
            continue
        e = int(ex[p // block_m])
        if e not in cache:
            cache[e] = weight_of(e)
        W = cache[e]
        h = W @ A64[s // a_row_div]
        if act == 1:
            n2 = W.shape[0] // 2
            h = silu(h[:n2]) * h[n2:]
        if tw is not None:
            h = h * tw[s]
        out[s] = h
    return out


def dense_gemm(A, qweight, scales, zeros=None):
    """The dense weight-only GEMM, as a definition: C = A @ W^T in float64, W the exact decoded
    weights of one weight matrix (uint4 g128 with integer zero points when zeros are given, int8
    with one scale per row otherwise).

    This is the one-expert, every-row-routed case of the grouped GEMM, and the operation the small-n
    GEMM benchmark of "[Kernel] optimize performance of gptq marlin kernel when n is small" times
    (benchmark script and table: m 16, k 8192, n 128 ... 32768, uint4, group 128, integer zero point).
    A [M, K]; qweight uint8 [N, K/2] or int8 [N, K]; scales [N, K/128] or [N]; returns [M, N]."""
    A64 = np.asarray(to_numpy(A), dtype=np.float64)
    if zeros is not None:
        W = dequant_uint4(to_numpy(qweight), to_numpy(scales), to_numpy(zeros))
    else:
        W = dequant_int8(to_numpy(qweight), to_numpy(scales))
    assert A64.shape[1] == W.shape[1], (A64.shape, W.shape)
    return A64 @ W.T


def batched_gemm(A, expert_num_tokens, weight_of, act: int = 0):
    """The grouped GEMM over activations already batched per expert, as a definition.

    The int8 MoE backend listing hands the experts their activations in the BatchedExperts format
    (select_int8_moe_backend, make_int8_moe_kernel: sized by a per-rank max_num_tokens); the pages
    print no layout, and the reading used is the plainest one: A [E, T, K] where rows r <
    expert_num_tokens[e] of expert e are tokens routed to it (T = max_num_tokens).  For each expert e
    and valid row r: h = A[e, r] @ W[e]^T (float64), with act == 1 c = SiLU(h[:N/2]) * h[N/2:],
    else c = h.  Returns {(e, r): row float64} for the valid rows only."""
    A64 = np.asarray(to_numpy(A), dtype=np.float64)
    counts = np.asarray(to_numpy(expert_num_tokens)).astype(np.int64)
    E, T = A64.shape[0], A64.shape[1]
    out = {}
    for e in range(E):
        n = int(min(max(counts[e], 0), T))
        if n == 0:
            continue
        W = weight_of(e)
        for r in range(n):
            h = W @ A64[e, r]
            if act == 1:
                n2 = W.shape[0] // 2
                h = silu(h[:n2]) * h[n2:]
            out[(e, r)] = h
    return out


def quant_int8_rows(x):
    """Dynamic symmetric int8 quantisation with one scale per row (per token), as a definition.

    The int8 MoE backend listing pairs int8 weights with activations quantised per token at run time
    (activation key kInt8DynamicTokenSym; int8_w8a8_moe_quant_config with per_act_token_quant); the
    pages print no formula, and the reading used is the plain symmetric one, in float32 (the
    precision the codes are decided in on the GPU): s = max|x_row| / 127 (one correctly rounded
    division), q = clamp(rint(x / s), -127, 127) with rint = round half to even; a row of zeros has
    s = 0 and q = 0.  x [R, K] (any float dtype) -> (q int8 [R, K], s float32 [R])."""
    x32 = np.asarray(to_numpy(x), dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    q = np.zeros(x32.shape, np.int8)
    nz = s > 0
    if nz.any():
        r = np.rint(x32[nz] / s[nz][:, None])          # float32 division, then round half to even
        q[nz] = np.clip(r, -127, 127).astype(np.int8)
    return q, s


def w8a8_grouped_gemm(Aq, a_scales, a_row_div: int, w_of, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, block_m: int, num_slots: int, topk_weights=None,
                      act: int = 0):
    """The grouped GEMM with int8 activations and int8 weights, as a definition.

    For every listed slot s (as in grouped_gemm): row = s // a_row_div, e = the block's expert,
    h[n] = (sum_k Aq[row, k] * qw[e, n, k]) * a_scales[row] * w_scales[e, n] (the integer sum is exact;
    float64 afterwards); act == 1: SiLU(h[:N/2]) * h[N/2:]; times topk_weights[s] if given.
    w_of(e) -> (qw int8 [N, K], w_scales [N]).  Returns {slot: row float64}."""
    Aq = np.asarray(to_numpy(Aq)).astype(np.int64)
    sa = np.asarray(to_numpy(a_scales), dtype=np.float64)
    st = np.asarray(sorted_token_ids)
    ex = np.asarray(expert_ids)
    tw = None if topk_weights is None else np.asarray(to_numpy(topk_weights), np.float64).reshape(-1)
    out = {}
    cache = {}
    for p in range(int(num_tokens_post_padded)):
        s = int(st[p])
        if s >= num_slots:
            continue
        e = int(ex[p // block_m])
        if e not in cache:
            qw, ws = w_of(e)
            cache[e] = (np.asarray(to_numpy(qw)).astype(np.int64),
                        np.asarray(to_numpy(ws), dtype=np.float64))
        qw, ws = cache[e]
        row = s // a_row_div
        h = (qw @ Aq[row]).astype(np.float64) * sa[row] * ws
        if act == 1:
            n2 = qw.shape[0] // 2
            h = silu(h[:n2]) * h[n2:]
        if tw is not None:
            h = h * tw[s]
        out[s] = h
    return out


def round_to_dtype(x64, dtype: str) -> np.ndarray:
    """Values rounded to fp16 or bf16 (through float32, round to nearest even), as float64."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    u = x32.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def moe_layer_w8a8_rows(x, topk_ids, topk_weights, layer: dict, dtype: str, rows=None,
                        workers: int = 1):
    """The layer with int8 experts and per-token int8 activations, as a definition.

    For token m and its j-th expert e: (xq, xs) = quant_int8_rows(x[m]);
    h = (W13q[e] @ xq) * xs * W13s[e]; a = SiLU(h[:I]) * h[I:] rounded to the activation dtype (the
    rows the two GEMMs exchange); (aq, as) = quant_int8_rows(a); y = (W2q[e] @ aq) * as * W2s[e];
    out[m] = sum_j w[m, j] * y_j (j ascending).  The integer sums are exact: they are formed in
    float64, where every partial sum of products of codes in [-127, 127] is an integer far below
    2^53; float64 elsewhere.  The (token, j) pairs of one expert are evaluated together (each row
    of a product is that pair's own sum), on `workers` threads across experts when > 1.
    layer: w13 int8 [E, 2I, H], w13_scales [E, 2I], w2 int8 [E, H, I], w2_scales [E, H]."""
    xs_all = np.asarray(to_numpy(x), dtype=np.float32)
    ids = np.asarray(to_numpy(topk_ids), dtype=np.int64)
    wts = np.asarray(to_numpy(topk_weights), dtype=np.float64)
    rows = np.arange(ids.shape[0]) if rows is None else np.asarray(rows)
    L = {k: np.asarray(to_numpy(v)) for k, v in layer.items() if v is not None}
    H = xs_all.shape[1]
    k = ids.shape[1]
    sub = ids[rows]
    assert H <= 131072 and L["w2"].shape[2] <= 131072        # 127^2 * K far below 2^53
    xq, xsc = quant_int8_rows(xs_all[rows])                  # per token: one row each

    def expert(e):
        rr, jj = np.nonzero(sub == e)
        w13q = L["w13"][e].astype(np.float64)
        I = w13q.shape[0] // 2
        h = (xq[rr].astype(np.float64) @ w13q.T) * xsc[rr].astype(np.float64)[:, None] * \
            L["w13_scales"][e].astype(np.float64)[None, :]
        a = round_to_dtype(silu(h[:, :I]) * h[:, I:], dtype)
        aq, asc = quant_int8_rows(a.astype(np.float32))
        y = (aq.astype(np.float64) @ L["w2"][e].astype(np.float64).T) * \
            asc.astype(np.float64)[:, None] * L["w2_scales"][e].astype(np.float64)[None, :]
        return rr, jj, y

    ys = np.zeros((len(rows), k, H), np.float64)
    for rr, jj, y in _per_expert(sorted(set(sub.reshape(-1).tolist())), expert, workers):
        ys[rr, jj] = y
    out = np.zeros((len(rows), H), np.float64)
    for j in range(k):
        out += wts[rows, j][:, None] * ys[:, j]
    return out


def dequant_uint4_gidx(qweight, scales, zeros, g_idx) -> np.ndarray:
    """Exact decoded weights of one expert whose input columns carry a group index (GPTQ act-order).

    The GEMM of "[Kernel] optimize performance of gptq marlin kernel when n is small" takes a
    g_idx and a sort_indices argument (its benchmark passes them empty); the reading used: input
    column k belongs to quantisation group g_idx[k] (128 columns per group, in any order), so
    w[n, k] = (q[n, k] - z[n, g_idx[k]]) * s[n, g_idx[k]] in float64, columns in their original order.
    qweight uint8 [N, K/2] (original column order), scales [N, K/128], zeros uint8 [N, K/256]."""
    q = unpack_uint4(to_numpy(qweight)).astype(np.float64)
    z = unpack_uint4(to_numpy(zeros)).astype(np.float64)
    s = np.asarray(to_numpy(scales), dtype=np.float64)
    g = np.asarray(to_numpy(g_idx)).astype(np.int64)
    assert q.shape[1] == g.shape[0] and g.min() >= 0 and g.max() < s.shape[1]
    return (q - z[:, g]) * s[:, g]



# ================================================================================================
# GPTQ / AWQ checkpoint storage -> the canonical storage
# ================================================================================================
# The review thread of "[Kernel] add triton fused moe kernel for gptq/awq" asks for a weight format
# that accepts GPTQ and AWQ checkpoints, and the small-n GEMM of "[Kernel] optimize performance of
# gptq marlin kernel when n is small" takes a g_idx and sort_indices; the pages print neither
# checkpoint's packing.  The reading used (the layouts those checkpoint families ship), per expert:
#   GPTQ: qweight int32 [K/8, N], code (k, n) in bits 4 (k % 8) .. + 3 of word [k / 8, n];
#         qzeros int32 [K/128, N/8], zero (g, n) in bits 4 (n % 8) of word [g, n / 8];
#         scales [K/128, N]; optional g_idx int32 [K] (act-order: the group of input column k).
#   AWQ:  qweight int32 [K, N/8], code (k, n) in nibble j of word [k, n / 8] where column
#         n % 8 = AWQ_PACK_ORDER[j]; qzeros int32 [K/128, N/8] packed the same way; scales [K/128, N].
# Zero points are stored as they are (no offset); decoded weight (q - z) * s.
AWQ_PACK_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def _nibble(words, j):
    return (np.asarray(words, dtype=np.int64) >> (4 * j)) & 0xF


def unpack_gptq(qweight, qzeros):
    """GPTQ words -> (q uint8 [K, N], z uint8 [K/128, N]) for one expert."""
    qw = np.asarray(to_numpy(qweight)).astype(np.int64) & 0xFFFFFFFF
    qz = np.asarray(to_numpy(qzeros)).astype(np.int64) & 0xFFFFFFFF
    K8, N = qw.shape
    q = np.empty((8 * K8, N), np.uint8)
    for j in range(8):                       # k = 8 * row + j
        q[j::8, :] = _nibble(qw, j)
    G, N8 = qz.shape
    z = np.empty((G, 8 * N8), np.uint8)
    for j in range(8):                       # n = 8 * word + j
        z[:, j::8] = _nibble(qz, j)
    return q, z


def unpack_awq(qweight, qzeros):
    """AWQ words -> (q uint8 [K, N], z uint8 [K/128, N]) for one expert."""
    qw = np.asarray(to_numpy(qweight)).astype(np.int64) & 0xFFFFFFFF
    qz = np.asarray(to_numpy(qzeros)).astype(np.int64) & 0xFFFFFFFF
    K, N8 = qw.shape
    q = np.empty((K, 8 * N8), np.uint8)
    z = np.empty((qz.shape[0], 8 * N8), np.uint8)
    for j, c in enumerate(AWQ_PACK_ORDER):   # nibble j holds column 8 * word + c
        q[:, c::8] = _nibble(qw, j)
        z[:, c::8] = _nibble(qz, j)
    return q, z


def canonical_from_checkpoint(q, z, scales, g_idx=None):
    """(q [K, N], z [G, N], scales [G, N], g_idx [K] or None) of one expert -> the canonical storage
    (qweight uint8 [N, K/2] with k = 2j in the low nibble of byte j, scales [N, G], zeros uint8
    [N, G/2] with group 2j in the low nibble of byte j) and, with g_idx, perm int32 [K]: the stable
    argsort of g_idx, the storage then holding column perm[j] at position j (the sorted storage of
    the act-order layer, whose group g is positions 128 g .. 128 g + 127)."""
    q = np.asarray(q, dtype=np.uint8)
    z = np.asarray(z, dtype=np.uint8)
    perm = None
    if g_idx is not None:
        perm = np.argsort(np.asarray(to_numpy(g_idx)).astype(np.int64), kind="stable")
        q = q[perm, :]
    qt = q.T                                  # [N, K]
    packed = (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)
    zt = z.T                                  # [N, G]
    zpacked = (zt[:, 0::2] | (zt[:, 1::2] << 4)).astype(np.uint8)
    sc = np.ascontiguousarray(np.asarray(to_numpy(scales)).T)
    return packed, sc, zpacked, (None if perm is None else perm.astype(np.int32))
