#!/usr/bin/env python
"""Throughput of the fused MoE layer with uint4/int8 experts on one MI355X; prints one JSON line.

A step is one call of the whole layer (routing, align, w13 grouped GEMM + SiLU*up, w2 grouped GEMM,
weighted combine) on one batch of M tokens whose inputs are already in HBM.  (One token, and two to
four tokens of the DeepSeek-V3 TP share, take the layer's dot-product paths instead: `layer_path`
in each workload row; their `w13_*` fields still time the grouped w13 GEMM alone.)  `value` is tokens/s
over exactly --steps steps of the Mixtral-shaped layer at M = 64, replayed as one HIP graph that
holds exactly --steps layer calls (after one graph of --warmup calls).  The layer exists in L device
copies that the calls cycle through, as a model's layer stack would, so that the experts a call
reads have been evicted from the 256 MiB Infinity Cache by the time the same copy comes round again.

Also reported: the roofline of the dominant kernel (the w13 grouped GEMM with the SiLU epilogue),
timed alone with HIP events on the stream it is launched on; `workloads`, every M of all five
workload shapes (the tiny layer, the Mixtral-, Qwen2- and DeepSeek-V3 TP-share decode layers, and
the DeepSeek-V3 full-expert prefill layer with uint4 and with int8 experts), each with its binding
roofline; the CPU oracle's throughput on a bounded sample of the headline batch, with all host
threads and with one; the dense uint4 GEMM at the small-n benchmark's shapes (m 16, k 8192, n 128
... 32768); the grouped GEMM over batched-experts activations on an expert-parallel share of 32
DeepSeek-V3-shaped experts; w8a8 (per-token int8 activations) against w8a16 on the DeepSeek-V3
int8 experts; and the layer with GPTQ act-order experts beside the plain layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
MIB = 1 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--m", type=int, default=0, help="tokens per step (default: largest decode M)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-workload table (every M of all five workload shapes)")
    ap.add_argument("--workloads", default="tiny,mixtral,qwen2,dsv3_tp8,dsv3_prefill_int4,"
                                           "dsv3_prefill_int8",
                    help="workloads of the per-workload table (comma-separated)")
    ap.add_argument("--sweep-steps", type=int, default=200,
                    help="layer calls per graph in the per-workload table and the side sweeps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the timed batch the CPU oracle runs (0: all of them; at the "
                         "default workload, every activated expert decoded once, ~10-20 s)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense uint4 GEMM sweep (m 16, k 8192, n 128 ... 32768)")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched-experts GEMM sweep (expert-parallel share, 32 experts)")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="skip the w8a8 vs w8a16 first-GEMM comparison (DeepSeek-V3 int8 experts)")
    ap.add_argument("--no-act-order", action="store_true",
                    help="skip the act-order layer sweep (same workload, permuted experts)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device-to-device copy (known bytes) so that "
                         "profiler traffic counters can be scaled")
    return ap.parse_args()


_HIP = None


def _graph_upload(g):
    """hipGraphUpload of a captured torch graph's executable graph on the current stream."""
    import ctypes

    import torch
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _HIP.hipGraphUpload.restype = ctypes.c_int
    rc = _HIP.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"hipGraphUpload failed ({rc})")


class GraphTimer:
    """Exactly `steps` calls cycling through fns (one per weight copy), captured as one HIP graph
    (uploaded to the device), and `warmup` calls captured as another.  time() replays the warmup
    graph untimed, then the timed graph once between HIP events on the current stream, and returns
    (seconds by the events, wall seconds, calls in the timed graph)."""

    def __init__(self, fns, steps, warmup):
        import torch
        self.torch = torch
        L = len(fns)
        for f in fns:                      # compile/warm every code path eagerly first
            f()
        torch.cuda.synchronize()

        def capture(n, first):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fns[(first + i) % L]()
            return g

        # the graphs hold raw device pointers: keep the calls (and so every tensor they use) alive
        # for as long as the graphs may be replayed
        self.fns = list(fns)
        self.timed = capture(steps, warmup)   # continues the rotation where the warmup stops
        _graph_upload(self.timed)
        self.warm = capture(warmup, 0) if warmup > 0 else None
        self.steps = steps

    def time(self):
        torch = self.torch
        if self.warm is not None:
            self.warm.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        t0 = time.perf_counter()
        self.timed.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end) / 1e3, wall, self.steps


def graph_replay(fns, steps, warmup):
    """GraphTimer(fns, steps, warmup).time()."""
    return GraphTimer(fns, steps, warmup).time()


class Bench:
    def __init__(self, wl, seed):
        import torch

        import synth
        import weight_only_int4_topk_amd as B
        self.torch, self.synth, self.B = torch, synth, B
        self.wl = wl
        self.seed = seed
        t0 = time.perf_counter()
        self.layer = synth.make_layer(wl, seed=seed, device="cuda")
        torch.cuda.synchronize()
        self.layer_bytes = sum(v.numel() * v.element_size() for v in self.layer.values()
                               if v is not None)
        log(f"[bench] drew {wl.name} layer ({self.layer_bytes / MIB:.0f} MiB) in "
            f"{time.perf_counter() - t0:.1f}s")
        self.copies = [self.layer]
        self.rt = B.routing(wl.score, wl.renormalize, wl.num_groups, wl.topk_groups, wl.scale)

    def ensure_copies(self, L):
        while len(self.copies) < L:
            self.copies.append({k: (v.clone() if v is not None else None)
                                for k, v in self.layer.items()})

    def n_copies(self, active_bytes):
        # between two uses of a copy, (L - 1) * active_bytes >= 512 MiB (twice the Infinity Cache)
        L = max(2, min(64, math.ceil(512 * MIB / max(active_bytes, 1)) + 1))
        cap = max(2, int((64 << 30) // self.layer_bytes))
        return min(L, cap)

    def measure(self, M, steps, warmup, defer=False):
        """Time the layer (and its w13 GEMM alone) at M tokens.  defer: capture the graphs now and
        return a function that times them later (with the GPU busy right before)."""
        torch, synth, B, wl = self.torch, self.synth, self.B, self.wl
        x = synth.make_x(wl, M, seed=self.seed, device="cuda")
        lg = synth.make_logits(wl, M, seed=self.seed, device="cuda")
        tw, ti = B.moe_topk_softmax(lg, wl.topk, self.rt)
        torch.cuda.synchronize()
        active = int(torch.unique(ti).numel())
        act_bytes = active * synth.weight_bytes_per_expert(wl)
        w13_bytes = active * synth.w13_bytes_per_expert(wl)
        L = self.n_copies(act_bytes)
        self.ensure_copies(L)
        bm = B.moe_pick_block_m(M, wl.E, wl.topk, wl.bits, wl.torch_dtype)
        quant = B.QUANT_INT4 if wl.bits == 4 else B.QUANT_INT8
        ws = torch.empty((B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, wl.E, wl.topk, quant,
                                                           wl.torch_dtype, 0),),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((M, wl.H), dtype=wl.torch_dtype, device="cuda")

        def layer_fn(c):
            return lambda: B.fused_moe_wna16(x, lg, wl.topk, self.rt, c["w13"], c["w13_scales"],
                                             c["w13_zeros"], c["w2"], c["w2_scales"],
                                             c["w2_zeros"], block_m=0, workspace=ws, out=out)

        g_layer = GraphTimer([layer_fn(c) for c in self.copies[:L]], steps, warmup)

        # the dominant kernel alone: w13 grouped GEMM with the SiLU epilogue, same tiles
        st, ex, npost = B.moe_align_block_size(ti, wl.E, bm)
        inter = torch.empty((M * wl.topk, wl.I), dtype=wl.torch_dtype, device="cuda")

        def gemm1_fn(c):
            return lambda: B.moe_wna16_gemm(x, wl.topk, c["w13"], c["w13_scales"], c["w13_zeros"],
                                            st, ex, npost, bm, M * wl.topk, act=1, C=inter)

        g_g1 = GraphTimer([gemm1_fn(c) for c in self.copies[:L]], steps, warmup)

        def finish():
            t_g1, _, _ = g_g1.time()
            t_layer, wall, G = g_layer.time()
            return self._result(M, bm, active, L, G, t_layer, t_g1, steps, act_bytes, w13_bytes), \
                t_layer, wall, (x, lg)

        return finish if defer else finish()

    def _result(self, M, bm, active, L, G, t_layer, t_g1, steps, act_bytes, w13_bytes):
        wl, B = self.wl, self.B
        us_layer = t_layer / steps * 1e6
        us_g1 = t_g1 / steps * 1e6
        flops_layer = 6.0 * wl.H * wl.I * M * wl.topk
        flops_g1 = 4.0 * wl.H * wl.I * M * wl.topk
        # binding roof of the layer: the larger of its HBM floor (activated experts' bytes at
        # 8 TB/s) and its MFMA floor (6 H I M k flops at 2.5 PFLOP/s)
        t_hbm = act_bytes / (HBM_PEAK_GBPS * 1e9)
        t_mfma = flops_layer / (MFMA_PEAK_TFLOPS * 1e12)
        path = {B.PATH_GROUPED: "grouped GEMMs", B.PATH_ONE_TOKEN: "one-token dot products",
                B.PATH_FEW_TOKENS: "few-token dot products"}[
            B.fused_moe_wna16_path(M, wl.H, wl.I, wl.E, wl.topk, wl.bits)]
        res = dict(
            M=M, layer_path=path, block_m=bm, active_experts=active, layer_copies=L,
            graph_calls=G,
            us_per_layer=round(us_layer, 2), tokens_per_s=round(M / (us_layer * 1e-6), 1),
            layer_GBps=round(act_bytes / (us_layer * 1e-6) / 1e9, 1),
            layer_hbm_frac=round(t_hbm / (us_layer * 1e-6), 4),
            layer_mfma_frac=round(t_mfma / (us_layer * 1e-6), 4),
            bound="mfma" if t_mfma > t_hbm else "hbm",
            frac=round(max(t_hbm, t_mfma) / (us_layer * 1e-6), 4),
            w13_us=round(us_g1, 2),
            w13_GBps=round(w13_bytes / (us_g1 * 1e-6) / 1e9, 1),
            w13_TFLOPs=round(flops_g1 / (us_g1 * 1e-6) / 1e12, 2),
            active_weight_bytes=act_bytes, w13_bytes=w13_bytes,
        )
        return res

    def release(self):
        self.copies = []
        self.layer = None
        self.torch.cuda.empty_cache()


DENSE_NS = (128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768)


def _decode_uint4_fp16(qw, scales, zeros):
    """[N, K/2] uint4 storage -> fp16 [N, K] decoded weights (q - z) * s, for the fp16 reference."""
    import torch
    N = qw.shape[0]
    q = torch.stack([qw & 15, qw >> 4], dim=-1).reshape(N, -1).float()
    z = torch.stack([zeros & 15, zeros >> 4], dim=-1).reshape(N, -1).float()
    K = q.shape[1]
    w = (q.view(N, K // 128, 128) - z[..., None]) * scales.float()[..., None]
    return w.reshape(N, K).to(torch.float16).contiguous()


def dense_sweep(steps, warmup, m=16, k=8192, seed=0):
    """The dense uint4 g128 GEMM (moe_wna16_dense_gemm) at the small-n benchmark's shapes: m 16,
    k 8192, fp16, n 128 ... 32768.  Time per call from graph replays cycling through copies of the
    weights (as the layer's copies), and the weight bytes streamed per second."""
    import torch

    import synth
    import weight_only_int4_topk_amd as B
    out = []
    for n in DENSE_NS:
        d = synth.make_dense(m, n, k, 4, "fp16", seed=seed, device="cuda")
        names = ("B", "scales", "zeros")
        wbytes = sum(d[t].numel() * d[t].element_size() for t in names)
        L = max(2, min(64, math.ceil(512 * MIB / wbytes) + 1))
        copies = [d] + [{t: d[t].clone() for t in names} for _ in range(L - 1)]
        ws_n = B.moe_wna16_dense_gemm_workspace_size(m, n, k, B.QUANT_INT4, torch.float16)
        ws = torch.empty((max(ws_n, 256),), dtype=torch.uint8, device="cuda")
        C = torch.empty((m, n), dtype=torch.float16, device="cuda")
        A = d["A"]
        fns = [(lambda w=w: B.moe_wna16_dense_gemm(A, w["B"], w["scales"], w["zeros"],
                                                   workspace=ws, C=C)) for w in copies]
        t, _, _ = graph_replay(fns, steps, warmup)
        us = t / steps * 1e6
        gbps = wbytes / (us * 1e-6) / 1e9
        # same-hardware reference: the plain fp16 GEMM with the weights stored decoded (torch's
        # linear, i.e. the vendor BLAS), as the benchmark's fp16 column; weight copies rotated alike
        w16 = _decode_uint4_fp16(d["B"], d["scales"], d["zeros"])
        L16 = max(2, min(64, math.ceil(512 * MIB / (w16.numel() * 2)) + 1))
        w16s = [w16] + [w16.clone() for _ in range(L16 - 1)]
        fns16 = [(lambda w=w: torch.nn.functional.linear(A, w, out=C)) for w in w16s]
        t16, _, _ = graph_replay(fns16, steps, warmup)
        us16 = t16 / steps * 1e6
        out.append({"m": m, "k": k, "n": n, "us": round(us, 2), "weight_GBps": round(gbps, 1),
                    "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                    "split_k": ws_n // (m * n * 4) if ws_n else 1, "weight_copies": L,
                    "fp16_gemm_us": round(us16, 2)})
        log(f"[bench] dense {out[-1]}")
        del copies, d, fns, A, w16, w16s, fns16
        torch.cuda.empty_cache()
    return out


def batched_sweep(steps, warmup, E=32, H=7168, I=2048, Ts=(8, 64), seed=0):
    """moe_wna16_batched_gemm on an expert-parallel share of the DeepSeek-V3 expert shape (32 local
    experts of H 7168, I 2048, uint4 g128, bf16), every expert with a full batch of T tokens: the w13
    GEMM with SiLU and the w2 GEMM, time per call from graph replays over rotated weight copies, and
    the weight bytes streamed per second."""
    import torch

    import synth
    import weight_only_int4_topk_amd as B
    wl = synth.Workload("ep_share", E=E, H=H, I=I, topk=1, Ms=(1,), dtype="bf16", bits=4)
    layer = synth.make_layer(wl, seed=seed, device="cuda")
    wb = {n: sum(layer[n + t].numel() * layer[n + t].element_size() for t in ("", "_scales", "_zeros"))
          for n in ("w13", "w2")}
    L = max(2, min(64, math.ceil(512 * MIB / wb["w13"]) + 1))
    copies = [layer] + [{k: v.clone() for k, v in layer.items()} for _ in range(L - 1)]
    out = []
    for T in Ts:
        cnt = torch.full((E,), T, dtype=torch.int32, device="cuda")
        x = (torch.randn((E, T, H), device="cuda") * 0.1).to(torch.bfloat16)
        h = torch.empty((E, T, I), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((E, T, H), dtype=torch.bfloat16, device="cuda")
        f13 = [(lambda c=c: B.moe_wna16_batched_gemm(x, cnt, c["w13"], c["w13_scales"], c["w13_zeros"],
                                                     act=1, C=h)) for c in copies]
        f2 = [(lambda c=c: B.moe_wna16_batched_gemm(h, cnt, c["w2"], c["w2_scales"], c["w2_zeros"],
                                                    act=0, C=y)) for c in copies]
        t13 = graph_replay(f13, steps, warmup)[0] / steps * 1e6
        t2 = graph_replay(f2, steps, warmup)[0] / steps * 1e6
        out.append({"experts": E, "tokens_per_expert": T, "w13_us": round(t13, 2),
                    "w13_GBps": round(wb["w13"] / (t13 * 1e-6) / 1e9, 1), "w2_us": round(t2, 2),
                    "w2_GBps": round(wb["w2"] / (t2 * 1e-6) / 1e9, 1), "weight_copies": L})
        log(f"[bench] batched {out[-1]}")
    del copies, layer
    torch.cuda.empty_cache()
    return out


def w8a8_sweep(steps, warmup, Ms=(1024, 4096), seed=0):
    """w8a8 against w8a16 on the DeepSeek-V3 full-expert layer with int8 weights (256 experts,
    H 7168, I 2048, top-8 grouped sigmoid routing, bf16): the per-token activation quantiser, the
    first grouped GEMM with SiLU on int8 activations (integer matrix cores), and the same GEMM on
    bf16 activations, on the same weights and routing; time per call from graph replays over two
    weight copies, and tera-operations per second against the dense peaks (int8 5.0 POP/s, bf16
    2.5 PFLOP/s)."""
    import torch

    import synth
    import weight_only_int4_topk_amd as B
    wl = synth.WORKLOADS["dsv3_prefill_int8"]
    layer = synth.make_layer(wl, seed=seed, device="cuda")
    copies = [layer, {k: (v.clone() if v is not None else None) for k, v in layer.items()}]
    rt = B.routing(wl.score, wl.renormalize, wl.num_groups, wl.topk_groups, wl.scale)
    out = []
    for M in Ms:
        x = synth.make_x(wl, M, seed=seed, device="cuda")
        lg = synth.make_logits(wl, M, seed=seed, device="cuda")
        tw, ti = B.moe_topk_softmax(lg, wl.topk, rt)
        # the layers' choices (the same block size for both at this shape)
        bm16 = B.moe_pick_block_m(M, wl.E, wl.topk, 8, wl.torch_dtype)
        bm8 = bm16
        st, ex, npost = B.moe_align_block_size(ti, wl.E, bm8)
        st16, ex16, np16 = B.moe_align_block_size(ti, wl.E, bm16)
        q, sa = B.moe_quant_int8_rows(x)
        ns = M * wl.topk
        h = torch.empty((ns, wl.I), dtype=wl.torch_dtype, device="cuda")
        t_q = graph_replay([lambda: B.moe_quant_int8_rows(x, q, sa)], steps, warmup)[0] / steps
        f8 = [(lambda c=c: B.moe_w8a8_gemm(q, sa, wl.topk, c["w13"], c["w13_scales"], st, ex, npost,
                                           bm8, ns, wl.torch_dtype, act=1, C=h)) for c in copies]
        f16 = [(lambda c=c: B.moe_wna16_gemm(x, wl.topk, c["w13"], c["w13_scales"], None, st16, ex16,
                                             np16, bm16, ns, act=1, C=h)) for c in copies]
        t8 = graph_replay(f8, steps, warmup)[0] / steps
        t16 = graph_replay(f16, steps, warmup)[0] / steps
        # the whole layer both ways, same weights, routing computed inside
        o = torch.empty((M, wl.H), dtype=wl.torch_dtype, device="cuda")
        ws8 = torch.empty((B.lib().fused_moe_w8a8_workspace_size(M, wl.H, wl.I, wl.E, wl.topk, 1, 0),),
                          dtype=torch.uint8, device="cuda")
        ws16 = torch.empty((B.fused_moe_wna16_workspace_size(M, wl.H, wl.I, wl.E, wl.topk,
                                                             B.QUANT_INT8, wl.torch_dtype),),
                           dtype=torch.uint8, device="cuda")
        l8 = [(lambda c=c: B.fused_moe_w8a8(x, lg, wl.topk, rt, c["w13"], c["w13_scales"], c["w2"],
                                            c["w2_scales"], workspace=ws8, out=o)) for c in copies]
        l16 = [(lambda c=c: B.fused_moe_wna16(x, lg, wl.topk, rt, c["w13"], c["w13_scales"], None,
                                              c["w2"], c["w2_scales"], None, workspace=ws16, out=o))
               for c in copies]
        tl8 = graph_replay(l8, steps, warmup)[0] / steps
        tl16 = graph_replay(l16, steps, warmup)[0] / steps
        ops = 4.0 * wl.H * wl.I * ns
        out.append({"M": M, "block_m_w8a8": bm8, "block_m_w8a16": bm16,
                    "quant_us": round(t_q * 1e6, 2),
                    "w8a8_w13_us": round(t8 * 1e6, 2), "w8a8_TOPs": round(ops / t8 / 1e12, 1),
                    "w8a8_int8_mfma_frac": round(ops / t8 / 1e12 / 5000.0, 4),
                    "w8a16_w13_us": round(t16 * 1e6, 2), "w8a16_TFLOPs": round(ops / t16 / 1e12, 1),
                    "w8a16_bf16_mfma_frac": round(ops / t16 / 1e12 / MFMA_PEAK_TFLOPS, 4),
                    "w8a8_layer_us": round(tl8 * 1e6, 1), "w8a16_layer_us": round(tl16 * 1e6, 1)})
        log(f"[bench] w8a8 {out[-1]}")
    del copies, layer
    torch.cuda.empty_cache()
    return out


def act_order_sweep(bench, Ms, steps, warmup):
    """The same layer as GPTQ act-order experts (fused_moe_wna16_act_order: the activation rows
    gathered per slot through each expert's input-column permutation before each GEMM) beside the
    plain fused layer, on the bench's own weight copies with a seeded permutation per expert."""
    torch, synth, B, wl = bench.torch, bench.synth, bench.B, bench.wl
    g = torch.Generator(device="cuda").manual_seed(bench.seed)
    p13 = torch.stack([torch.randperm(wl.H, generator=g, device="cuda") for _ in range(wl.E)]).to(torch.int32)
    p2 = torch.stack([torch.randperm(wl.I, generator=g, device="cuda") for _ in range(wl.E)]).to(torch.int32)
    out = []
    for M in Ms:
        x = synth.make_x(wl, M, seed=bench.seed, device="cuda")
        lg = synth.make_logits(wl, M, seed=bench.seed, device="cuda")
        o = torch.empty((M, wl.H), dtype=wl.torch_dtype, device="cuda")
        ws = torch.empty((B.lib().fused_moe_wna16_act_order_workspace_size(
            M, wl.H, wl.I, wl.E, wl.topk, 0 if wl.dtype == "fp16" else 1, 0),), dtype=torch.uint8,
            device="cuda")
        L = len(bench.copies)
        fa = [(lambda c=c: B.fused_moe_wna16_act_order(
            x, lg, wl.topk, bench.rt, c["w13"], c["w13_scales"], c["w13_zeros"], p13, c["w2"],
            c["w2_scales"], c["w2_zeros"], p2, workspace=ws, out=o)) for c in bench.copies[:L]]
        t = graph_replay(fa, steps, warmup)[0] / steps
        out.append({"M": M, "act_order_us_per_layer": round(t * 1e6, 2)})
        log(f"[bench] act-order {out[-1]}")
    return out


KERNEL_SOURCES = ("gemm.hip", "common.h", "launch.h", "api.cpp")


def committed_traffic(workload, M):
    """HBM bytes per launch of the dominant kernel from the committed profile summary, if that
    summary was taken on the current kernel sources (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"w13_gemm_{workload}_m{M}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        k, _, v = line.partition(":")
        fields[k.strip()] = v.strip()
    csrc = os.path.join(ROOT, "weight_only_int4_topk_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in KERNEL_SOURCES)
    if fields.get("traffic_kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name (lscpu's "Model name", else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(bench, M, x, lg, ntok):
    """The oracle as it stands on the first ntok tokens of the batch (host cores): once with the
    BLAS threads it starts with, once with one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    torch, wl = bench.torch, bench.wl
    rows = np.arange(min(ntok, M) if ntok > 0 else M)
    lg_np = O.to_numpy(lg)[rows]
    ids, _ = O.route(lg_np, wl.topk, wl.score, wl.renormalize, wl.num_groups, wl.topk_groups,
                     wl.scale)
    experts = sorted(set(ids.reshape(-1).tolist()))
    idx = torch.tensor(experts, dtype=torch.long, device="cuda")
    sub = {k: (v.index_select(0, idx).cpu() if v is not None else None)
           for k, v in bench.layer.items()}
    xs = x[: len(rows)].cpu()
    cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])

    def run():
        t0 = time.perf_counter()
        ids, w = O.route(lg_np, wl.topk, wl.score, wl.renormalize, wl.num_groups,
                         wl.topk_groups, wl.scale)
        O.moe_layer_rows(xs, ids, w, O.ExpertSource(sub, wl.bits, experts))
        return time.perf_counter() - t0

    dt = run()
    with threadpool_limits(1):
        dt1 = run()
    return {"value": round(len(rows) / dt, 4), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{len(rows)} of the {M} tokens of the timed batch ({len(experts)} experts): "
                      f"routing, float64 decoding of those experts and their FFN, {dt:.1f} s",
            "one_thread_value": round(len(rows) / dt1, 4), "one_thread_s": round(dt1, 2),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the layer is measured on one GPU's share of the experts; runs across several GPUs are not implemented",
              file=sys.stderr)
        sys.exit(2)
    import synth
    wl = synth.WORKLOADS[args.workload]
    decode = [m for m in wl.Ms if m <= 64]
    M = args.m or (max(decode) if decode else max(wl.Ms))
    bench = Bench(wl, args.seed)
    sweep_warm = max(10, args.warmup // 4)

    # The headline's graphs are captured now and timed last, right after the other GPU work: after
    # the GPU has idled (host-side set-up, the CPU baseline) its first milliseconds of work run at a
    # lower clock (measured: the first two replays of a 20-call graph 215-233 us per call, later
    # ones 201-209 us), which a 5-step warmup does not cover.
    finish_headline = bench.measure(M, args.steps, args.warmup, defer=True)
    x = synth.make_x(wl, M, seed=args.seed, device="cuda")
    lg = synth.make_logits(wl, M, seed=args.seed, device="cuda")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bench, M, x, lg, args.cpu_tokens)
        log(f"[bench] cpu baseline: {cpu}")

    if args.calibrate_copy:
        import torch
        src = torch.empty(512 * MIB, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 5 x 512 MiB device-to-device")

    # every M of every workload shape, each with its binding roofline (the headline workload's
    # layer copies are reused)
    table = []
    if not args.no_sweep:
        for name in [n for n in args.workloads.split(",") if n]:
            b = bench if name == wl.name else Bench(synth.WORKLOADS[name], args.seed)
            for m in b.wl.Ms:
                r = {"workload": name, **b.measure(m, args.sweep_steps, sweep_warm)[0]}
                if name == "tiny":
                    r["note"] = "parity workload: its 1.6 MB of experts stay cache-resident"
                table.append(r)
                log(f"[bench] {name} M={m}: {r}")
            if b is not bench:
                b.release()
                del b

    act_order = None
    if not args.no_act_order and wl.bits == 4:
        act_order = act_order_sweep(bench, [m for m in wl.Ms if m <= 64] or [M], args.sweep_steps,
                                    sweep_warm)
        for r in act_order:
            plain = next((t["us_per_layer"] for t in table
                          if t["workload"] == wl.name and t["M"] == r["M"]), None)
            r["plain_us_per_layer"] = plain
    dense = None if args.no_dense else dense_sweep(args.sweep_steps, sweep_warm)
    batched = None if args.no_batched else batched_sweep(args.sweep_steps, sweep_warm)
    w8a8 = None if args.no_w8a8 else w8a8_sweep(max(20, args.sweep_steps // 4),
                                                 max(5, args.warmup // 8))

    res, t_layer, wall, _ = finish_headline()
    log(f"[bench] headline M={M}: {res}")
    bench.release()

    hbm_frac = res["w13_GBps"] / HBM_PEAK_GBPS
    mfma_frac = res["w13_TFLOPs"] / MFMA_PEAK_TFLOPS
    if mfma_frac > hbm_frac:
        roof = {"bound": "mfma", "achieved": res["w13_TFLOPs"], "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(mfma_frac, 4), "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": res["w13_GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(hbm_frac, 4), "traffic": None}
    traffic = committed_traffic(wl.name, M)
    if traffic is not None:
        roof["traffic"] = round(traffic / (res["w13_us"] * 1e-6) / 1e9, 1)
        roof["traffic_bytes_per_launch"] = traffic
    kname = "prefill_gemm_kernel" if res["block_m"] >= 128 else "wna16_gemm_kernel"
    roof.update({"kernel": f"{kname} (w13 + SiLU*up, block_m {res['block_m']})",
                 "avg_launch_us": res["w13_us"],
                 "algorithmic_per_launch": (res["w13_bytes"] if roof["bound"] == "hbm"
                                            else 4.0 * wl.H * wl.I * M * wl.topk)})

    value = M * args.steps / t_layer
    line = {
        "metric": "fused-MoE w4a16 layer tokens/s + achieved HBM GB/s vs peak, M=1..4096",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_layer / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,0.02^2) experts encoded "
                + ("uint4 g128 asymmetric" if wl.bits == 4 else "int8 per-channel symmetric")
                + ", N(0,0.1^2) activations, N(0,1) router logits",
        "config": {"workload": f"{wl.name}: {wl.notes}", "E": wl.E, "H": wl.H, "I": wl.I,
                   "topk": wl.topk, "M": M, "bits": wl.bits, "block_m": res["block_m"],
                   "layer_copies": res["layer_copies"], "active_experts": res["active_experts"],
                   "layer_GBps": res["layer_GBps"], "layer_hbm_frac": res["layer_hbm_frac"],
                   "timed_graph_calls": res["graph_calls"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": table,
        "act_order": act_order,
        "dense_w4a16": dense,
        "batched_experts": batched,
        "w8a8": w8a8,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
