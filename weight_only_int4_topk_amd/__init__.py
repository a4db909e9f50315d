"""Python binding of the moe_wna16 C ABI (include/moe_wna16.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of libmoe_wna16.so.
torch provides device memory and the current stream; this module passes pointers, sizes and the
stream handle, allocates outputs the caller did not provide, and turns a non-zero status into a
MoeError.  There is no fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MoeError", "MoeQuant", "MoeRouting", "lib", "LIB_PATH", "QUANT_INT4", "QUANT_INT8", "routing",
    "moe_topk_softmax", "moe_align_capacity", "moe_align_block_size", "moe_pick_block_m",
    "moe_wna16_gemm", "moe_wna16_dense_gemm", "moe_wna16_dense_gemm_workspace_size",
    "moe_wna16_batched_gemm", "moe_quant_int8_rows", "moe_w8a8_gemm", "fused_moe_w8a8",
    "fused_moe_wna16_act_order", "fused_moe_wna16_workspace_size", "fused_moe_wna16",
    "fused_moe_wna16_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_repack_uint4", "FORMAT_GPTQ",
    "FORMAT_AWQ", "fused_moe_wna16_path", "PATH_GROUPED", "PATH_ONE_TOKEN", "PATH_FEW_TOKENS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_wna16.so")


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe_wna16 status {status}: {message}")
        self.status = status


class MoeQuant(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("has_zero", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("scale", ctypes.c_float)]


QUANT_INT4 = MoeQuant(4, 128, 1)
QUANT_INT8 = MoeQuant(8, 0, 0)

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SIGS = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_topk_softmax": ([_P, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _P, _P], _I),
    "moe_align_capacity": ([_I, _I, _I], _I64),
    "moe_pick_block_m": ([_I, _I, _I, _I, _I], _I),
    "fused_moe_wna16_path": ([_I, _I, _I, _I, _I, ctypes.POINTER(MoeQuant), _I, _I], _I),
    "moe_align_block_size": ([_P, _I, _I, _I, _P, _P, _P, _I64, _P], _I),
    "moe_wna16_gemm": ([_P, _I, _I, _P, _P, _P, ctypes.POINTER(MoeQuant), _I, _I, _I, _I,
                        _P, _P, _P, _I64, _I, _I, _P, _I, _P, _P], _I),
    "moe_wna16_dense_gemm": ([_P, _I, _I, _P, _P, _P, ctypes.POINTER(MoeQuant), _I, _I, _P,
                              ctypes.c_size_t, _P, _P], _I),
    "moe_wna16_dense_gemm_workspace_size": ([_I, _I, _I, ctypes.POINTER(MoeQuant), _I],
                                            ctypes.c_size_t),
    "moe_quant_int8_rows": ([_P, _I, _I, _I, _P, _P, _P], _I),
    "moe_w8a8_gemm": ([_P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I64, _I, _I, _P, _I,
                       _P, _P], _I),
    "fused_moe_w8a8": ([_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _P, _P, _P, _I,
                        _I, _P, ctypes.c_size_t, _P, _P, _P, _P], _I),
    "fused_moe_w8a8_workspace_size": ([_I, _I, _I, _I, _I, _I, _I], ctypes.c_size_t),
    "fused_moe_wna16_act_order": ([_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _P,
                                   _P, _P, _P, _P, _P, _P, _I, _I, _P, ctypes.c_size_t, _P, _P,
                                   _P, _P], _I),
    "fused_moe_wna16_act_order_workspace_size": ([_I, _I, _I, _I, _I, _I, _I], ctypes.c_size_t),
    "moe_wna16_batched_gemm": ([_P, _I, _I, _I, _P, _P, _P, _P, ctypes.POINTER(MoeQuant), _I, _I,
                                _I, _I, _P, _P], _I),
    "fused_moe_wna16_workspace_size": ([_I, _I, _I, _I, _I, ctypes.POINTER(MoeQuant), _I, _I],
                                       ctypes.c_size_t),
    "fused_moe_wna16": ([_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _P, _P, _P,
                         _P, _P, ctypes.POINTER(MoeQuant), _I, _I, _P, ctypes.c_size_t, _P, _P,
                         _P, _P], _I),
    "fused_moe_wna16_noalloc": ([_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _P,
                                 _P, _P, _P, _P, ctypes.POINTER(MoeQuant), _I, _I, _P, _P, _P, _P],
                                _I),
}

_SIGS["moe_repack_uint4"] = ([_I, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P], _I)
FORMAT_GPTQ, FORMAT_AWQ = 0, 1

# MOE_NOALLOC_SCRATCH_BYTES of the header: the static scratch of fused_moe_wna16_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m weight_only_int4_topk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError(-1, "tensor is not on a GPU device")
    if not t.is_contiguous():
        raise MoeError(-1, "tensor is not contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt) -> int:
    if dt == torch.float16:
        return 0
    if dt == torch.bfloat16:
        return 1
    raise MoeError(-2, f"unsupported activation dtype {dt}")


def _quant_of(B: torch.Tensor, zeros) -> MoeQuant:
    if B.dtype == torch.uint8 and zeros is not None:
        return QUANT_INT4
    if B.dtype == torch.int8 and zeros is None:
        return QUANT_INT8
    raise MoeError(-2, f"weights of dtype {B.dtype} with zeros={'set' if zeros is not None else 'None'}")


# The library takes plain pointers and trusts the sizes passed beside them, so every tensor is
# checked here against the shape those sizes imply before its pointer is handed over.
def _want(t, shape, dtype, name):
    """Raise unless t (when given) has exactly this shape and dtype."""
    if t is None:
        return
    shape = tuple(int(s) for s in shape)
    if tuple(t.shape) != shape:
        raise MoeError(-1, f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(-1, f"{name} has dtype {t.dtype}, expected {dtype}")


def _want_len(t, n, dtype, name):
    """Raise unless t (when given) holds at least n elements of this dtype."""
    if t is None:
        return
    if t.numel() < n:
        raise MoeError(-1, f"{name} holds {t.numel()} elements, needs {n}")
    if t.dtype != dtype:
        raise MoeError(-1, f"{name} has dtype {t.dtype}, expected {dtype}")


def _want_weights(name, B, scales, zeros, lead, N, K, act_dtype):
    """Weight storage of the header's layouts; lead = (E,) for experts, () for one matrix."""
    lead = tuple(lead)
    if B.dtype == torch.uint8:
        _want(B, lead + (N, K // 2), torch.uint8, name)
        _want(scales, lead + (N, K // 128), act_dtype, name + " scales")
        _want(zeros, lead + (N, K // 256), torch.uint8, name + " zeros")
    else:
        _want(B, lead + (N, K), torch.int8, name)
        _want(scales, lead + (N,), act_dtype, name + " scales")


def routing(score="softmax", renormalize=True, num_groups=1, topk_groups=1, scale=1.0) -> MoeRouting:
    return MoeRouting(0 if score == "softmax" else 1, int(bool(renormalize)), num_groups,
                      topk_groups, float(scale))


def moe_topk_softmax(logits, topk, rt: MoeRouting, topk_weights=None, topk_ids=None, stream=None):
    M, E = logits.shape
    _want(logits, (M, E), torch.float32, "logits")
    _want(topk_weights, (M, topk), torch.float32, "topk_weights")
    _want(topk_ids, (M, topk), torch.int32, "topk_ids")
    if topk_weights is None:
        topk_weights = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    if topk_ids is None:
        topk_ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
    _check(lib().moe_topk_softmax(_ptr(logits), M, E, topk, ctypes.byref(rt), _ptr(topk_weights),
                                  _ptr(topk_ids), _stream(stream)))
    return topk_weights, topk_ids


PATH_GROUPED, PATH_ONE_TOKEN, PATH_FEW_TOKENS = 0, 1, 2


def fused_moe_wna16_path(M, H, I, E, topk, bits=4, block_m=0, act_order=False) -> int:
    """The launch sequence fused_moe_wna16 takes for these sizes (PATH_*; -1: sizes it rejects)."""
    q = QUANT_INT4 if bits == 4 else QUANT_INT8
    return int(lib().fused_moe_wna16_path(M, H, I, E, topk, ctypes.byref(q), block_m,
                                          1 if act_order else 0))


def moe_pick_block_m(M, E, topk, bits=4, dtype=torch.float16) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().moe_pick_block_m(M, E, topk, bits, code))


def moe_align_capacity(numel, E, block_m) -> int:
    return int(lib().moe_align_capacity(numel, E, block_m))


def moe_align_block_size(topk_ids, E, block_m, capacity=None, stream=None):
    numel = topk_ids.numel()
    _want_len(topk_ids, numel, torch.int32, "topk_ids")
    cap = moe_align_capacity(numel, E, block_m) if capacity is None else capacity
    dev = topk_ids.device
    sorted_ids = torch.empty((cap,), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(((cap + block_m - 1) // block_m,), dtype=torch.int32, device=dev)
    num_post = torch.empty((1,), dtype=torch.int32, device=dev)
    _check(lib().moe_align_block_size(_ptr(topk_ids), numel, E, block_m, _ptr(sorted_ids),
                                      _ptr(expert_ids), _ptr(num_post), cap, _stream(stream)))
    return sorted_ids, expert_ids, num_post


def moe_wna16_gemm(A, a_row_div, B, scales, zeros, sorted_ids, expert_ids, num_post, block_m,
                   num_slots, topk_weights=None, act=0, C=None, stream=None):
    quant = _quant_of(B, zeros)
    E, N = B.shape[0], B.shape[1]
    K = B.shape[2] * (2 if quant.bits == 4 else 1)
    n_out = N // 2 if act == 1 else N
    _want(A, (A.shape[0], K), A.dtype, "A")
    _dtype_code(A.dtype)
    _want_weights("B", B, scales, zeros, (E,), N, K, A.dtype)
    _want_len(sorted_ids, sorted_ids.numel(), torch.int32, "sorted_ids")
    _want_len(expert_ids, -(-sorted_ids.numel() // block_m) if block_m > 0 else 0, torch.int32,
              "expert_ids")
    _want_len(num_post, 1, torch.int32, "num_post")
    _want_len(topk_weights, num_slots, torch.float32, "topk_weights")
    _want(C, (num_slots, n_out), A.dtype, "C")
    if C is None:
        C = torch.empty((num_slots, n_out), dtype=A.dtype, device=A.device)
    _check(lib().moe_wna16_gemm(_ptr(A), A.shape[0], a_row_div, _ptr(B), _ptr(scales), _ptr(zeros),
                                ctypes.byref(quant), E, N, K, _dtype_code(A.dtype),
                                _ptr(sorted_ids), _ptr(expert_ids), _ptr(num_post),
                                sorted_ids.numel(), block_m, num_slots, _ptr(topk_weights), act,
                                _ptr(C), _stream(stream)))
    return C


def moe_wna16_dense_gemm_workspace_size(M, N, K, quant: MoeQuant, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().moe_wna16_dense_gemm_workspace_size(M, N, K, ctypes.byref(quant), code))


def moe_wna16_dense_gemm(A, B, scales, zeros=None, workspace=None, C=None, stream=None):
    """C [M, N] = A [M, K] . W^T for one weight matrix B ([N, K/2] uint8 or [N, K] int8)."""
    quant = _quant_of(B, zeros)
    M, K = A.shape
    N = B.shape[0]
    _want_weights("B", B, scales, zeros, (), N, K, A.dtype)
    _want(C, (M, N), A.dtype, "C")
    need = moe_wna16_dense_gemm_workspace_size(M, N, K, quant, A.dtype)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=A.device)
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _check(lib().moe_wna16_dense_gemm(_ptr(A), M, K, _ptr(B), _ptr(scales), _ptr(zeros),
                                      ctypes.byref(quant), N, _dtype_code(A.dtype),
                                      _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                      _ptr(C), _stream(stream)))
    return C


def moe_wna16_batched_gemm(A, expert_num_tokens, B, scales, zeros=None, act=0, block_m=0, C=None,
                           stream=None):
    """C [E, T, N or N/2] from A [E, T, K] batched per expert (rows below expert_num_tokens[e])."""
    quant = _quant_of(B, zeros)
    E, T, K = A.shape
    N = B.shape[1]
    _want_weights("B", B, scales, zeros, (E,), N, K, A.dtype)
    _want(expert_num_tokens, (E,), torch.int32, "expert_num_tokens")
    _want(C, (E, T, N // 2 if act == 1 else N), A.dtype, "C")
    if C is None:
        C = torch.empty((E, T, N // 2 if act == 1 else N), dtype=A.dtype, device=A.device)
    _check(lib().moe_wna16_batched_gemm(_ptr(A), E, T, K, _ptr(expert_num_tokens), _ptr(B),
                                        _ptr(scales), _ptr(zeros), ctypes.byref(quant), N,
                                        _dtype_code(A.dtype), block_m, act, _ptr(C),
                                        _stream(stream)))
    return C


def moe_quant_int8_rows(x, q=None, scales=None, stream=None):
    """(q int8 [R, K], scales float [R]) = per-row symmetric int8 of x [R, K] (fp16/bf16)."""
    R, K = x.shape
    _want(q, (R, K), torch.int8, "q")
    _want(scales, (R,), torch.float32, "scales")
    if q is None:
        q = torch.empty((R, K), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((R,), dtype=torch.float32, device=x.device)
    _check(lib().moe_quant_int8_rows(_ptr(x), R, K, _dtype_code(x.dtype), _ptr(q), _ptr(scales),
                                     _stream(stream)))
    return q, scales


def moe_w8a8_gemm(Aq, a_scales, a_row_div, B, w_scales, sorted_ids, expert_ids, num_post, block_m,
                  num_slots, dtype, topk_weights=None, act=0, C=None, stream=None):
    """Grouped GEMM of int8 activations (per-row scales) with int8 weights (per-channel scales)."""
    E, N, K = B.shape
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    odt = torch.float16 if code == 0 else torch.bfloat16
    _want(Aq, (Aq.shape[0], K), torch.int8, "Aq")
    _want(a_scales, (Aq.shape[0],), torch.float32, "a_scales")
    _want_weights("B", B, w_scales, None, (E,), N, K, odt)
    _want_len(expert_ids, -(-sorted_ids.numel() // block_m) if block_m > 0 else 0, torch.int32,
              "expert_ids")
    _want_len(sorted_ids, sorted_ids.numel(), torch.int32, "sorted_ids")
    _want_len(num_post, 1, torch.int32, "num_post")
    _want_len(topk_weights, num_slots, torch.float32, "topk_weights")
    _want(C, (num_slots, N // 2 if act == 1 else N), odt, "C")
    if C is None:
        C = torch.empty((num_slots, N // 2 if act == 1 else N),
                        dtype=torch.float16 if code == 0 else torch.bfloat16, device=Aq.device)
    _check(lib().moe_w8a8_gemm(_ptr(Aq), _ptr(a_scales), Aq.shape[0], a_row_div, _ptr(B),
                               _ptr(w_scales), E, N, K, code, _ptr(sorted_ids), _ptr(expert_ids),
                               _ptr(num_post), sorted_ids.numel(), block_m, num_slots,
                               _ptr(topk_weights), act, _ptr(C), _stream(stream)))
    return C


def _want_layer_io(x, router_logits, E, topk, out, topk_weights, topk_ids):
    M, H = x.shape
    _dtype_code(x.dtype)
    _want(router_logits, (M, E), torch.float32, "router_logits")
    _want(out, (M, H), x.dtype, "out")
    _want(topk_weights, (M, topk), torch.float32, "topk_weights")
    _want(topk_ids, (M, topk), torch.int32, "topk_ids")


def fused_moe_w8a8(x, router_logits, topk, rt: MoeRouting, w13, w13_scales, w2, w2_scales,
                   block_m=0, workspace=None, out=None, topk_weights=None, topk_ids=None,
                   stream=None):
    """The whole layer with int8 experts and per-token int8 activations; returns out [M, H]."""
    M, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    code = _dtype_code(x.dtype)
    _want_layer_io(x, router_logits, E, topk, out, topk_weights, topk_ids)
    _want_weights("w13", w13, w13_scales, None, (E,), 2 * I, H, x.dtype)
    _want_weights("w2", w2, w2_scales, None, (E,), H, I, x.dtype)
    need = int(lib().fused_moe_w8a8_workspace_size(M, H, I, E, topk, code, block_m))
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=x.dtype, device=x.device)
    _check(lib().fused_moe_w8a8(_ptr(x), _ptr(router_logits), M, H, I, E, topk, ctypes.byref(rt),
                                _ptr(w13), _ptr(w13_scales), _ptr(w2), _ptr(w2_scales), code,
                                block_m, _ptr(workspace), workspace.numel(), _ptr(out),
                                _ptr(topk_weights), _ptr(topk_ids), _stream(stream)))
    return out


def fused_moe_wna16_act_order(x, router_logits, topk, rt: MoeRouting, w13, w13_scales, w13_zeros,
                              w13_perm, w2, w2_scales, w2_zeros, w2_perm, block_m=0,
                              workspace=None, out=None, topk_weights=None, topk_ids=None,
                              stream=None):
    """The layer with act-order uint4 experts in sorted storage plus per-expert permutations."""
    M, H = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    code = _dtype_code(x.dtype)
    _want_layer_io(x, router_logits, E, topk, out, topk_weights, topk_ids)
    _want_weights("w13", w13, w13_scales, w13_zeros, (E,), 2 * I, H, x.dtype)
    _want_weights("w2", w2, w2_scales, w2_zeros, (E,), H, I, x.dtype)
    _want(w13_perm, (E, H), torch.int32, "w13_perm")
    _want(w2_perm, (E, I), torch.int32, "w2_perm")
    need = int(lib().fused_moe_wna16_act_order_workspace_size(M, H, I, E, topk, code, block_m))
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=x.dtype, device=x.device)
    _check(lib().fused_moe_wna16_act_order(
        _ptr(x), _ptr(router_logits), M, H, I, E, topk, ctypes.byref(rt), _ptr(w13),
        _ptr(w13_scales), _ptr(w13_zeros), _ptr(w13_perm), _ptr(w2), _ptr(w2_scales),
        _ptr(w2_zeros), _ptr(w2_perm), code, block_m, _ptr(workspace), workspace.numel(),
        _ptr(out), _ptr(topk_weights), _ptr(topk_ids), _stream(stream)))
    return out


def fused_moe_wna16_workspace_size(M, H, I, E, topk, quant: MoeQuant, dtype, block_m=0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().fused_moe_wna16_workspace_size(M, H, I, E, topk, ctypes.byref(quant), code,
                                                    block_m))


def fused_moe_wna16(x, router_logits, topk, rt: MoeRouting, w13, w13_scales, w13_zeros, w2,
                    w2_scales, w2_zeros, block_m=0, workspace=None, out=None, topk_weights=None,
                    topk_ids=None, stream=None):
    """The whole layer; returns out [M, H] (and writes topk_weights / topk_ids if given)."""
    quant = _quant_of(w13, w13_zeros)
    M, H = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    _want_layer_io(x, router_logits, E, topk, out, topk_weights, topk_ids)
    _want_weights("w13", w13, w13_scales, w13_zeros, (E,), 2 * I, H, x.dtype)
    _want_weights("w2", w2, w2_scales, w2_zeros, (E,), H, I, x.dtype)
    need = fused_moe_wna16_workspace_size(M, H, I, E, topk, quant, x.dtype, block_m)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=x.dtype, device=x.device)
    _check(lib().fused_moe_wna16(_ptr(x), _ptr(router_logits), M, H, I, E, topk, ctypes.byref(rt),
                                 _ptr(w13), _ptr(w13_scales), _ptr(w13_zeros), _ptr(w2),
                                 _ptr(w2_scales), _ptr(w2_zeros), ctypes.byref(quant),
                                 _dtype_code(x.dtype), block_m, _ptr(workspace),
                                 workspace.numel(), _ptr(out), _ptr(topk_weights),
                                 _ptr(topk_ids), _stream(stream)))
    return out


def fused_moe_wna16_noalloc(x, router_logits, topk, rt: MoeRouting, w13, w13_scales, w13_zeros, w2,
                            w2_scales, w2_zeros, out, block_m=0, topk_weights=None, topk_ids=None,
                            stream=None):
    """The whole layer on the library's static scratch: no workspace and nothing allocated here
    either (out, and topk_weights / topk_ids if wanted, are the caller's)."""
    quant = _quant_of(w13, w13_zeros)
    M, H = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    _want_layer_io(x, router_logits, E, topk, out, topk_weights, topk_ids)
    _want_weights("w13", w13, w13_scales, w13_zeros, (E,), 2 * I, H, x.dtype)
    _want_weights("w2", w2, w2_scales, w2_zeros, (E,), H, I, x.dtype)
    _check(lib().fused_moe_wna16_noalloc(_ptr(x), _ptr(router_logits), M, H, I, E, topk,
                                         ctypes.byref(rt), _ptr(w13), _ptr(w13_scales),
                                         _ptr(w13_zeros), _ptr(w2), _ptr(w2_scales),
                                         _ptr(w2_zeros), ctypes.byref(quant),
                                         _dtype_code(x.dtype), block_m, _ptr(out),
                                         _ptr(topk_weights), _ptr(topk_ids), _stream(stream)))
    return out


def moe_repack_uint4(fmt, qweight, qzeros, scales, g_idx=None, invalid=None, stream=None):
    """GPTQ (fmt 0) / AWQ (fmt 1) checkpoint tensors of E experts -> (B, scales, zeros[, perm]) in
    the canonical storage (with g_idx: the act-order sorted storage and its permutation)."""
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise MoeError(-1, "qweight and qzeros must be int32")
    E = qweight.shape[0]
    if fmt == FORMAT_GPTQ:
        K, N = qweight.shape[1] * 8, qweight.shape[2]
    else:
        K, N = qweight.shape[1], qweight.shape[2] * 8
    G = K // 128
    _want(qweight, (E, K // 8, N) if fmt == FORMAT_GPTQ else (E, K, N // 8), torch.int32, "qweight")
    _want(qzeros, (E, G, N // 8), torch.int32, "qzeros")
    _want(scales, (E, G, N), scales.dtype, "scales")
    _want(g_idx, (E, K), torch.int32, "g_idx")
    _want(invalid, (1,), torch.int32, "invalid")
    dev = qweight.device
    B = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    so = torch.empty((E, N, G), dtype=scales.dtype, device=dev)
    zo = torch.empty((E, N, G // 2), dtype=torch.uint8, device=dev)
    perm = torch.empty((E, K), dtype=torch.int32, device=dev) if g_idx is not None else None
    _check(lib().moe_repack_uint4(fmt, _ptr(qweight), _ptr(qzeros), _ptr(scales), _ptr(g_idx), E, N,
                                  K, _dtype_code(scales.dtype), _ptr(B), _ptr(so), _ptr(zo),
                                  _ptr(perm), _ptr(invalid), _stream(stream)))
    return (B, so, zo) if perm is None else (B, so, zo, perm)
