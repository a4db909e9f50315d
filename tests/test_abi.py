"""The C ABI without a GPU: the library loads, exports every function include/*.h declares, and
its host-side argument checks return the documented status codes (no call here reaches a launch)."""
import ctypes
import glob
import os
import re

import pytest

import weight_only_int4_topk_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: every call below fails validation
NULL = None


def _declared_functions():
    names = []
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_wna16.so is not built (python -m weight_only_int4_topk_amd.build)")
    return B.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_topk_softmax", "moe_align_block_size", "moe_align_capacity", "moe_wna16_gemm",
              "fused_moe_wna16", "fused_moe_wna16_workspace_size", "moe_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n
        assert n in B._SIGS, f"binding has no signature for {n}"


def _rt(score=0, renorm=1, ng=1, tg=1, scale=1.0):
    return ctypes.byref(B.MoeRouting(score, renorm, ng, tg, scale))


def test_routing_validation(lib):
    f = lib.moe_topk_softmax
    assert f(FAKE, 4, 8, 2, None, FAKE, FAKE, NULL) == INVALID            # routing NULL
    assert f(NULL, 4, 8, 2, _rt(), FAKE, FAKE, NULL) == INVALID           # logits NULL
    assert f(FAKE, -1, 8, 2, _rt(), FAKE, FAKE, NULL) == INVALID
    assert f(FAKE, 4, 2000, 2, _rt(), FAKE, FAKE, NULL) == UNSUPPORTED    # E > 1024
    assert f(FAKE, 4, 8, 9, _rt(), FAKE, FAKE, NULL) == INVALID           # topk > E
    assert f(FAKE, 4, 8, 2, _rt(0, 1, 2, 1), FAKE, FAKE, NULL) == UNSUPPORTED  # grouped softmax
    assert f(FAKE, 4, 256, 8, _rt(1, 1, 7, 4), FAKE, FAKE, NULL) == INVALID    # groups !| E
    assert f(FAKE, 4, 256, 8, _rt(1, 1, 8, 9), FAKE, FAKE, NULL) == INVALID    # topk_groups > groups
    assert f(FAKE, 4, 16, 8, _rt(1, 1, 8, 2), FAKE, FAKE, NULL) == INVALID     # 8 > 2 groups * 2
    assert f(FAKE, 4, 8, 9, _rt(), FAKE, FAKE, NULL) == INVALID
    assert b"topk" in lib.moe_last_error()
    assert f(FAKE, 4, 8, 2, _rt(5), FAKE, FAKE, NULL) == INVALID               # unknown score
    assert b"score" in lib.moe_last_error()
    assert f(NULL, 0, 8, 2, _rt(), NULL, NULL, NULL) == OK                      # M == 0: no-op


def test_pick_block_m(lib):
    fp16, bf16 = 0, 1
    assert lib.moe_pick_block_m(16, 8, 2, 4, fp16) == 16       # 4 slots per expert
    assert lib.moe_pick_block_m(64, 8, 2, 4, fp16) == 32       # 16 per expert -> 24 needed
    assert lib.moe_pick_block_m(1024, 256, 8, 4, bf16) == 64   # 32 per expert -> 48 needed
    assert lib.moe_pick_block_m(4096, 256, 8, 4, bf16) == 256  # 128 per expert -> 192 needed
    assert lib.moe_pick_block_m(4096, 256, 8, 4, fp16) == 64   # fp16 uint4 stops at 64
    assert lib.moe_pick_block_m(4096, 256, 8, 8, bf16) == 256
    assert lib.moe_pick_block_m(2048, 256, 8, 8, bf16) == 128  # 64 per expert -> 96 needed
    assert lib.moe_pick_block_m(2048, 256, 8, 4, bf16) == 64
    assert lib.moe_pick_block_m(1024, 256, 8, 8, bf16) == 64
    # fp16 uint4: 32 rows where up to 128 would be needed (Qwen2 shape at M = 512: 64 per expert)
    assert lib.moe_pick_block_m(512, 64, 8, 4, fp16) == 32
    assert lib.moe_pick_block_m(512, 64, 8, 4, bf16) == 64
    assert lib.moe_pick_block_m(512, 64, 8, 8, fp16) == 128
    assert lib.moe_pick_block_m(8192, 64, 8, 4, fp16) == 64    # 1024 per expert: beyond the rule
    assert lib.moe_pick_block_m(0, 8, 2, 4, fp16) == -1
    assert lib.moe_pick_block_m(16, 8, 2, 3, fp16) == -1
    assert lib.moe_pick_block_m(16, 8, 2, 4, 2) == -1


def test_layer_path():
    """The launch sequence of the fused layer, decided from the sizes alone."""
    path = B.fused_moe_wna16_path
    one, few, grouped = B.PATH_ONE_TOKEN, B.PATH_FEW_TOKENS, B.PATH_GROUPED
    assert path(1, 4096, 14336, 8, 2) == one              # Mixtral shape
    assert path(1, 3584, 2560, 64, 8) == one              # Qwen2 shape
    assert path(1, 7168, 256, 256, 8) == one              # DeepSeek-V3 TP share
    assert path(1, 7168, 2048, 256, 8) == one             # DeepSeek-V3 all experts
    assert path(2, 7168, 256, 256, 8) == few
    assert path(4, 7168, 256, 256, 8) == few
    assert path(5, 7168, 256, 256, 8) == few
    assert path(6, 7168, 256, 256, 8) == grouped          # more tokens
    assert path(16, 7168, 256, 256, 8) == grouped
    assert path(2, 4096, 14336, 8, 2) == grouped          # wider I
    assert path(2, 3584, 2560, 64, 8) == grouped
    assert path(4, 16384, 256, 64, 8) == grouped          # H past 8192
    assert path(1, 4096, 14336, 8, 2, block_m=16) == grouped
    assert path(1, 4096, 14336, 8, 2, bits=8) == grouped
    assert path(1, 4096, 14336, 8, 2, act_order=True) == grouped
    assert path(1, 4096, 1024, 512, 8) == grouped         # E past 256
    assert path(1, 256, 32768, 4, 4) == grouped           # staged rows past LDS
    assert path(1, 256, 32768, 2, 2) == one
    assert path(0, 4096, 14336, 8, 2) == -1
    assert path(1, 100, 14336, 8, 2) == -1
    assert path(1, 4096, 14336, 8, 9) == -1               # topk > E
    assert path(1, 4096, 14336, 8, 2, block_m=48) == -1


def test_align_capacity_formula(lib):
    assert lib.moe_align_capacity(8, 4, 4) == 20      # hand-worked fixture
    assert lib.moe_align_capacity(8, 5, 2) == 13
    assert lib.moe_align_capacity(1, 256, 16) == 16
    assert lib.moe_align_capacity(32768, 256, 128) == 32768 + 256 * 127
    assert lib.moe_align_capacity(-1, 4, 4) == -1


def test_align_validation(lib):
    f = lib.moe_align_block_size
    assert f(FAKE, 8, 4, 48, FAKE, FAKE, FAKE, 100, NULL) == UNSUPPORTED   # block_m 48
    assert f(FAKE, 8, 4, 512, FAKE, FAKE, FAKE, 10000, NULL) == UNSUPPORTED  # block_m 512
    assert f(FAKE, 8, 4, 256, FAKE, FAKE, FAKE, 8 + 4 * 255 - 1, NULL) == CAPACITY  # 256 accepted
    assert f(FAKE, 8, 0, 16, FAKE, FAKE, FAKE, 100, NULL) == INVALID
    assert f(FAKE, 8, 2048, 16, FAKE, FAKE, FAKE, 100, NULL) == UNSUPPORTED
    assert f(FAKE, 8, 4, 4 * 4, NULL, FAKE, FAKE, 100, NULL) == INVALID    # sorted NULL
    assert f(FAKE, 8, 4, 16, FAKE, FAKE, FAKE, 8 + 4 * 15 - 1, NULL) == CAPACITY
    assert b"capacity" in lib.moe_last_error()
    assert f(ctypes.c_void_p(0x100002), 8, 4, 16, FAKE, FAKE, FAKE, 100, NULL) == INVALID  # align


def _q(bits, g, z):
    return ctypes.byref(B.MoeQuant(bits, g, z))


def _gemm(lib, **kw):
    a = dict(A=FAKE, rows=32, div=2, Bw=FAKE, S=FAKE, Z=FAKE, q=_q(4, 128, 1), E=8, N=1024, K=256,
             dt=0, st=FAKE, ex=FAKE, npost=FAKE, cap=152, bm=16, slots=32, tw=NULL, act=1, C=FAKE)
    a.update(kw)
    return lib.moe_wna16_gemm(a["A"], a["rows"], a["div"], a["Bw"], a["S"], a["Z"], a["q"], a["E"],
                              a["N"], a["K"], a["dt"], a["st"], a["ex"], a["npost"], a["cap"],
                              a["bm"], a["slots"], a["tw"], a["act"], a["C"], NULL)


def test_gemm_validation(lib):
    assert _gemm(lib, q=_q(3, 128, 1)) == UNSUPPORTED          # bits
    assert _gemm(lib, q=_q(4, 64, 1)) == UNSUPPORTED           # K tile must be the 128 group
    assert _gemm(lib, q=_q(4, 128, 0)) == UNSUPPORTED          # uint4 needs zero points
    assert _gemm(lib, q=_q(8, 0, 1)) == UNSUPPORTED            # int8 is symmetric
    assert _gemm(lib, q=_q(8, 0, 0)) == INVALID                # zeros given with has_zero = 0
    assert _gemm(lib, Z=NULL) == INVALID                       # zeros missing with has_zero = 1
    assert _gemm(lib, Z=ctypes.c_void_p(0x100001)) == INVALID  # zeros not 2-byte aligned
    assert _gemm(lib, S=ctypes.c_void_p(0x100002)) == INVALID  # uint4 scales: 4-byte loads
    assert b"4-byte" in lib.moe_last_error()
    # int8 scales are read 2 bytes at a time
    assert _gemm(lib, q=_q(8, 0, 0), Z=NULL, S=ctypes.c_void_p(0x100002), slots=0) == OK
    assert _gemm(lib, q=_q(8, 0, 0), Z=NULL, S=ctypes.c_void_p(0x100001)) == INVALID
    assert _gemm(lib, dt=2) == UNSUPPORTED
    assert _gemm(lib, K=300) == UNSUPPORTED
    assert _gemm(lib, N=1000) == UNSUPPORTED
    assert _gemm(lib, bm=24) == UNSUPPORTED
    assert _gemm(lib, bm=512) == UNSUPPORTED
    # 256-row blocks run the prefill kernel only: whole 256-column workgroups of N
    assert _gemm(lib, bm=256, N=1152) == UNSUPPORTED
    assert b"256" in lib.moe_last_error()
    assert _gemm(lib, bm=256, slots=0) == OK
    assert _gemm(lib, act=2) == INVALID
    assert _gemm(lib, rows=15) == INVALID                      # 15 rows * 2 < 32 slots
    assert _gemm(lib, A=ctypes.c_void_p(0x100008)) == INVALID  # A not 16-byte aligned
    assert _gemm(lib, Bw=NULL) == INVALID
    assert _gemm(lib, slots=0) == OK                           # nothing to do, no launch
    assert _gemm(lib, slots=0, rows=0, A=NULL, C=NULL, st=NULL, ex=NULL, npost=NULL) == OK
    # uint4 scales of the whole K range must fit in LDS beside the activation tiles
    assert _gemm(lib, K=36096 + 256, bm=16) == UNSUPPORTED
    assert b"LDS" in lib.moe_last_error()
    assert _gemm(lib, K=35840 + 256, bm=32) == UNSUPPORTED
    # block_m 64 and 128 keep two k-blocks of scales in LDS: a long K passes validation (a capacity
    # below one block leaves no block to launch, so nothing runs)
    assert _gemm(lib, K=65536, bm=128, rows=64, slots=32, cap=8) == OK


def test_fused_validation_and_workspace(lib):
    q4 = _q(4, 128, 1)
    ws = lib.fused_moe_wna16_workspace_size(16, 256, 512, 8, 2, q4, 0, 16)
    assert ws > 16 * 2 * 512 * 2                              # at least the intermediate rows
    assert lib.fused_moe_wna16_workspace_size(16, 256, 512, 8, 2, q4, 0, 24) == 0
    assert lib.fused_moe_wna16_workspace_size(16, 256, 512, 8, 2, q4, 0, 256) > ws
    assert (lib.fused_moe_wna16_workspace_size(64, 4096, 14336, 8, 2, q4, 0, 0)
            > lib.fused_moe_wna16_workspace_size(1, 4096, 14336, 8, 2, q4, 0, 0))

    def fused(**kw):
        a = dict(x=FAKE, lg=FAKE, M=16, H=256, I=512, E=8, k=2, rt=_rt(), w13=FAKE, s13=FAKE,
                 z13=FAKE, w2=FAKE, s2=FAKE, z2=FAKE, q=q4, dt=0, bm=16, ws=FAKE, wsb=ws,
                 out=FAKE, tw=NULL, ti=NULL)
        a.update(kw)
        return lib.fused_moe_wna16(a["x"], a["lg"], a["M"], a["H"], a["I"], a["E"], a["k"],
                                   a["rt"], a["w13"], a["s13"], a["z13"], a["w2"], a["s2"],
                                   a["z2"], a["q"], a["dt"], a["bm"], a["ws"], a["wsb"], a["out"],
                                   a["tw"], a["ti"], NULL)

    assert fused(wsb=ws - 1) == WORKSPACE
    assert b"workspace" in lib.moe_last_error()
    # DeepSeek-V3 prefill shape: 65535 tokens keep the intermediate under 2 GiB, 65536 do not
    big = dict(H=7168, I=2048, E=256, k=8, bm=0, wsb=1 << 62)
    assert fused(M=65536, **big) == UNSUPPORTED
    assert b"2 GiB" in lib.moe_last_error()
    assert fused(H=320) == UNSUPPORTED
    assert fused(I=200) == UNSUPPORTED
    assert fused(bm=8) == UNSUPPORTED
    assert fused(z2=NULL) == INVALID
    assert fused(out=NULL) == INVALID
    assert fused(ws=ctypes.c_void_p(0x100010)) == INVALID       # workspace needs 256-byte alignment
    assert fused(rt=_rt(1, 1, 3, 1)) == INVALID
    assert fused(M=0) == OK


def test_dense_gemm_validation_and_workspace(lib):
    q4, q8 = _q(4, 128, 1), _q(8, 0, 0)
    # the small-n benchmark shape (m 16, k 8192): n = 4096 splits K into float32 partials, n = 32768
    # has enough column chunks to split less, and a split never leaves fewer than 4 k-blocks
    ws4096 = lib.moe_wna16_dense_gemm_workspace_size(16, 4096, 8192, q4, 0)
    assert ws4096 > 0 and ws4096 % (16 * 4096 * 4) == 0
    assert ws4096 // (16 * 4096 * 4) <= 8192 // 128 // 4
    ws32k = lib.moe_wna16_dense_gemm_workspace_size(16, 32768, 8192, q4, 0)
    assert ws32k // (16 * 32768 * 4) < ws4096 // (16 * 4096 * 4)
    assert lib.moe_wna16_dense_gemm_workspace_size(16, 4096, 8192, _q(5, 128, 1), 0) == 0
    assert lib.moe_wna16_dense_gemm_workspace_size(0, 4096, 8192, q4, 0) == 0

    def dense(**kw):
        a = dict(A=FAKE, M=16, K=8192, Bw=FAKE, S=FAKE, Z=FAKE, q=q4, N=4096, dt=0, ws=FAKE,
                 wsb=ws4096, C=FAKE)
        a.update(kw)
        return lib.moe_wna16_dense_gemm(a["A"], a["M"], a["K"], a["Bw"], a["S"], a["Z"], a["q"],
                                        a["N"], a["dt"], a["ws"], a["wsb"], a["C"], NULL)

    assert dense(wsb=ws4096 - 1) == WORKSPACE
    assert dense(ws=NULL) == INVALID                            # a split needs the workspace
    assert dense(ws=ctypes.c_void_p(0x100010)) == INVALID       # 256-byte alignment
    assert dense(K=8000) == UNSUPPORTED
    assert dense(N=4000) == UNSUPPORTED
    assert dense(q=q8) == INVALID                               # int8 takes no zero points
    assert dense(Z=NULL) == INVALID
    assert dense(dt=3) == UNSUPPORTED
    assert dense(C=NULL) == INVALID
    assert dense(A=ctypes.c_void_p(0x100008)) == INVALID
    assert dense(M=-1) == INVALID
    assert dense(M=0) == OK


def test_batched_gemm_validation(lib):
    q4 = _q(4, 128, 1)

    def batched(**kw):
        a = dict(A=FAKE, E=8, T=16, K=512, cnt=FAKE, Bw=FAKE, S=FAKE, Z=FAKE, q=q4, N=256, dt=0,
                 bm=0, act=1, C=FAKE)
        a.update(kw)
        return lib.moe_wna16_batched_gemm(a["A"], a["E"], a["T"], a["K"], a["cnt"], a["Bw"], a["S"],
                                          a["Z"], a["q"], a["N"], a["dt"], a["bm"], a["act"],
                                          a["C"], NULL)

    assert batched(E=0) == INVALID
    assert batched(E=1025) == UNSUPPORTED
    assert batched(T=-1) == INVALID
    assert batched(act=2) == INVALID
    assert batched(bm=24) == UNSUPPORTED
    assert batched(K=384) == UNSUPPORTED
    assert batched(N=200) == UNSUPPORTED
    assert batched(cnt=NULL) == INVALID
    assert batched(cnt=ctypes.c_void_p(0x100002)) == INVALID   # counts need 4-byte alignment
    assert batched(C=ctypes.c_void_p(0x100008)) == INVALID
    assert batched(Z=NULL) == INVALID
    assert batched(T=0) == OK                                  # nothing to do, no launch
    # A (rows * K * 2 bytes) is bounded at 2 GiB, C (rows * N * 2) is not: 64 experts x 4096
    # tokens, K 2048, N 7168 (C 3.8 GB) passes the size checks and stops at C's alignment
    big = dict(E=64, T=4096, K=2048, N=7168, act=0)
    assert batched(C=ctypes.c_void_p(0x100008), **big) == INVALID
    assert b"alignment" in lib.moe_last_error()
    assert batched(C=ctypes.c_void_p(0x100008), **{**big, "T": 8192}) == UNSUPPORTED  # A: 2 GiB


def test_w8a8_validation(lib):
    assert lib.moe_quant_int8_rows(FAKE, 4, 300, 0, FAKE, FAKE, NULL) == UNSUPPORTED  # K % 256
    assert lib.moe_quant_int8_rows(FAKE, 4, 256, 2, FAKE, FAKE, NULL) == UNSUPPORTED  # dtype
    assert lib.moe_quant_int8_rows(FAKE, -1, 256, 0, FAKE, FAKE, NULL) == INVALID
    assert lib.moe_quant_int8_rows(FAKE, 4, 256, 0, NULL, FAKE, NULL) == INVALID
    assert lib.moe_quant_int8_rows(FAKE, 0, 256, 0, NULL, NULL, NULL) == OK         # no rows

    def w8(**kw):
        a = dict(A=FAKE, sa=FAKE, rows=32, div=2, Bw=FAKE, ws=FAKE, E=8, N=1024, K=256, dt=0,
                 st=FAKE, ex=FAKE, npost=FAKE, cap=152, bm=16, slots=32, tw=NULL, act=1, C=FAKE)
        a.update(kw)
        return lib.moe_w8a8_gemm(a["A"], a["sa"], a["rows"], a["div"], a["Bw"], a["ws"], a["E"],
                                 a["N"], a["K"], a["dt"], a["st"], a["ex"], a["npost"], a["cap"],
                                 a["bm"], a["slots"], a["tw"], a["act"], a["C"], NULL)

    assert w8(bm=24) == UNSUPPORTED
    # 256-row blocks only on the 32x32 integer kernel: N / 2 (act 1) a multiple of 128, N (act 0)
    # a multiple of 256
    assert w8(bm=256, N=1152) == UNSUPPORTED
    assert w8(bm=256, N=1152, act=0) == UNSUPPORTED
    assert w8(bm=512) == UNSUPPORTED
    assert w8(slots=0, rows=0, A=NULL, sa=NULL, C=NULL, st=NULL, ex=NULL, npost=NULL) == OK
    assert w8(K=320) == UNSUPPORTED
    assert w8(N=1000) == UNSUPPORTED
    assert w8(act=3) == INVALID
    assert w8(rows=15) == INVALID                               # 15 rows * 2 < 32 slots
    assert w8(sa=NULL) == INVALID
    assert w8(A=ctypes.c_void_p(0x100008)) == INVALID
    assert w8(dt=5) == UNSUPPORTED
    assert w8(slots=0) == OK
    # int32 sums of code products: K up to 131072 (127^2 * K < 2^31), one more k-block refused
    assert w8(K=131072 + 256, rows=8, slots=16, cap=8 * 2 + 8 * 15) == UNSUPPORTED
    assert b"int32" in lib.moe_last_error()

    def fused8(M, wsb, H=7168, I=2048, E=256, k=8):
        return lib.fused_moe_w8a8(FAKE, FAKE, M, H, I, E, k, _rt(), FAKE, FAKE, FAKE, FAKE, 1, 0,
                                  FAKE, wsb, FAKE, NULL, NULL, NULL)

    # DeepSeek-V3 int8 shape: the second GEMM's int8 activations (M * topk * I bytes) bound the
    # batch at 131071 tokens; the float32 rows after it are addressed with 64 bits.  (A one-byte
    # workspace stops the accepted call at its workspace check, before any launch.)
    assert fused8(4, 1 << 62, H=131072 + 256, I=256) == UNSUPPORTED
    assert b"int32" in lib.moe_last_error()
    assert fused8(131072, 1 << 62) == UNSUPPORTED
    assert b"2 GiB" in lib.moe_last_error()
    assert fused8(131071, 1) == WORKSPACE


def test_act_order_size_limits(lib):
    """The act-order layer's first GEMM reads the gathered rows [M * topk, H] with 32-bit offsets:
    at the DeepSeek-V3 shape 18724 tokens fit (stopped here by a one-byte workspace, before any
    launch) and 18725 are refused."""
    def ao(M, wsb):
        return lib.fused_moe_wna16_act_order(FAKE, FAKE, M, 7168, 2048, 256, 8, _rt(), FAKE, FAKE,
                                             FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, FAKE, wsb,
                                             FAKE, NULL, NULL, NULL)

    assert 18724 * 8 * 7168 * 2 < 2**31 <= 18725 * 8 * 7168 * 2
    assert ao(18725, 1 << 62) == UNSUPPORTED
    assert b"gathered" in lib.moe_last_error()
    assert ao(18724, 1) == WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError):
        B.lib()


def test_binding_rejects_mis_shaped_tensors():
    """The binding checks every tensor against the sizes it passes to the library (which trusts
    them) before any pointer is taken: CPU tensors of the wrong shape or dtype raise here."""
    import torch
    import weight_only_int4_topk_amd as B

    def raises(fn, what):
        with pytest.raises(B.MoeError, match=what):
            fn()

    E, H, I, M, k = 8, 256, 256, 4, 2
    lg = torch.zeros(M, E)
    raises(lambda: B.moe_topk_softmax(lg, k, B.routing(), topk_ids=torch.zeros(M, 3, dtype=torch.int32)),
           "topk_ids has shape")
    raises(lambda: B.moe_topk_softmax(lg.double(), k, B.routing()), "logits has dtype")
    raises(lambda: B.moe_align_block_size(torch.zeros(8, dtype=torch.int64), E, 16),
           "topk_ids has dtype")
    x = torch.zeros(M, H, dtype=torch.float16)
    w13 = torch.zeros(E, 2 * I, H // 2, dtype=torch.uint8)
    s13 = torch.zeros(E, 2 * I, H // 128, dtype=torch.float16)
    z13 = torch.zeros(E, 2 * I, H // 256, dtype=torch.uint8)
    w2 = torch.zeros(E, H, I // 2, dtype=torch.uint8)
    s2 = torch.zeros(E, H, I // 128, dtype=torch.float16)
    z2 = torch.zeros(E, H, I // 256, dtype=torch.uint8)
    args = (x, lg, k, B.routing(), w13, s13, z13, w2, s2, z2)
    raises(lambda: B.fused_moe_wna16(*args, out=torch.zeros(M, H - 8, dtype=torch.float16)),
           "out has shape")
    raises(lambda: B.fused_moe_wna16(*args, out=torch.zeros(M, H, dtype=torch.bfloat16)),
           "out has dtype")
    raises(lambda: B.fused_moe_wna16(*args, topk_ids=torch.zeros(M, k, dtype=torch.int64)),
           "topk_ids has dtype")
    raises(lambda: B.fused_moe_wna16(x, lg, k, B.routing(), w13, s13.bfloat16(), z13, w2, s2, z2),
           "w13 scales has dtype")
    raises(lambda: B.fused_moe_wna16(x, lg, k, B.routing(), w13, s13, z13, w2, s2[:, :, :1], z2),
           "w2 scales has shape")
    raises(lambda: B.fused_moe_wna16(x, lg[:, :4], k, B.routing(), w13, s13, z13, w2, s2, z2),
           "router_logits has shape")
    st = torch.zeros(152, dtype=torch.int32)
    ex = torch.zeros(10, dtype=torch.int32)
    npost = torch.zeros(1, dtype=torch.int32)
    raises(lambda: B.moe_wna16_gemm(x, k, w13, s13, z13, st, ex, npost, 16, M * k, act=1,
                                    C=torch.zeros(M * k, 2 * I, dtype=torch.float16)), "C has shape")
    raises(lambda: B.moe_wna16_gemm(x, k, w13, s13, z13, st, ex[:5], npost, 16, M * k, act=1),
           "expert_ids holds")
    raises(lambda: B.moe_wna16_gemm(x, k, w13, s13, z13, st, ex, npost, 16, M * k, act=1,
                                    topk_weights=torch.zeros(M * k - 1)), "topk_weights holds")
    raises(lambda: B.moe_wna16_dense_gemm(x, w13[0], s13[0], z13[0],
                                          C=torch.zeros(M, 2 * I + 16, dtype=torch.float16)),
           "C has shape")
    raises(lambda: B.moe_quant_int8_rows(x, q=torch.zeros(M, H, dtype=torch.uint8)), "q has dtype")
    w8 = torch.zeros(E, 2 * I, H, dtype=torch.int8)
    raises(lambda: B.moe_w8a8_gemm(torch.zeros(M, H, dtype=torch.int8), torch.zeros(M), k, w8,
                                   torch.zeros(E, 2 * I, dtype=torch.float16), st, ex, npost, 16,
                                   M * k, torch.bfloat16, act=1), "B scales has dtype")
    raises(lambda: B.fused_moe_w8a8(x, lg, k, B.routing(), w8, torch.zeros(E, 2 * I, dtype=torch.float16),
                                    torch.zeros(E, H, I + 256, dtype=torch.int8),
                                    torch.zeros(E, H, dtype=torch.float16)), "w2 has shape")
    raises(lambda: B.fused_moe_wna16_act_order(x, lg, k, B.routing(), w13, s13, z13,
                                               torch.zeros(E, H, dtype=torch.int64), w2, s2, z2,
                                               torch.zeros(E, I, dtype=torch.int32)),
           "w13_perm has dtype")
    raises(lambda: B.moe_wna16_batched_gemm(torch.zeros(E, 16, H, dtype=torch.float16),
                                            torch.zeros(E - 1, dtype=torch.int32), w13, s13, z13, act=1),
           "expert_num_tokens has shape")


def test_noalloc_scratch_limit(lib):
    """fused_moe_wna16_noalloc refuses, before any device call, a batch whose workspace exceeds its
    64 MiB static scratch (the Mixtral shape at 4096 tokens needs about 1.1 GB), and an empty
    batch returns at once."""
    q4 = _q(4, 128, 1)
    f = lib.fused_moe_wna16_noalloc
    assert lib.fused_moe_wna16_workspace_size(4096, 4096, 14336, 8, 2, q4, 0, 0) > (64 << 20)
    assert f(FAKE, FAKE, 4096, 4096, 14336, 8, 2, _rt(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, q4, 0,
             0, FAKE, NULL, NULL, NULL) == WORKSPACE
    assert b"static scratch" in lib.moe_last_error()
    assert f(FAKE, FAKE, 0, 4096, 14336, 8, 2, _rt(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, q4, 0,
             0, FAKE, NULL, NULL, NULL) == OK
    assert B.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_repack_validation(lib):
    f = lib.moe_repack_uint4
    def r(fmt=0, qw=FAKE, qz=FAKE, sc=FAKE, g=NULL, E=2, N=64, K=256, dt=0, b=FAKE, so=FAKE, zo=FAKE,
          perm=NULL, inv=NULL):
        return f(fmt, qw, qz, sc, g, E, N, K, dt, b, so, zo, perm, inv, NULL)
    assert r(fmt=2) == INVALID
    assert r(dt=3) == UNSUPPORTED
    assert r(K=300) == UNSUPPORTED
    assert r(N=60) == UNSUPPORTED                               # N % 8
    assert r(fmt=1, g=FAKE, perm=FAKE) == UNSUPPORTED           # AWQ has no act-order
    assert r(g=FAKE) == INVALID                                 # g_idx without perm_out
    assert r(perm=FAKE) == INVALID                              # perm_out without g_idx
    assert r(g=FAKE, perm=FAKE, K=16384 + 256) == UNSUPPORTED   # group ids staged in LDS
    assert r(qw=NULL) == INVALID
    assert r(b=ctypes.c_void_p(0x100008)) == INVALID            # B must be 16-byte aligned
    assert r(E=0) == INVALID
