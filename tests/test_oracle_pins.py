"""Pins of the CPU oracle against things other than itself: hand-worked fixtures, library routines,
closed forms, brute force and the quantisation error bound.  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth


# ------------------------------------------------------------------------------------------------
# storage decoding
# ------------------------------------------------------------------------------------------------
def test_uint4_layout_golden(golden):
    g = golden("uint4_layout.txt")
    period = bytes.fromhex(g["row_bytes_period"][0].replace(" ", ""))
    row = np.frombuffer(period * 16, dtype=np.uint8)[None, :]
    zeros = np.array([[int(g["zero_byte"][0], 16)]], dtype=np.uint8)
    sbits = [int(v, 16) for v in g["scales_fp16_bits"][0].split()]
    scales = np.array([sbits], dtype=np.uint16).view(np.float16)
    w = O.dequant_uint4(row, scales, zeros)[0]
    for item in g["expect"]:
        k, v = item.split()
        assert w[int(k)] == float(v), (k, w[int(k)], v)
    # and the whole row from the closed form of the fixture
    k = np.arange(256)
    q = (7 * k + 3) % 16
    ref = np.where(k < 128, (q - 3) * 0.5, (q - 12) * 0.25)
    assert np.array_equal(w, ref)


def test_unpack_is_inverse_of_encoder_packing():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(7, 512), dtype=np.uint8)
    packed = (torch.from_numpy(q[:, 0::2]) | (torch.from_numpy(q[:, 1::2]) << 4)).numpy()
    assert np.array_equal(O.unpack_uint4(packed), q)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_encode_decode_on_grid_is_exact(dt):
    """Weights placed exactly on a uint4 grid whose extremes hit codes 0 and 15 come back exactly:
    the encoder recovers (q, z, s) and the oracle's decoding reproduces w bit for bit."""
    rng = np.random.default_rng(2)
    N, K = 8, 512
    ng = K // 128
    s = np.array([[2.0 ** -rng.integers(4, 9) * (1 + rng.integers(0, 8) / 8) for _ in range(ng)]
                  for _ in range(N)])
    s = torch.tensor(s).to(dt).double().numpy()           # representable in the scale dtype
    z = rng.integers(1, 15, size=(N, ng))
    q = rng.integers(0, 16, size=(N, K))
    q[:, 0::128] = 0                                        # lo hits code 0
    q[:, 1::128] = 15                                       # hi hits code 15
    w = (q.reshape(N, ng, 128) - z[..., None]) * s[..., None]
    w = w.reshape(N, K)
    qp, sc, zp = synth.encode_uint4_g128(torch.tensor(w, dtype=torch.float64).float(), dt)
    assert np.array_equal(O.unpack_uint4(qp.numpy()), q)
    assert np.array_equal(O.unpack_uint4(zp.numpy()), z)
    assert np.array_equal(sc.double().numpy(), s)
    back = O.dequant_uint4(qp.numpy(), O.to_numpy(sc), zp.numpy())
    assert np.array_equal(back, w)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_uint4_error_bound_half_scale(dt):
    """Every dequantised weight is within s/2 of the drawn weight (asymmetric min/max, scale rounded
    up), and all codes are in [0, 15]."""
    g = torch.Generator().manual_seed(3)
    w = torch.randn(64, 1024, generator=g) * 0.02
    qp, sc, zp = synth.encode_uint4_g128(w, dt)
    back = O.dequant_uint4(qp.numpy(), O.to_numpy(sc), zp.numpy())
    s = np.repeat(O.to_numpy(sc).astype(np.float64), 128, axis=1)
    err = np.abs(back - w.double().numpy())
    assert (err <= s / 2).all(), float((err / s).max())
    # scale rounded up: 15 s >= hi - lo for every group
    wg = w.double().numpy().reshape(64, 8, 128)
    assert (15 * O.to_numpy(sc).astype(np.float64) >= wg.max(-1) - wg.min(-1)).all()


def test_int8_error_bound_half_scale():
    g = torch.Generator().manual_seed(4)
    w = torch.randn(32, 768, generator=g) * 0.02
    q, s = synth.encode_int8_channel(w, torch.bfloat16)
    assert int(q.abs().max()) <= 127
    back = O.dequant_int8(q.numpy(), O.to_numpy(s))
    err = np.abs(back - w.double().numpy())
    assert (err <= O.to_numpy(s).astype(np.float64)[:, None] / 2).all()


def test_dequant_bits_matches_torch_rounding():
    """The bit-exact dequantised object rounds (q - z) * s to the activation dtype; check the oracle's
    rounding against torch's float64 -> fp16 / float32 -> bf16 conversion (library routine)."""
    rng = np.random.default_rng(5)
    v = (rng.integers(-15, 16, 4096) * rng.uniform(1e-4, 1e-1, 4096))
    v32 = v.astype(np.float32).astype(np.float64)         # make each value an exact fp32
    assert np.array_equal(O.dequant_bits(v32, "fp16"),
                          torch.tensor(v32).to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(O.dequant_bits(v32, "bf16"),
                          torch.tensor(v32, dtype=torch.float32).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))


def _torch_round(x64, dt):
    t = torch.tensor(np.asarray(x64, np.float64)).float()       # float64 -> float32, RNE
    return t.to(torch.float16 if dt == "fp16" else torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_round_to_dtype_matches_torch_rounding(dt):
    """round_to_dtype (the rows the w8a8 layer's two GEMMs exchange) rounds float64 through float32
    to fp16 / bf16 to nearest even; check it against torch's conversions over signed values from
    fp16 subnormals to past the fp16 range, and on exact ties, where truncation or round-half-up
    would differ."""
    rng = np.random.default_rng(17)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(np.log(1e-8), np.log(1e5), 20000))
    np.testing.assert_array_equal(O.round_to_dtype(v, dt), _torch_round(v, dt))
    if dt == "bf16":
        # float32 bit patterns: the low half exactly 0x8000 is a tie (upper half 0x3F80 even,
        # 0x3F81 odd), and one unit above a tie rounds up
        u = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0xBF818000, 0x3F807FFF], np.uint32)
        want = np.array([0x3F800000, 0x3F820000, 0x3F810000, 0xBF820000, 0x3F800000], np.uint32)
        x = u.view(np.float32).astype(np.float64)
    else:
        # 1 + 2^-11 is halfway between 1 and 1 + 2^-10 (to even: 1); 1 + 3 * 2^-11 goes up to
        # 1 + 2^-9; 65520 is halfway between 65504 and the next binade (to even: inf); 2^-25 is
        # halfway between 0 and the smallest subnormal 2^-24 (to even: 0)
        x = np.array([1 + 2.0**-11, 1 + 3 * 2.0**-11, 65520.0, -(1 + 2.0**-11), 2.0**-25,
                      3 * 2.0**-25])
        want = np.array([1.0, 1 + 2.0**-9, np.inf, -1.0, 0.0, 2.0**-23]).astype(np.float32)
    np.testing.assert_array_equal(O.round_to_dtype(x, dt), want.view(np.float32).astype(np.float64)
                                  if dt == "bf16" else want.astype(np.float64))
    np.testing.assert_array_equal(O.round_to_dtype(x, dt), _torch_round(x, dt))


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------
def _ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


def test_exp_spec_within_one_ulp_of_libm():
    x = np.linspace(-80, 80, 200001, dtype=np.float32)
    got = O.exp_f32_spec(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    err = np.abs(got - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert err.max() <= 1.5, err.max()


def test_sigmoid_spec_close_to_exact():
    x = np.linspace(-20, 20, 100001, dtype=np.float32)
    got = O.sigmoid_f32_spec(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    err = np.abs(got - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    # exp error (<= 1.5 ulp) + rounding of 1 + e + rounding of the division, each up to 0.5 ulp
    # relative, measured in ulps of the result's binade (up to 2x apart): at most 3 ulp
    assert err.max() <= 3.0, err.max()
    assert O.sigmoid_f32_spec(np.float32(0.0)) == np.float32(0.5)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 8)])
def test_route_softmax_vs_argsort(E, k):
    rng = np.random.default_rng(E)
    lg = rng.standard_normal((40, E)).astype(np.float32)
    ids, w = O.route_softmax(lg, k, renormalize=True)
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable")[:, :k])
    # renormalised softmax over the chosen experts == softmax of the chosen logits alone
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-12)
    ids2, w2 = O.route_softmax(lg, k, renormalize=False)
    full = torch.softmax(torch.tensor(lg, dtype=torch.float64), dim=1).numpy()
    np.testing.assert_allclose(w2, np.take_along_axis(full, ids2.astype(np.int64), 1), rtol=1e-12)


def test_route_softmax_ties_go_to_lower_id():
    lg = np.array([[0.5, 1.0, 1.0, -1.0, 1.0]], np.float32)
    ids, _ = O.route_softmax(lg, 3)
    assert ids.tolist() == [[1, 2, 4]]


def _brute_grouped(sig, num_groups, topk_groups, topk):
    """Brute force: score every group by the best pair sum, try every set of kept groups, keep the
    set with the largest total score, then the topk experts inside by sigma."""
    E = sig.size
    gs = E // num_groups
    score = []
    for g in range(num_groups):
        m = sig[g * gs:(g + 1) * gs]
        if gs == 1:
            score.append(float(m[0]))
        else:
            score.append(max(float(np.float32(m[a]) + np.float32(m[b]))
                             for a in range(gs) for b in range(gs) if a != b))
    best = max(itertools.combinations(range(num_groups), topk_groups),
               key=lambda c: sum(score[g] for g in c))
    cand = [e for e in range(E) if e // gs in best]
    cand.sort(key=lambda e: -float(sig[e]))
    return cand[:topk]


@pytest.mark.parametrize("E,ng,tg,k", [(256, 8, 4, 8), (64, 8, 3, 6), (32, 4, 2, 4)])
def test_route_sigmoid_grouped_vs_brute_force(E, ng, tg, k):
    rng = np.random.default_rng(E + ng)
    lg = rng.standard_normal((30, E)).astype(np.float32)
    ids, w = O.route_sigmoid_grouped(lg, k, ng, tg, renormalize=True, scale=2.5)
    sig = O.sigmoid_f32_spec(lg)
    for m in range(lg.shape[0]):
        assert ids[m].tolist() == _brute_grouped(sig[m], ng, tg, k)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-12)
    # weights are proportional to sigma of the chosen experts
    s_sel = np.take_along_axis(sig.astype(np.float64), ids.astype(np.int64), 1)
    np.testing.assert_allclose(w / s_sel, (w / s_sel)[:, :1].repeat(k, 1), rtol=1e-12)


def test_route_sigmoid_single_group_is_plain_topk():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((50, 64)).astype(np.float32)
    ids, _ = O.route_sigmoid_grouped(lg, 6, 1, 1)
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable")[:, :6])


# ------------------------------------------------------------------------------------------------
# align
# ------------------------------------------------------------------------------------------------
def test_align_golden(golden):
    g = golden("align_example.txt")
    ids = np.array([int(v) for v in g["topk_ids"][0].split()], np.int32).reshape(-1, 2)
    for case in ("A", "B", "C"):
        E = int(g[f"{case}.E"][0])
        bm = int(g[f"{case}.block_m"][0])
        st, ex, T = O.align_block_size(ids, E, bm)
        assert st.tolist() == [int(v) for v in g[f"{case}.sorted_token_ids"][0].split()]
        assert ex.tolist() == [int(v) for v in g[f"{case}.expert_ids"][0].split()]
        assert T == int(g[f"{case}.num_tokens_post_padded"][0])


def _align_by_argsort(flat, E, bm):
    order = np.argsort(flat, kind="stable")       # library stable sort
    cnt = np.bincount(flat, minlength=E)
    pieces, experts = [], []
    start = 0
    for e in range(E):
        c = int(cnt[e])
        if c == 0:
            continue
        p = -(-c // bm) * bm
        pieces.append(np.concatenate([order[start:start + c], np.full(p - c, flat.size)]))
        experts += [e] * (p // bm)
        start += c
    return np.concatenate(pieces), np.array(experts)


@pytest.mark.parametrize("M,k,E,bm", [(16, 2, 8, 16), (1, 8, 256, 16), (64, 8, 256, 32),
                                      (512, 8, 64, 64), (333, 2, 8, 128), (7, 3, 5, 4)])
def test_align_vs_stable_sort_and_invariants(M, k, E, bm):
    rng = np.random.default_rng(M * 31 + E)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    flat = ids.reshape(-1)
    st, ex, T = O.align_block_size(ids, E, bm)
    ref_st, ref_ex = _align_by_argsort(flat, E, bm)
    assert T == ref_st.size
    assert np.array_equal(st[:T], ref_st)
    assert np.array_equal(ex[:T // bm], ref_ex)
    cap = O.align_capacity(flat.size, E, bm)
    assert st.size == cap and T <= cap and T % bm == 0
    assert (st[T:] == flat.size).all() and (ex[T // bm:] == -1).all()
    real = st[st < flat.size]
    assert np.array_equal(np.sort(real), np.arange(flat.size))    # a permutation of the slots
    for b in range(T // bm):                                        # every block single-expert
        blk = st[b * bm:(b + 1) * bm]
        blk = blk[blk < flat.size]
        assert (flat[blk] == ex[b]).all()


# ------------------------------------------------------------------------------------------------
# the layer
# ------------------------------------------------------------------------------------------------
def _tiny_layer(E=4, H=256, I=256, bits=4, dt="fp16", seed=0):
    wl = synth.Workload("t", E=E, H=H, I=I, topk=2, Ms=(5,), dtype=dt, bits=bits)
    return wl, synth.make_layer(wl, seed=seed)


@pytest.mark.parametrize("bits,dt", [(4, "fp16"), (4, "bf16"), (8, "bf16")])
def test_layer_vs_dense_all_experts(bits, dt):
    """Dense formulation: evaluate every expert on every token with explicit loops over experts and
    a dense gate matrix that is zero off the chosen experts; must equal the routed oracle."""
    wl, layer = _tiny_layer(bits=bits, dt=dt)
    x = synth.make_x(wl, 5, seed=1)
    lg = synth.make_logits(wl, 5, seed=1)
    ids, w = O.route_softmax(O.to_numpy(lg), 2)
    src = O.ExpertSource(layer, bits)
    out = O.moe_layer(x, ids, w, src)
    x64 = O.to_numpy(x).astype(np.float64)
    G = np.zeros((5, wl.E))
    for m in range(5):
        for j in range(2):
            G[m, ids[m, j]] += w[m, j]
    ref = np.zeros_like(out)
    for e in range(wl.E):
        W13, W2 = src.w13(e), src.w2(e)
        t = torch.tensor(x64)
        h = t @ torch.tensor(W13).T
        a = torch.nn.functional.silu(h[:, :wl.I]) * h[:, wl.I:]
        ref += G[:, e:e + 1] * (a @ torch.tensor(W2).T).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)


def test_layer_one_expert_weight_one_is_dense_ffn_of_drawn_weights():
    """Route every token to one expert with weight 1 and put the drawn weights exactly on the quant
    grid: the layer equals the dense SwiGLU FFN of the original float weights (torch, float64)."""
    wl = synth.Workload("t", E=3, H=256, I=256, topk=1, Ms=(6,), dtype="fp16")
    w13, w2 = synth.expert_weights_fp32(wl, 1, seed=7)
    # snap to the grid the encoder would produce, so encoding is lossless
    q13, s13, z13 = synth.encode_uint4_g128(w13, torch.float16)
    q2, s2, z2 = synth.encode_uint4_g128(w2, torch.float16)
    W13 = O.dequant_uint4(q13.numpy(), O.to_numpy(s13), z13.numpy())
    W2 = O.dequant_uint4(q2.numpy(), O.to_numpy(s2), z2.numpy())
    layer = synth.make_layer(wl, seed=7)
    src = O.ExpertSource(layer, 4)
    x = synth.make_x(wl, 6, seed=7)
    ids = np.ones((6, 1), np.int32)
    out = O.moe_layer(x, ids, np.ones((6, 1)), src)
    t = torch.tensor(O.to_numpy(x), dtype=torch.float64)
    h1 = t @ torch.tensor(W13[:256]).T
    h3 = t @ torch.tensor(W13[256:]).T
    ref = (torch.nn.functional.silu(h1) * h3) @ torch.tensor(W2).T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-15)
    # and the dequantised grid is within s/2 of the original draws
    assert np.abs(W13 - w13.double().numpy()).max() <= O.to_numpy(s13).max() / 2


def test_layer_brute_force_python_loops():
    """Tiny case with plain Python loops (no numpy products) for the FFN of each routed slot."""
    wl = synth.Workload("t", E=3, H=256, I=256, topk=2, Ms=(2,), dtype="fp16")
    layer = synth.make_layer(wl, seed=11)
    src = O.ExpertSource(layer, 4)
    x = O.to_numpy(synth.make_x(wl, 2, seed=11)).astype(np.float64)
    lg = O.to_numpy(synth.make_logits(wl, 2, seed=11))
    ids, w = O.route_softmax(lg, 2)
    out = O.moe_layer(x, ids, w, src)
    for m in range(2):
        acc = [0.0] * wl.H
        for j in range(2):
            W13 = src.w13(ids[m, j]).tolist()
            W2 = src.w2(ids[m, j]).tolist()
            xm = x[m].tolist()
            h = [sum(W13[r][c] * xm[c] for c in range(wl.H)) for r in range(2 * wl.I)]
            a = [h[i] / (1.0 + math.exp(-h[i])) * h[wl.I + i] for i in range(wl.I)]
            for r in range(wl.H):
                acc[r] += w[m, j] * sum(W2[r][i] * a[i] for i in range(wl.I))
        np.testing.assert_allclose(out[m], acc, rtol=1e-10, atol=1e-14)


def test_grouped_gemm_definition_matches_layer():
    """GEMM1 with SiLU-and-mul, then GEMM2 scaled by the routing weight, summed over j in order,
    equals the per-token layer (two formulations over the align output)."""
    wl = synth.WORKLOADS["tiny"]
    layer = synth.make_layer(wl, seed=0)
    src = O.ExpertSource(layer, 4)
    M = 16
    x = synth.make_x(wl, M)
    lg = synth.make_logits(wl, M)
    ids, w = O.route_softmax(O.to_numpy(lg), wl.topk)
    st, ex, T = O.align_block_size(ids, wl.E, 16)
    ns = M * wl.topk
    a = O.grouped_gemm(x, wl.topk, src.w13, st, ex, T, 16, ns, act=1)
    A = np.stack([a[s] for s in range(ns)])
    y = O.grouped_gemm(A, 1, src.w2, st, ex, T, 16, ns, topk_weights=w)
    out = np.zeros((M, wl.H))
    for m in range(M):
        for j in range(wl.topk):
            out[m] += y[m * wl.topk + j]
    np.testing.assert_allclose(out, O.moe_layer(x, ids, w, src), rtol=1e-12, atol=1e-16)


# ---- dense GEMM (one weight matrix, every row routed) -------------------------------------------
def _pack_nibbles(v):
    """uint4 codes [R, 2n] -> bytes [R, n], even index in bits 0-3 (written here, not the oracle's)."""
    v = np.asarray(v, dtype=np.uint8)
    return (v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8)


def test_dense_gemm_uint4_equals_matmul_of_grid_weights():
    """Integer codes, zero points and power-of-two-ish scales chosen here: C must be A @ W^T of the
    weights (q - z) * s built directly from them.  N != K != M, so a transposed operand fails."""
    rng = np.random.default_rng(11)
    M, N, K = 5, 24, 512
    ng = K // 128
    q = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, ng))
    s = 2.0 ** -rng.integers(3, 9, size=(N, ng)).astype(np.float64)
    W = ((q.reshape(N, ng, 128) - z[..., None]) * s[..., None]).reshape(N, K)
    A = rng.standard_normal((M, K))
    C = O.dense_gemm(A, _pack_nibbles(q), s, _pack_nibbles(z))
    assert C.shape == (M, N)
    np.testing.assert_allclose(C, A @ W.T, rtol=1e-12, atol=1e-15)


def test_dense_gemm_int8_equals_matmul_of_grid_weights():
    rng = np.random.default_rng(12)
    M, N, K = 3, 40, 256
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s = 2.0 ** -rng.integers(5, 12, size=N).astype(np.float64)
    A = rng.standard_normal((M, K))
    np.testing.assert_allclose(O.dense_gemm(A, q, s), A @ (q.astype(np.float64) * s[:, None]).T,
                               rtol=1e-12, atol=1e-15)


def test_dense_gemm_one_hot_rows_read_back_weight_columns():
    """A = one-hot rows selecting k_i: row i of C is column k_i of the decoded weights, exactly."""
    rng = np.random.default_rng(13)
    N, K = 16, 256
    q = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, K // 128))
    s = rng.uniform(0.01, 0.1, size=(N, K // 128))
    ks = np.array([0, 1, 127, 128, 200, 255])
    A = np.zeros((len(ks), K))
    A[np.arange(len(ks)), ks] = 1.0
    C = O.dense_gemm(A, _pack_nibbles(q), s, _pack_nibbles(z))
    expect = (q[:, ks] - z[:, ks // 128]) * s[:, ks // 128]
    assert np.array_equal(C, expect.T)


def test_dense_gemm_is_the_one_expert_grouped_gemm():
    """The dense case of the grouped GEMM: one expert, every row its own slot (align of all-zero ids)."""
    rng = np.random.default_rng(14)
    M, N, K = 20, 32, 256
    q = rng.integers(0, 16, size=(1, N, K))
    z = rng.integers(0, 16, size=(1, N, K // 128))
    s = rng.uniform(0.01, 0.1, size=(1, N, K // 128))
    qp, zp = _pack_nibbles(q[0]), _pack_nibbles(z[0])
    A = rng.standard_normal((M, K))
    st, ex, T = O.align_block_size(np.zeros(M, dtype=np.int32), 1, 16)
    rows = O.grouped_gemm(A, 1, lambda e: O.dequant_uint4(qp, s[0], zp), st, ex, T, 16, M)
    dense = O.dense_gemm(A, qp, s[0], zp)
    for r in range(M):
        np.testing.assert_allclose(rows[r], dense[r], rtol=1e-13, atol=1e-15)


# ---- batched-experts activation format --------------------------------------------------------
def test_batched_gemm_is_the_grouped_gemm_of_the_same_rows():
    """Rows of A [E, T, K] below each expert's count, routed as slots to that expert through the
    align definition, give the same products (SiLU and plain); rows past a count are absent."""
    rng = np.random.default_rng(21)
    E, T, K, N = 3, 5, 256, 32
    counts = np.array([5, 0, 2])
    q = rng.integers(0, 16, size=(E, N, K))
    z = rng.integers(0, 16, size=(E, N, K // 128))
    s = rng.uniform(0.01, 0.1, size=(E, N, K // 128))
    W = [((q[e].reshape(N, 2, 128) - z[e][..., None]) * s[e][..., None]).reshape(N, K) for e in range(E)]
    A = rng.standard_normal((E, T, K))
    # the same rows as slots of a grouped GEMM: slot list in (e, r) order, ids = e
    pairs = [(e, r) for e in range(E) for r in range(counts[e])]
    A_rows = np.stack([A[e, r] for e, r in pairs])
    ids = np.array([e for e, _ in pairs], np.int32)
    st, ex, Tp = O.align_block_size(ids, E, 16)
    for act in (0, 1):
        b = O.batched_gemm(A, counts, lambda e: W[e], act=act)
        g = O.grouped_gemm(A_rows, 1, lambda e: W[e], st, ex, Tp, 16, len(pairs), act=act)
        assert sorted(b) == sorted(pairs)
        for i, pr in enumerate(pairs):
            np.testing.assert_allclose(b[pr], g[i], rtol=1e-13, atol=1e-15)
            # and the plain definition, written out
            h = W[pr[0]] @ A[pr]
            ref = h if act == 0 else (h[: N // 2] / (1 + np.exp(-h[: N // 2]))) * h[N // 2:]
            np.testing.assert_allclose(b[pr], ref, rtol=1e-12, atol=1e-15)


def test_batched_gemm_counts_are_clamped_to_the_batch():
    rng = np.random.default_rng(22)
    A = rng.standard_normal((2, 3, 256))
    W = [rng.standard_normal((16, 256)) for _ in range(2)]
    out = O.batched_gemm(A, np.array([7, -1]), lambda e: W[e])
    assert sorted(out) == [(0, 0), (0, 1), (0, 2)]


# ---- w8a8: per-token int8 activations, per-channel int8 weights ---------------------------------
def test_quant_int8_rows_error_bound_and_range():
    """|q * s - x| <= s / 2 for every element (round to nearest), codes in [-127, 127], the row
    maximum maps to +-127, and a zero row gives zero codes and scale 0."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((9, 512)) * 0.1).astype(np.float32)
    x[3] = 0.0
    q, s = O.quant_int8_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(q.astype(np.int32)).max() <= 127
    assert s[3] == 0 and not q[3].any()
    for r in range(9):
        if r == 3:
            continue
        err = np.abs(q[r].astype(np.float64) * s[r] - x[r].astype(np.float64))
        assert (err <= s[r] / 2 * (1 + 1e-6)).all()
        assert np.abs(q[r]).max() == 127


def test_quant_int8_rows_on_grid_is_exact():
    """Rows that are integer multiples of a power-of-two step, with the extreme at 127 steps,
    come back as exactly those integers."""
    rng = np.random.default_rng(32)
    codes = rng.integers(-127, 128, size=(4, 256))
    codes[:, 0] = 127
    step = np.float32(2.0 ** -9)
    x = (codes * step).astype(np.float32)
    q, s = O.quant_int8_rows(x)
    assert np.array_equal(q, codes.astype(np.int8))
    assert np.all(s == np.float32(127 * step) / np.float32(127))


def test_w8a8_grouped_gemm_is_the_scaled_integer_product():
    """Against the products written out per slot with integer dot products, on a tiny routed
    batch; a non-square weight so a transposed operand fails."""
    rng = np.random.default_rng(33)
    E, N, K, M, k = 3, 24, 256, 5, 2
    qw = rng.integers(-127, 128, size=(E, N, K)).astype(np.int8)
    ws = rng.uniform(0.001, 0.01, size=(E, N))
    x = (rng.standard_normal((M, K)) * 0.1).astype(np.float32)
    Aq, sa = O.quant_int8_rows(x)
    ids = np.array([[0, 2], [1, 2], [2, 0], [1, 0], [2, 1]], np.int32)
    st, ex, T = O.align_block_size(ids, E, 16)
    for act in (0, 1):
        got = O.w8a8_grouped_gemm(Aq, sa, k, lambda e: (qw[e], ws[e]), st, ex, T, 16, M * k, act=act)
        for s in range(M * k):
            e, row = ids.reshape(-1)[s], s // k
            h = np.array([float(sum(int(a) * int(b) for a, b in zip(Aq[row], qw[e, n])))
                          for n in range(N)]) * float(sa[row]) * ws[e]
            if act:
                h = h[: N // 2] / (1 + np.exp(-h[: N // 2])) * h[N // 2:]
            np.testing.assert_allclose(got[s], h, rtol=1e-13, atol=1e-15)


def test_w8a8_layer_is_the_grouped_pipeline():
    """The per-token layer definition equals the grouped form: GEMM1 with SiLU over align output,
    rows rounded to the activation dtype and quantised per slot, GEMM2, then the weighted sum in
    slot order; and it stays within int8 quantisation error of the float layer on the same weights."""
    wl = synth.Workload("l8", E=4, H=256, I=256, topk=2, Ms=(6,), dtype="bf16", bits=8)
    layer = synth.make_layer(wl, seed=12)
    x = synth.make_x(wl, 6, seed=12)
    ids, w = O.route(O.to_numpy(synth.make_logits(wl, 6, seed=12)), 2)
    L = {k: O.to_numpy(v) for k, v in layer.items() if v is not None}
    ref = O.moe_layer_w8a8_rows(x, ids, w, L, "bf16")
    xq, xs = O.quant_int8_rows(x)
    st, ex, T = O.align_block_size(ids, wl.E, 16)
    ns = 12
    g1 = O.w8a8_grouped_gemm(xq, xs, 2, lambda e: (L["w13"][e], L["w13_scales"][e]), st, ex, T, 16,
                             ns, act=1)
    inter = np.stack([O.round_to_dtype(g1[s], "bf16") for s in range(ns)]).astype(np.float32)
    iq, isc = O.quant_int8_rows(inter)
    g2 = O.w8a8_grouped_gemm(iq, isc, 1, lambda e: (L["w2"][e], L["w2_scales"][e]), st, ex, T, 16, ns)
    grouped = np.stack([w[m, 0] * g2[2 * m] + w[m, 1] * g2[2 * m + 1] for m in range(6)])
    np.testing.assert_allclose(ref, grouped, rtol=1e-12, atol=1e-15)
    flt = O.moe_layer(x, ids, w, O.ExpertSource(layer, 8))
    assert np.linalg.norm(ref - flt) / np.linalg.norm(flt) < 2e-2


# ---- GPTQ act-order: input columns carry their group index ------------------------------------
def test_dequant_gidx_in_column_order_is_plain_decoding():
    """With g_idx[k] = k // 128 the group-indexed decoding is the plain one."""
    rng = np.random.default_rng(41)
    N, K = 8, 512
    q = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, K // 128))
    s = rng.uniform(0.01, 0.1, size=(N, K // 128))
    got = O.dequant_uint4_gidx(_pack_nibbles(q), s, _pack_nibbles(z), np.arange(K) // 128)
    np.testing.assert_array_equal(got, O.dequant_uint4(_pack_nibbles(q), s, _pack_nibbles(z)))


def test_dequant_gidx_sorted_columns_give_the_grouped_storage():
    """Columns permuted so that every group is contiguous (the sorted storage the layer reads) decode
    to the same weights: w_gidx[:, perm] equals the plain decoding of the permuted codes, with
    perm = stable argsort(g_idx) and w written out per element."""
    rng = np.random.default_rng(42)
    N, K = 6, 768
    perm_true = rng.permutation(K)
    g_idx = np.empty(K, np.int64)
    g_idx[perm_true] = np.arange(K) // 128                 # group g = columns perm_true[128g:...]
    q = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, K // 128))
    s = rng.uniform(0.01, 0.1, size=(N, K // 128))
    w = O.dequant_uint4_gidx(_pack_nibbles(q), s, _pack_nibbles(z), g_idx)
    for n, k in [(0, 0), (5, 767), (3, 400)]:
        assert w[n, k] == (q[n, k] - z[n, g_idx[k]]) * s[n, g_idx[k]]
    perm = np.argsort(g_idx, kind="stable")
    sorted_w = O.dequant_uint4(_pack_nibbles(q[:, perm]), s, _pack_nibbles(z))
    np.testing.assert_array_equal(w[:, perm], sorted_w)


# ---- GPTQ / AWQ checkpoint storage -> canonical storage ----------------------------------------
def _pack_words(vals):
    """[..., 8] nibble values -> int32 words (value i in bits 4i..4i+3), written out directly."""
    v = np.asarray(vals, dtype=np.int64)
    w = np.zeros(v.shape[:-1], np.int64)
    for i in range(8):
        w |= v[..., i] << (4 * i)
    return w.astype(np.uint32).view(np.int32)


def _golden_expert():
    K, N = 256, 8
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    q = (k + 3 * n) % 16                                        # [K, N]
    g = np.arange(K // 128)[:, None]
    z = (g + n + 1) % 16                                        # [G, N]
    s = (0.125 * (g + 1) + 0.0078125 * n).astype(np.float16)    # [G, N]
    return q, z, s


def test_gptq_awq_unpack_golden(golden):
    """The hand-worked words of tests/golden/gptq_awq_layout.txt: the test packs whole tensors by
    the stated layout (its own code), checks those words, and the oracle unpacks them back."""
    g = golden("gptq_awq_layout.txt")
    q, z, s = _golden_expert()
    K, N = q.shape
    # GPTQ: word [k8, n] = codes k = 8 k8 .. 8 k8 + 7; zeros word [g, n8] = columns 8 n8 ..
    gq = _pack_words(q.reshape(K // 8, 8, N).transpose(0, 2, 1))
    gz = _pack_words(z.reshape(z.shape[0], N // 8, 8))
    # AWQ: word [k, n8], nibble j = column 8 n8 + order[j]
    order = list(O.AWQ_PACK_ORDER)
    aq = _pack_words(q.reshape(K, N // 8, 8)[..., order])
    az = _pack_words(z.reshape(z.shape[0], N // 8, 8)[..., order])
    h = lambda v: int(v) & 0xFFFFFFFF
    assert h(gq[0, 0]) == int(g["gptq.qweight[0,0]"][0], 16)
    assert h(gq[1, 1]) == int(g["gptq.qweight[1,1]"][0], 16)
    assert h(gz[0, 0]) == int(g["gptq.qzeros[0,0]"][0], 16)
    assert h(aq[0, 0]) == int(g["awq.qweight[0,0]"][0], 16)
    assert h(az[1, 0]) == int(g["awq.qzeros[1,0]"][0], 16)
    for unpack, (wq, wz) in ((O.unpack_gptq, (gq, gz)), (O.unpack_awq, (aq, az))):
        uq, uz = unpack(wq, wz)
        np.testing.assert_array_equal(uq, q)
        np.testing.assert_array_equal(uz, z)


def test_canonical_from_checkpoint_golden(golden):
    g = golden("gptq_awq_layout.txt")
    q, z, s = _golden_expert()
    B, sc, zz, perm = O.canonical_from_checkpoint(q, z, s)
    assert perm is None
    assert B[1, 0] == int(g["canon.B[1,0]"][0], 16)
    assert B[0, 5] == int(g["canon.B[0,5]"][0], 16)
    assert zz[2, 0] == int(g["canon.zeros[2,0]"][0], 16)
    assert float(sc[3, 1]) == float(g["canon.scales[3,1]"][0])
    # the canonical storage decodes to (q - z) * s of the checkpoint, element by element
    w = O.dequant_uint4(B, sc, zz)
    for (kk, nn) in [(0, 0), (255, 7), (130, 3)]:
        assert w[nn, kk] == (q[kk, nn] - z[kk // 128, nn]) * float(s[kk // 128, nn])
    # act-order
    g_idx = (np.arange(256) // 2) % 2
    B2, sc2, zz2, perm = O.canonical_from_checkpoint(q, z, s, g_idx)
    assert perm[0:4].tolist() == [int(v) for v in g["act.perm.0_to_3"][0].split()]
    assert perm[128:132].tolist() == [int(v) for v in g["act.perm.128_to_131"][0].split()]
    assert B2[0, 1] == int(g["act.B[0,1]"][0], 16)
    assert B2[0, 64] == int(g["act.B[0,64]"][0], 16)
    # the sorted storage with its permutation decodes like the GPTQ definition with g_idx
    qpacked_orig = (q.T[:, 0::2] | (q.T[:, 1::2] << 4)).astype(np.uint8)
    w_gidx = O.dequant_uint4_gidx(qpacked_orig, s.T, zz2, g_idx)
    np.testing.assert_array_equal(O.dequant_uint4(B2, sc2, zz2), w_gidx[:, perm])
