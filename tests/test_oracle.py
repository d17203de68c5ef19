"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: an explicit
dense-transition brute force, closed forms, textbook special cases, the
chunk (WY) algebra computed separately in fp64, invariants of the
recurrence (split = chain, linearity), and the page's worked chunk-table
example.  Non-square key/value sizes (dk != dv) make a transposed operand
fail loudly.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, lengths, H, dk, dv, h0=True, gscale=5.0):
    lengths = list(lengths)
    T = int(sum(lengths))
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q = rng.standard_normal((T, H, dk)).astype(np.float32) / np.float32(math.sqrt(dk))
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True).astype(np.float32)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    g = (-gscale / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((N, H, dk, dv))).astype(np.float32) if h0 else None
    return q, k, v, g, beta, cu, S0


def rel(a, b):
    return oracle.rel_fro_err(a, b)


@pytest.mark.parametrize("dk,dv", [(8, 6), (5, 9), (128, 128)])
def test_token_oracle_matches_dense_brute_force(dk, dv):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [13, 0, 19], H=2, dk=dk, dv=dv)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0, scale=0.7)
    ob, fb = oracle.brute_force(q, k, v, g, beta, cu, S0, scale=0.7)
    assert rel(o, ob) < 1e-12
    assert rel(fin, fb) < 1e-12


def test_token_oracle_brute_force_without_initial_state():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, cu, _ = rand_inputs(rng, [32], H=3, dk=16, dv=12, h0=False)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, None)
    ob, fb = oracle.brute_force(q, k, v, g, beta, cu, None)
    assert rel(o, ob) < 1e-12 and rel(fin, fb) < 1e-12


def test_beta_zero_is_pure_decay_closed_form():
    rng = np.random.default_rng(13)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [40, 7, 0, 25], H=2, dk=16, dv=10)
    beta[:] = 0.0
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0)
    oc, fc = oracle.decay_closed_form(q, g, cu, S0)
    assert rel(o, oc) < 1e-12
    assert rel(fin, fc) < 1e-12


def test_beta_zero_g_zero_is_a_plain_readout():
    # g = 0 and beta = 0: the state is frozen, o_t = scale * S_0^T q_t.
    rng = np.random.default_rng(14)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [30], H=1, dk=12, dv=7)
    g[:] = 0.0
    beta[:] = 0.0
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0, scale=0.5)
    expect = 0.5 * q[:, 0].astype(np.float64) @ S0[0, 0].astype(np.float64)
    assert np.max(np.abs(o[:, 0] - expect)) < 1e-13
    assert np.array_equal(fin[0, 0], S0[0, 0].astype(np.float64))


def test_orthonormal_keys_reduce_to_causal_linear_attention():
    rng = np.random.default_rng(15)
    T, dk, dv = 24, 32, 20
    q, _, v, _, beta, cu, _ = rand_inputs(rng, [T], H=2, dk=dk, dv=dv, h0=False)
    k = np.zeros((T, 2, dk), dtype=np.float64)
    for h in range(2):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[:, h] = Qm[:, :T].T                         # T orthonormal keys
    g = np.zeros((T, 2, dk), dtype=np.float32)
    o, _ = oracle.kda_fwd(q, k, v, g, beta, cu, None)
    ol = oracle.linear_attention(q, k, v, beta)
    # k went through fp32 on its way into the oracle; compare against the
    # same fp32 keys.
    ol32 = oracle.linear_attention(q, k.astype(np.float32), v, beta)
    assert rel(o, ol32) < 1e-6
    assert rel(ol, ol32) < 1e-6


def test_one_hot_key_with_unit_beta_overwrites_the_slot():
    # g = 0, beta = 1, k = e_i: S[i,:] is replaced by v_t, other rows kept.
    rng = np.random.default_rng(16)
    dk, dv, T = 6, 5, 9
    slots = rng.integers(0, dk, size=T)
    k = np.zeros((T, 1, dk), dtype=np.float32)
    k[np.arange(T), 0, slots] = 1.0
    q = rng.standard_normal((T, 1, dk)).astype(np.float32)
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    g = np.zeros((T, 1, dk), dtype=np.float32)
    beta = np.ones((T, 1), dtype=np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32)
    cu = np.array([0, T], dtype=np.int32)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0, scale=1.0)
    S = S0[0, 0].astype(np.float64).copy()
    for t in range(T):
        S[slots[t]] = v[t, 0]
        assert np.allclose(o[t, 0], S.T @ q[t, 0].astype(np.float64), atol=1e-12)
    assert np.allclose(fin[0, 0], S, atol=1e-12)


def test_split_equals_chain_bitwise():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [150], H=2, dk=16, dv=8)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0)
    cut = 67
    cuA = np.array([0, cut], dtype=np.int32)
    cuB = np.array([0, 150 - cut], dtype=np.int32)
    oA, fA = oracle.kda_fwd(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], cuA, S0)
    # the chained call gets the fp64 state; feed it through float64 inputs
    # by running the brute force free variant: compare against the packed
    # run of [A;B] as two sequences with B's initial state = fA.
    cu2 = np.array([0, cut, 150], dtype=np.int32)
    h2 = np.concatenate([S0, fA.astype(np.float32)], axis=0)
    o2, f2 = oracle.kda_fwd(q, k, v, g, beta, cu2, h2)
    assert np.array_equal(o2[:cut], oA)
    assert np.array_equal(o[:cut], oA)
    # second half: bitwise equal to a standalone run from the same state
    oB, fB = oracle.kda_fwd(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], cuB,
                            fA.astype(np.float32))
    assert np.array_equal(o2[cut:], oB)
    assert np.array_equal(f2[1], fB[0])
    # and, up to the fp32 rounding of the handed-over state, the full run
    assert rel(oB, o[cut:]) < 1e-6 and rel(fB, fin) < 1e-6


def test_packing_order_and_neighbours_do_not_matter():
    rng = np.random.default_rng(18)
    lens = [33, 0, 70, 5]
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, lens, H=2, dk=8, dv=8)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0)
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        cus = np.array([0, b - a], dtype=np.int32)
        os_, fs = oracle.kda_fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], cus,
                                 S0[s:s + 1])
        assert np.array_equal(o[a:b], os_)
        assert np.array_equal(fin[s], fs[0])
    # empty sequence: final_state = initial_state, bitwise
    assert np.array_equal(fin[1], S0[1].astype(np.float64))


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(19)
    q, k, v1, g, beta, cu, S1 = rand_inputs(rng, [45, 20], H=2, dk=12, dv=10)
    v2 = rng.standard_normal(v1.shape).astype(np.float32)
    S2 = rng.standard_normal(S1.shape).astype(np.float32)
    a = 0.75
    o1, f1 = oracle.kda_fwd(q, k, v1, g, beta, cu, S1)
    o2, f2 = oracle.kda_fwd(q, k, v2, g, beta, cu, S2)
    vm = (a * v1.astype(np.float64) + v2).astype(np.float32)
    Sm = (a * S1.astype(np.float64) + S2).astype(np.float32)
    om, fm = oracle.kda_fwd(q, k, vm, g, beta, cu, Sm)
    # the fp32 rounding of the mixed inputs bounds the agreement
    assert rel(om, a * o1 + o2) < 1e-6
    assert rel(fm, a * f1 + f2) < 1e-6


@pytest.mark.parametrize("lens", [[130, 64, 210], [53, 14, 13, 33, 16, 8, 1, 77]])
def test_chunked_form_matches_token_form(lens):
    rng = np.random.default_rng(20)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, lens, H=2, dk=16, dv=12)
    g[:, :, :3] = -5.0                                # pinned lower bound
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0)
    oc, fc = oracle.chunked_fwd(q, k, v, g, beta, cu, S0, bt=64)
    assert rel(oc, o) < 1e-12
    assert rel(fc, fin) < 1e-12
    oc16, fc16 = oracle.chunked_fwd(q, k, v, g, beta, cu, S0, bt=16)
    assert rel(oc16, o) < 1e-12 and rel(fc16, fin) < 1e-12


def test_chunked_form_at_full_head_size():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [200], H=1, dk=128, dv=128)
    o, fin = oracle.kda_fwd(q, k, v, g, beta, cu, S0)
    oc, fc = oracle.chunked_fwd(q, k, v, g, beta, cu, S0)
    assert rel(oc, o) < 1e-12 and rel(fc, fin) < 1e-12


def test_chunk_table_matches_page_example():
    with open(os.path.join(GOLDEN, "chunk_table_70_130.json")) as f:
        gold = json.load(f)
    lens = gold["lengths"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = oracle.chunk_table(cu, bt=gold["chunk_size"])
    assert [[r["seq"], r["local"]] for r in rows] == gold["chunk_indices"]
    assert [r["aligned_start"] for r in rows] == gold["starts"]
    aligned = [((L + 63) // 64) * 64 for L in lens]
    assert aligned == gold["aligned_lengths"]
    assert list(np.concatenate([[0], np.cumsum(aligned)])) == gold["aligned_cu_seqlens"]
    assert [r["start_flag"] for r in rows] == [1, 0, 1, 0, 0]
    assert [r["end_flag"] for r in rows] == [0, 1, 0, 0, 1]
    assert [r["start"] for r in rows] == [0, 64, 70, 134, 198]
    assert [r["length"] for r in rows] == [64, 6, 64, 64, 2]


def test_chunk_table_empty_and_exact_multiples():
    cu = np.array([0, 0, 64, 64, 192, 193], dtype=np.int32)
    rows = oracle.chunk_table(cu)
    assert [r["seq"] for r in rows] == [1, 3, 3, 4]
    assert [r["length"] for r in rows] == [64, 64, 64, 1]
    assert [(r["start_flag"], r["end_flag"]) for r in rows] == [(1, 1), (1, 0), (0, 1), (1, 1)]


def test_strip_exponent_budget_reached_at_the_lower_bound():
    # All gates at the lower bound -5: the subblock-midpoint reference keeps
    # every factor within 8 steps * 5 = 40 nats, i.e. 57.7 bits < 126.
    g = np.full((64, 4), -5.0)
    worst = oracle.strip_exponents(g)
    assert worst == pytest.approx(40.0)
    assert worst / math.log(2.0) == pytest.approx(57.7, abs=0.05)
    assert worst / math.log(2.0) < 126
    rng = np.random.default_rng(22)
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((64, 128))))
    assert oracle.strip_exponents(g) < 40.0
    # a partial last chunk clamps the reference row and stays in budget
    assert oracle.strip_exponents(np.full((37, 2), -5.0)) <= 40.0


def test_error_metrics():
    a = np.array([1.0, 2.0, 2.0])
    b = np.array([1.0, 2.0, 3.0])
    assert oracle.max_abs_err(a, b) == 1.0
    assert oracle.rel_fro_err(a, b) == pytest.approx(1.0 / math.sqrt(14.0))


def test_prologue_sigmoid_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4 and 1/4, sigmoid(-x) = 1 - sigmoid(x)
    x = np.array([[0.0, np.log(3.0), -np.log(3.0)]])
    z = np.zeros((1, 3, 4))
    _, _, beta = oracle.prologue(z, z, x)
    assert np.allclose(beta, [[0.5, 0.75, 0.25]], rtol=0, atol=1e-15)
    r = np.random.default_rng(21).normal(size=(5, 7))
    _, _, b1 = oracle.prologue(np.zeros((5, 7, 2)), np.zeros((5, 7, 2)), r)
    _, _, b2 = oracle.prologue(np.zeros((5, 7, 2)), np.zeros((5, 7, 2)), -r)
    assert np.allclose(b1 + b2, 1.0, rtol=0, atol=1e-15)


def test_prologue_l2norm_closed_forms():
    rng = np.random.default_rng(22)
    q = rng.normal(size=(6, 3, 128)) * 3.0
    k = rng.normal(size=(6, 3, 128)) * 0.1
    b = np.zeros((6, 3))
    qn, kn, _ = oracle.prologue(q, k, b, qk_eps=0.0)
    # unit rows, each a positive multiple of its input
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(np.linalg.norm(kn, axis=-1), 1.0, rtol=0, atol=1e-14)
    cos = (qn * q).sum(-1) / np.linalg.norm(q, axis=-1)
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)
    # with eps: |x'|^2 = s / (s + eps), s = |x|^2
    eps = 1e-3
    _, ke, _ = oracle.prologue(q, k, b, qk_eps=eps)
    s2 = (k * k).sum(-1)
    assert np.allclose((ke * ke).sum(-1), s2 / (s2 + eps), rtol=1e-13, atol=0)
    # a zero row stays zero, also with eps = 0
    z = np.zeros((2, 1, 128))
    zq, _, _ = oracle.prologue(z, z, np.zeros((2, 1)), qk_eps=0.0)
    assert np.array_equal(zq, z)
    # without eps, q and k pass through
    qp, kp, _ = oracle.prologue(q, k, b)
    assert np.array_equal(qp, q) and np.array_equal(kp, k)


def test_gated_rmsnorm_closed_forms():
    rng = np.random.default_rng(23)
    x = rng.normal(size=(5, 3, 128)) * rng.uniform(0.1, 10, size=(5, 3, 1))
    w1, big = np.ones(128), np.full((5, 3, 128), 40.0)   # sigmoid(40) = 1 in fp64
    # eps = 0, unit weight, open gate: every row has mean square 1
    y = oracle.gated_rmsnorm(x, big, w1, 0.0)
    assert np.allclose((y * y).mean(-1), 1.0, rtol=0, atol=1e-13)
    # scale invariance and oddness at eps = 0
    assert np.allclose(oracle.gated_rmsnorm(3.5 * x, big, w1, 0.0), y, rtol=0, atol=1e-13)
    assert np.allclose(oracle.gated_rmsnorm(-x, big, w1, 0.0), -y, rtol=0, atol=1e-13)
    # with eps: mean(y^2) = ms / (ms + eps)
    ms = (x * x).mean(-1)
    ye = oracle.gated_rmsnorm(x, big, w1, 0.5)
    assert np.allclose((ye * ye).mean(-1), ms / (ms + 0.5), rtol=1e-13, atol=0)
    # a constant row c: y = w * c / sqrt(c^2 + eps) * act(z)
    c = np.full((1, 1, 128), -2.0)
    w = rng.uniform(-1, 1, size=128)
    z = np.zeros((1, 1, 128))
    yc = oracle.gated_rmsnorm(c, z, w, 1.0)
    assert np.allclose(yc[0, 0], w * (-2.0 / np.sqrt(5.0)) * 0.5, rtol=1e-14, atol=0)
    # SiLU: silu(0) = 0, silu(ln 3) = 0.75 ln 3, silu(-ln 3) = -0.25 ln 3
    assert np.array_equal(oracle.gated_rmsnorm(c, z, w, 1.0, act="silu"), np.zeros_like(c))
    zl = np.full((1, 1, 128), np.log(3.0))
    ys = oracle.gated_rmsnorm(c, zl, w1, 0.0, act="silu")
    assert np.allclose(ys, -0.75 * np.log(3.0), rtol=1e-14, atol=0)
    ys = oracle.gated_rmsnorm(c, -zl, w1, 0.0, act="silu")
    assert np.allclose(ys, 0.25 * np.log(3.0), rtol=1e-14, atol=0)
    # weights act per channel; a zero row stays zero with eps = 0
    e = np.zeros(128)
    e[5] = 2.0
    ye = oracle.gated_rmsnorm(x, big, e, 0.0)
    assert np.count_nonzero(ye[..., np.arange(128) != 5]) == 0
    assert np.allclose(ye[..., 5], 2.0 * y[..., 5], rtol=1e-14, atol=0)
    zr = oracle.gated_rmsnorm(np.zeros((2, 1, 128)), big[:2, :1], w1, 0.0)
    assert np.array_equal(zr, np.zeros((2, 1, 128)))


def test_norms_reduce_to_library_routines():
    # with an open gate (sigmoid = 1 in fp64) the gated RMSNorm is torch's
    # rms_norm; with eps = 0 the prologue's L2 norm is torch's normalize
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(24)
    x = rng.normal(size=(7, 3, 128)) * rng.uniform(0.05, 20, size=(7, 3, 1))
    w = rng.uniform(-2, 2, size=128)
    for eps in (0.0, 1e-6, 0.3):
        y = oracle.gated_rmsnorm(x, np.full_like(x, 40.0), w, eps)
        ref = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(w), eps=eps)
        assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12), eps
    qn, kn, _ = oracle.prologue(x, 3.0 * x, np.zeros((7, 3)), qk_eps=0.0)
    ref = F.normalize(torch.from_numpy(x), dim=-1, eps=0.0).numpy()
    assert np.allclose(qn, ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(kn, ref, rtol=1e-13, atol=1e-15)


def test_widen_matches_torch_bfloat16_conversion():
    # oracle.widen turns bf16 bit patterns into fp32.  Pinned against torch's
    # own bfloat16 -> float32 conversion over every one of the 65,536 bit
    # patterns, and against values fixed by the bf16 format itself (sign,
    # 8-bit exponent, 7-bit mantissa): 0x3F80 = 1, 0xC000 = -2, 0x3F81 =
    # 1 + 2^-7, 0x0001 = 2^-133 (smallest subnormal), 0x7F80 = +inf.
    import torch
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(bits)
    assert got.dtype == np.float32
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    fixed = oracle.widen(np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000], np.uint16))
    assert fixed[0] == 1.0 and fixed[1] == -2.0 and fixed[2] == 1.0 + 2.0 ** -7
    assert fixed[3] == 2.0 ** -133 and np.isposinf(fixed[4])
    assert fixed[5] == 0.0 and np.signbit(fixed[5])
    # float arrays pass through unchanged
    f = np.array([0.1, -3.5], np.float32)
    assert oracle.widen(f) is f


def test_bf16_bit_inputs_equal_their_float_values():
    # the GPU parity tests hand the oracle bf16 bit patterns: the run must
    # equal the run on the same values given as floats (bitwise)
    import torch
    rng = np.random.default_rng(25)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [70, 0, 33], H=2, dk=128, dv=128)

    def to_bits(x):
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy()

    (qb, qf), (kb, kf), (vb, vf) = to_bits(q), to_bits(k), to_bits(v)
    o1, f1 = oracle.kda_fwd(qb, kb, vb, g, beta, cu, S0)
    o2, f2 = oracle.kda_fwd(qf, kf, vf, g, beta, cu, S0)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_head_sampling_equals_columns_of_the_full_run():
    # kda_fwd(heads=...) is the reference of every sampled-head GPU parity
    # test: it must give exactly the matching head columns of the full run,
    # in the order asked for, with and without an initial state
    rng = np.random.default_rng(26)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [45, 0, 80, 3], H=6, dk=128, dv=128)
    for h0 in (S0, None):
        o, f = oracle.kda_fwd(q, k, v, g, beta, cu, h0, scale=0.9)
        for heads in ([4], [5, 0, 2], [1, 1]):
            os_, fs = oracle.kda_fwd(q, k, v, g, beta, cu, h0, scale=0.9, heads=heads)
            assert os_.shape == (q.shape[0], len(heads), 128)
            assert fs.shape == (len(cu) - 1, len(heads), 128, 128)
            assert np.array_equal(os_, o[:, heads]) and np.array_equal(fs, f[:, heads])
    # a head's result does not depend on the other heads' inputs
    q2 = q.copy()
    q2[:, 3] += 1.0
    o3, f3 = oracle.kda_fwd(q2, k, v, g, beta, cu, S0, heads=[0, 5])
    o4, f4 = oracle.kda_fwd(q, k, v, g, beta, cu, S0, heads=[0, 5])
    assert np.array_equal(o3, o4) and np.array_equal(f3, f4)
