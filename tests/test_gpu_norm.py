"""kda_gated_rmsnorm (the gated RMSNorm after the operation) against the
fp64 oracle, alone on the same bf16 inputs and chained after the fused
forward."""

import numpy as np
import pytest

import oracle
from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, MAX_ABS, REL_FRO

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def _bf(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def _inputs(T, H, seed, pre=(8, 24)):
    """x and gate as bf16 bits inside wider rows [T, pre + H*128 + 8]:
    column slices at offsets pre[0] and pre[1] (multiples of 8)."""
    rng = np.random.default_rng(seed)
    W = max(pre) + H * 128 + 8
    xf = wl.f32_to_bf16_bits(rng.normal(size=(T, W)).astype(np.float32) * 2.0)
    zf = wl.f32_to_bf16_bits(rng.normal(size=(T, W)).astype(np.float32) * 3.0)
    w = rng.uniform(-2.0, 2.0, size=128).astype(np.float32)
    return xf, zf, w, pre


# The kernel alone, on the oracle's own bf16 inputs: fp32 arithmetic (about
# 1e-6 relative) and one bf16 rounding of y (at most half an ulp: 2^-8
# relative with 8 significant bits), so every element obeys
# |y - y_ref| <= (2^-8 + 1e-5) |y_ref| + 1e-5.
ELEM_REL, ELEM_ABS = 2.0 ** -8 + 1e-5, 1e-5


def _check(y, y_ref, label):
    d = np.abs(y - y_ref)
    err = float(d.max(initial=0.0)), oracle.rel_fro_err(y, y_ref)
    log(f"[parity] {label}: y_maxabs={err[0]:.3e} y_relF={err[1]:.3e}")
    assert np.all(np.isfinite(y))
    assert err[1] <= REL_FRO, (label, err)
    worst = float((d - ELEM_REL * np.abs(y_ref)).max(initial=0.0))
    assert worst <= ELEM_ABS, (label, worst)


@pytest.mark.parametrize("T,H", [(1, 1), (37, 3), (8192, 16)], ids=["1x1", "37x3", "8192x16"])
@pytest.mark.parametrize("act", ["sigmoid", "silu"])
@pytest.mark.parametrize("eps", [1e-6, 0.5], ids=["eps1e-6", "eps0.5"])
def test_gated_rmsnorm_matches_oracle(dev, T, H, act, eps):
    import torch
    import chunked_kda_prefill_amd as kda
    xf, zf, w, (px, pz) = _inputs(T, H, seed=400 + T + H)
    log(f"[case] gated_rmsnorm T={T} H={H} act={act} eps={eps}")
    X, Z = _bf(xf, dev), _bf(zf, dev)
    x = X[:, px:px + H * 128].view(T, H, 128)
    z = Z[:, pz:pz + H * 128].view(T, H, 128)
    y = kda.gated_rmsnorm(x, z, torch.from_numpy(w).to(dev), eps=eps, activation=act)
    torch.cuda.synchronize()
    y_ref = oracle.gated_rmsnorm(xf[:, px:px + H * 128].reshape(T, H, 128),
                                 zf[:, pz:pz + H * 128].reshape(T, H, 128), w, eps, act)
    _check(wl.bf16_tensor_to_f32(y).astype(np.float64), y_ref, f"norm {T}x{H} {act} {eps}")


def test_gated_rmsnorm_in_place_and_zero_rows(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    T, H = 50, 2
    xf, zf, w, _ = _inputs(T, H, seed=410)
    x = xf[:, :H * 128].reshape(T, H, 128).copy()
    x[7] = 0                                     # all-zero rows stay zero, eps = 0 included
    z = zf[:, :H * 128].reshape(T, H, 128)
    wt = torch.from_numpy(w).to(dev)
    log("[case] gated_rmsnorm in place, zero rows, eps 0")
    xt = _bf(x, dev)
    y = kda.gated_rmsnorm(xt, _bf(z, dev), wt, eps=0.0)
    y2 = kda.gated_rmsnorm(xt, _bf(z, dev), wt, eps=0.0, out=xt)
    torch.cuda.synchronize()
    assert y2.data_ptr() == xt.data_ptr()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    yf = wl.bf16_tensor_to_f32(y)
    assert np.all(yf[7] == 0)
    _check(yf.astype(np.float64), oracle.gated_rmsnorm(x, z, w, 0.0), "norm in place")


def test_gated_rmsnorm_after_fused_forward(dev):
    # the whole chain, fused prologue + forward + epilogue, each stage at its
    # own bar: o against the oracle's prologue and recurrence (the forward's
    # bar), and y against the oracle's epilogue of that o (the elementwise
    # bound).  A bar on y against the all-fp64 chain would measure o's mean
    # per-row relative error instead: normalisation gives every row the same
    # weight, where o's relF is dominated by its large rows.
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([0, 1, 63, 64, 65, 130, 200, 17], H=3, seed=75)
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 301)
    T, H = w.T, w.H
    _, zf, wn, (_, pz) = _inputs(T, H, seed=411)
    t = wl.to_torch(w, dev)
    log("[case] fused forward + gated_rmsnorm")
    o, _ = kda.chunk_fwd_fused(_bf(rq, dev), _bf(rk, dev), t["v"], t["g"],
                               _bf(bfull, dev)[:, pre:pre + H], t["cu_seqlens"],
                               initial_state=t["initial_state"], scale=1.0)
    z = _bf(zf, dev)[:, pz:pz + H * 128].view(T, H, 128)
    y = kda.gated_rmsnorm(o, z, torch.from_numpy(wn).to(dev), eps=1e-6)
    torch.cuda.synchronize()
    qn, kn, beta = oracle.prologue(rq, rk, bfull[:, pre:pre + H], qk_eps=1e-6)
    o_ref, _ = oracle.kda_fwd(qn, kn, w.v, w.g, beta, w.cu_seqlens, w.initial_state, scale=1.0)
    o_gpu = wl.bf16_tensor_to_f32(o).astype(np.float64)
    eo = oracle.max_abs_err(o_gpu, o_ref), oracle.rel_fro_err(o_gpu, o_ref)
    log(f"[parity] fused forward o: maxabs={eo[0]:.3e} relF={eo[1]:.3e}")
    assert eo[0] <= MAX_ABS and eo[1] <= REL_FRO, eo
    z_ref = zf[:, pz:pz + H * 128].reshape(T, H, 128)
    _check(wl.bf16_tensor_to_f32(y).astype(np.float64),
           oracle.gated_rmsnorm(o_gpu, z_ref, wn, 1e-6), "norm of the forward's o")
    # and the chain against the all-fp64 one, row by row.  With u = x / rms(x)
    # and D = diag(w * act(z)): y = D u, |u' - u| <= 2 |o' - o| / rms(o), and
    # the rounding of y adds at most 2^-8 max|D| per element, so
    # |y' - y| <= max|D| sqrt(128) (2 e_o + 2^-8), e_o = |o' - o| / |o|
    y_all = oracle.gated_rmsnorm(o_ref, z_ref, wn, 1e-6)
    sig = 1.0 / (1.0 + np.exp(-wl.bf16_bits_to_f32(z_ref).astype(np.float64)))
    dmax = np.abs(wn * sig).max(axis=-1)
    d = np.linalg.norm(wl.bf16_tensor_to_f32(y).astype(np.float64) - y_all, axis=-1)
    e_o = np.linalg.norm(o_gpu - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)
    bound = dmax * np.sqrt(128.0) * (2.0 * e_o + 2.0 ** -8) + 1e-5
    log(f"[parity] chain rows: max |y - y_ref| / bound = {(d / bound).max():.3f}, "
        f"max e_o = {e_o.max():.3e}")
    assert np.all(d <= bound)


def test_gated_rmsnorm_rejects_bad_views(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    x = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device=dev)
    w = torch.ones(128, dtype=torch.float32, device=dev)
    wide = torch.zeros((4, 2 * 128 + 12), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        kda.gated_rmsnorm(x, x.transpose(0, 1).contiguous().transpose(0, 1), w)
    with pytest.raises(ValueError):
        kda.gated_rmsnorm(x, x, w, activation="relu")
    with pytest.raises(kda.KDAError):            # slice at an offset of 4 elements: misaligned
        kda.gated_rmsnorm(x, wide[:, 4:4 + 256].view(4, 2, 128), w)


@pytest.mark.parametrize("users,tokens,H", [(16, 1, 12), (16, 4, 12), (5, 9, 3)],
                         ids=["decode16x1_h12", "verify16x4_h12", "5x9_h3"])
@pytest.mark.parametrize("act", ["sigmoid", "silu"])
def test_decode_step_fused(dev, users, tokens, H, act):
    # the whole decode step in one kernel: o and the state bitwise equal to
    # kda_decode_fwd_fused (the same per-column arithmetic and reduction
    # order), y against the oracle's chain row by row
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.decode_step(users, tokens, H)
    T = w.T
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 302)
    _, zf, wn, (_, pz) = _inputs(T, H, seed=412)
    t = wl.to_torch(w, dev)
    q, k = _bf(rq, dev), _bf(rk, dev)
    b = _bf(bfull, dev)[:, pre:pre + H]
    z = _bf(zf, dev)[:, pz:pz + H * 128].view(T, H, 128)
    wt = torch.from_numpy(wn).to(dev)
    log(f"[case] decode_step_fused {users}x{tokens} H={H} act={act}")
    o, y, f = kda.decode_step_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"], z, wt,
                                    initial_state=t["initial_state"], scale=1.0, activation=act)
    o2, f2 = kda.decode_fwd_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"],
                                  initial_state=t["initial_state"], scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f, f2)
    qn, kn, beta = oracle.prologue(rq, rk, bfull[:, pre:pre + H], qk_eps=1e-6)
    o_ref, f_ref = oracle.kda_fwd(qn, kn, w.v, w.g, beta, w.cu_seqlens, w.initial_state,
                                  scale=1.0)
    o_gpu = wl.bf16_tensor_to_f32(o).astype(np.float64)
    eo = oracle.max_abs_err(o_gpu, o_ref), oracle.rel_fro_err(o_gpu, o_ref)
    assert eo[0] <= MAX_ABS and eo[1] <= REL_FRO, eo
    z_ref = zf[:, pz:pz + H * 128].reshape(T, H, 128)
    y_all = oracle.gated_rmsnorm(o_ref, z_ref, wn, 1e-6, act)
    zz = wl.bf16_bits_to_f32(z_ref).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-zz))
    dmax = np.abs(wn * (sig if act == "sigmoid" else zz * sig)).max(axis=-1)
    d = np.linalg.norm(wl.bf16_tensor_to_f32(y).astype(np.float64) - y_all, axis=-1)
    # the kernel normalises o's fp32 row; the bf16 o read back is within
    # 2^-8 of it per row, so e_o of the fp32 row <= e_o(bf16) + 2^-8
    e_o = np.linalg.norm(o_gpu - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)
    bound = dmax * np.sqrt(128.0) * (2.0 * (e_o + 2.0 ** -8) + 2.0 ** -8) + 1e-5
    log(f"[parity] decode step y rows: max |y - y_ref| / bound = {(d / bound).max():.3f}, "
        f"y relF {oracle.rel_fro_err(wl.bf16_tensor_to_f32(y).astype(np.float64), y_all):.3e}")
    assert np.all(np.isfinite(d)) and np.all(d <= bound)


def test_decode_step_fused_varlen_empty(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([0, 1, 2, 0, 3, 5, 8, 4], H=3, seed=76)
    T, H = w.T, w.H
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 303)
    _, zf, wn, (_, pz) = _inputs(T, H, seed=413)
    t = wl.to_torch(w, dev)
    q, k, b = _bf(rq, dev), _bf(rk, dev), _bf(bfull, dev)[:, pre:pre + H]
    z = _bf(zf, dev)[:, pz:pz + H * 128].view(T, H, 128)
    log("[case] decode_step_fused varlen with empty sequences")
    o, y, f = kda.decode_step_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"], z,
                                    torch.from_numpy(wn).to(dev),
                                    initial_state=t["initial_state"])
    o2, f2 = kda.decode_fwd_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"],
                                  initial_state=t["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(f, f2)
    ff = f.cpu().numpy()
    for s in (0, 3):
        assert np.array_equal(ff[s], w.initial_state[s])
    assert np.all(np.isfinite(wl.bf16_tensor_to_f32(y)))


def test_decode_step_fused_empty_batch_and_no_norm(dev):
    # T = 0: the states pass through; qk_eps None: q and k as given
    import torch
    import chunked_kda_prefill_amd as kda
    H = 2
    e = torch.zeros((0, H, 128), dtype=torch.bfloat16, device=dev)
    eg = torch.zeros((0, H, 128), dtype=torch.float32, device=dev)
    eb = torch.zeros((0, H), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    h0 = torch.randn((2, H, 128, 128), device=dev)
    wt = torch.ones(128, dtype=torch.float32, device=dev)
    log("[case] decode_step_fused T=0")
    o, y, f = kda.decode_step_fused(e, e, e, eg, eb, cu, e, wt, initial_state=h0)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and y.shape[0] == 0 and torch.equal(f, h0)
    w = wl.decode_step(8, 2, 2)
    T = w.T
    _, zf, wn, (_, pz) = _inputs(T, 2, seed=414)
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 304)
    t = wl.to_torch(w, dev)
    b = _bf(bfull, dev)[:, pre:pre + 2]
    z = _bf(zf, dev)[:, pz:pz + 256].view(T, 2, 128)
    log("[case] decode_step_fused qk_eps=None")
    o, y, f = kda.decode_step_fused(t["q"], t["k"], t["v"], t["g"], b, t["cu_seqlens"], z,
                                    torch.from_numpy(wn).to(dev),
                                    initial_state=t["initial_state"], qk_eps=None)
    o2, f2 = kda.decode_fwd_fused(t["q"], t["k"], t["v"], t["g"], b, t["cu_seqlens"],
                                  initial_state=t["initial_state"], qk_eps=None)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(f, f2)
