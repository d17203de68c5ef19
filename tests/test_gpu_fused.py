"""kda_chunk_fwd_fused and kda_decode_fwd_fused (beta from bf16 logits, q/k
L2-normalised in the kernel) against the fp64 oracle fed the fp64 prologue."""

import numpy as np
import pytest

import oracle
from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def _bf(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def run_fused(w, dev, qk_eps=1e-6, raw=True, decode=False, heads=None, seed=300):
    """Runs the fused entry point on ``w``'s v, g, state and lengths, with raw
    q, k and strided logits (or, raw=False, ``w``'s own q, k); returns the GPU
    (o, final) and the oracle's, the oracle restricted to ``heads``."""
    import torch
    import chunked_kda_prefill_amd as kda
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, seed)
    q, k = (rq, rk) if raw else (w.q, w.k)
    H = w.H
    t = wl.to_torch(w, dev)
    b = _bf(bfull, dev)[:, pre:pre + H]
    assert b.stride(0) == bfull.shape[1] and not b.is_contiguous() or w.T <= 1
    fn = kda.decode_fwd_fused if decode else kda.chunk_fwd_fused
    o, f = fn(_bf(q, dev), _bf(k, dev), t["v"], t["g"], b, t["cu_seqlens"],
              initial_state=t["initial_state"], scale=w.scale, qk_eps=qk_eps)
    torch.cuda.synchronize()
    o = wl.bf16_tensor_to_f32(o).astype(np.float64)
    f = f.cpu().numpy().astype(np.float64)
    qn, kn, beta = oracle.prologue(q, k, bfull[:, pre:pre + H], qk_eps=qk_eps)
    o_ref, f_ref = oracle.kda_fwd(qn, kn, w.v, w.g, beta, w.cu_seqlens, w.initial_state,
                                  scale=w.scale, heads=heads)
    if heads is not None:
        o, f = o[:, heads], f[:, heads]
    return o, f, o_ref, f_ref


# lengths span several chunks, partial chunks and empty sequences
LENGTHS = [0, 1, 63, 64, 65, 130, 200, 17]


@pytest.mark.parametrize("qk_eps", [1e-6, 64.0], ids=["eps1e-6", "eps64"])
def test_chunk_fused_matches_oracle(dev, qk_eps):
    # eps = 64 against rows with sum x^2 near 128 (q) and 2048 (k): the eps
    # term moves the result far beyond the tolerance, so its placement is pinned
    w = wl.small(LENGTHS, H=3, seed=71)
    log(f"[case] chunk_fwd_fused varlen qk_eps={qk_eps}")
    parity(*run_fused(w, dev, qk_eps=qk_eps), f"chunk fused eps={qk_eps}")


def test_chunk_fused_without_norm(dev):
    # qk_eps None: q and k pass through, only beta comes from the logits
    w = wl.small(LENGTHS, H=2, seed=72)
    log("[case] chunk_fwd_fused qk_eps=None")
    parity(*run_fused(w, dev, qk_eps=None, raw=False), "chunk fused no norm")


def test_chunk_fused_headline_sampled_heads(dev):
    # 4 x 2048 tokens, 16 heads, in the launch configuration the bench times;
    # the oracle runs three of the heads (heads are independent)
    w = wl.headline()
    log("[case] chunk_fwd_fused headline, heads 0 7 15")
    parity(*run_fused(w, dev, heads=[0, 7, 15]), "chunk fused headline")


@pytest.mark.parametrize("users,tokens,H", [(16, 1, 12), (16, 4, 12), (5, 9, 3)],
                         ids=["decode16x1_h12", "verify16x4_h12", "5x9_h3"])
@pytest.mark.parametrize("qk_eps", [1e-6, 64.0, None], ids=["eps1e-6", "eps64", "nonorm"])
def test_decode_fused_matches_oracle(dev, users, tokens, H, qk_eps):
    w = wl.decode_step(users, tokens, H)
    log(f"[case] decode_fwd_fused {users}x{tokens} H={H} qk_eps={qk_eps}")
    parity(*run_fused(w, dev, qk_eps=qk_eps, raw=qk_eps is not None, decode=True),
           f"decode fused {users}x{tokens} eps={qk_eps}")


def test_decode_fused_varlen_empty(dev):
    w = wl.small([0, 1, 2, 0, 3, 5, 8, 4], H=3, seed=73)
    log("[case] decode_fwd_fused varlen with empty sequences")
    o, f, o_ref, f_ref = run_fused(w, dev, decode=True)
    parity(o, f, o_ref, f_ref, "decode fused varlen")
    for s in (0, 3):
        assert np.array_equal(f[s], w.initial_state[s].astype(np.float64))


def test_fused_rejects_bad_logits(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([5, 3], H=2, seed=74)
    t = wl.to_torch(w, dev)
    args = (t["q"], t["k"], t["v"], t["g"])
    good = torch.zeros((w.T, 2), dtype=torch.bfloat16, device=dev)
    for bad in (good.float(), good.t().contiguous().t(), torch.zeros((w.T, 3), dtype=torch.bfloat16,
                                                                   device=dev)):
        with pytest.raises(ValueError):
            kda.chunk_fwd_fused(*args, bad, t["cu_seqlens"])
        with pytest.raises(ValueError):
            kda.decode_fwd_fused(*args, bad, t["cu_seqlens"])


def test_chunk_fused_many_sequences(dev):
    # past 1,024 sequences a separate kernel builds the chunk table: the
    # fused prologue on that side of the switch too
    lens = list(np.random.default_rng(6).integers(0, 140, size=1100))
    w = wl.make_workload("fused_many_N1100", lens, H=2, seed=77, h0="normal")
    log(f"[case] chunk_fwd_fused N=1100 T={w.T}")
    parity(*run_fused(w, dev), "chunk fused N=1100")
