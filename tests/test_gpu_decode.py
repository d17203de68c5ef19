"""kda_decode_fwd (token-serial decode / speculative-verification step)
against the fp64 oracle, plus its state contracts."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def run_decode(w, dev, scale=None, with_h0=True, **kw):
    import torch
    import chunked_kda_prefill_amd as kda
    t = wl.to_torch(w, dev)
    o, f = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                          initial_state=t["initial_state"] if with_h0 else None,
                          scale=w.scale if scale is None else scale, **kw)
    torch.cuda.synchronize()
    return wl.bf16_tensor_to_f32(o).astype(np.float64), f.cpu().numpy().astype(np.float64)


# the MI355X post's shapes: 16 users, 1 token or a 4-token window, 96 heads
# over 8 GPUs = 12 per GPU; and a larger batch at 16 heads
@pytest.mark.parametrize("users,tokens,H", [(16, 1, 12), (16, 4, 12), (64, 1, 16), (3, 16, 2)],
                         ids=["decode16x1_h12", "verify16x4_h12", "decode64x1_h16", "3x16_h2"])
@pytest.mark.parametrize("scale", [None, 1.0], ids=["scale_rsqrt128", "scale_1"])
def test_decode_matches_oracle(dev, users, tokens, H, scale):
    w = wl.decode_step(users, tokens, H)
    log(f"[case] decode {users}x{tokens} H={H} scale={scale}")
    o, f = run_decode(w, dev, scale=scale)
    parity(o, f, *run_oracle(w, scale=scale), f"decode {users}x{tokens} H={H} scale={scale}")


def test_decode_varlen_and_empty_sequences(dev):
    # lengths 0..8 mixed, explicit state: empty sequences return their state
    w = wl.small([0, 1, 2, 0, 3, 5, 8, 4], H=3, seed=61)
    log("[case] decode varlen with empty sequences")
    o, f = run_decode(w, dev)
    parity(o, f, *run_oracle(w), "decode varlen")
    for s in (0, 3):
        assert np.array_equal(f[s], w.initial_state[s].astype(np.float64))


def test_decode_null_state_and_in_place_update(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([1, 4, 2], H=2, seed=62, h0="zeros")
    log("[case] decode NULL state == zeros; in-place update")
    o0, f0 = run_decode(w, dev, with_h0=False)
    o1, f1 = run_decode(w, dev)
    assert np.array_equal(o0, o1) and np.array_equal(f0, f1)
    w2 = wl.small([1, 4, 2], H=2, seed=63)
    t = wl.to_torch(w2, dev)
    st = t["initial_state"].clone()
    o2, f2 = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                            initial_state=st, final_state=st, scale=w2.scale)
    o3, f3 = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                            initial_state=t["initial_state"], scale=w2.scale)
    torch.cuda.synchronize()
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(f2, f3) and torch.equal(o2.view(torch.int16), o3.view(torch.int16))


def test_decode_steps_chain_bitwise(dev):
    # a 4-token window equals four 1-token steps chained through the state:
    # the state stays fp32 in both, so the chain is exact
    import torch
    import chunked_kda_prefill_amd as kda
    users, H = 8, 4
    w = wl.decode_step(users, 4, H)
    log("[case] decode window == chained single steps")
    t = wl.to_torch(w, dev)
    o_win, f_win = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                  initial_state=t["initial_state"], scale=w.scale)
    st = t["initial_state"].clone()
    cu1 = torch.arange(users + 1, dtype=torch.int32, device=dev)
    outs = []
    for j in range(4):
        idx = torch.arange(users, device=dev) * 4 + j
        o_j, st = kda.decode_fwd(t["q"][idx].contiguous(), t["k"][idx].contiguous(),
                                 t["v"][idx].contiguous(), t["g"][idx].contiguous(),
                                 t["beta"][idx].contiguous(), cu1, initial_state=st,
                                 scale=w.scale)
        outs.append(o_j)
    torch.cuda.synchronize()
    o_chain = torch.stack(outs, dim=1).reshape(users * 4, H, 128)
    assert torch.equal(o_chain.view(torch.int16), o_win.view(torch.int16))
    assert torch.equal(st, f_win)


def test_decode_agrees_with_chunked_prefill(dev):
    # the two entry points compute the same function (rounding apart)
    import torch
    import chunked_kda_prefill_amd as kda
    from oracle import max_abs_err, rel_fro_err
    w = wl.small([5, 64, 70, 1], H=2, seed=64)
    log("[case] decode vs chunked prefill")
    t = wl.to_torch(w, dev)
    od, fd = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                            initial_state=t["initial_state"], scale=1.0)
    oc, fc = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                           initial_state=t["initial_state"], scale=1.0)
    torch.cuda.synchronize()
    a = wl.bf16_tensor_to_f32(od).astype(np.float64)
    b = wl.bf16_tensor_to_f32(oc).astype(np.float64)
    assert max_abs_err(a, b) <= 2e-2 and rel_fro_err(a, b) <= 5e-3
    fa, fb = fd.cpu().numpy().astype(np.float64), fc.cpu().numpy().astype(np.float64)
    assert max_abs_err(fa, fb) <= 2e-2 and rel_fro_err(fa, fb) <= 5e-3
