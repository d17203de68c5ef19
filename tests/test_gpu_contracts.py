"""Output contracts of the forward entry points on the GPU: a NULL
final_state (the state is not written, o is unchanged), an empty batch
(T = 0), and the speculative-verification flow of the MI355X serving post
(section 1.2): a verification pass over each user's window keeps no state,
then a replay over the accepted prefixes commits it."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


@pytest.mark.parametrize("entry", ["chunk_fwd", "decode_fwd"])
def test_null_final_state(dev, entry):
    # final_state NULL: nothing is written there, and o is bitwise the o of
    # the call that also writes the state
    import torch
    import chunked_kda_prefill_amd as kda
    lens = [130, 0, 64, 17] if entry == "chunk_fwd" else [1, 4, 0, 3]
    w = wl.small(lens, H=3, seed=71)
    log(f"[case] {entry} with final_state NULL")
    t = wl.to_torch(w, dev)
    fn = getattr(kda, entry)
    o1, f1 = fn(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                initial_state=t["initial_state"], scale=w.scale)
    o2, f2 = fn(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                initial_state=t["initial_state"], scale=w.scale, output_final_state=False)
    torch.cuda.synchronize()
    assert f2 is None
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    parity(wl.bf16_tensor_to_f32(o2).astype(np.float64), f1.cpu().numpy().astype(np.float64),
           *run_oracle(w), f"{entry} NULL final_state")


@pytest.mark.parametrize("entry", ["chunk_fwd", "decode_fwd"])
def test_empty_batch(dev, entry):
    # T = 0 with three empty sequences: no rows of o; each final state is its
    # initial state bitwise (or zeros without one)
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([0, 0, 0], H=2, seed=72)
    log(f"[case] {entry} with T = 0")
    t = wl.to_torch(w, dev)
    fn = getattr(kda, entry)
    o, f = fn(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
              initial_state=t["initial_state"], scale=w.scale)
    o0, f0 = fn(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], scale=w.scale)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and o0.shape == (0, 2, 128)
    assert torch.equal(f, t["initial_state"])
    assert torch.count_nonzero(f0).item() == 0


def test_verify_then_replay_commits_the_accepted_prefix(dev):
    # Verification: every user's 4-token draft window runs from its cached
    # state with final_state NULL (no per-position state is saved).  The
    # window's outputs are those of the same tokens run one step at a time.
    # Replay: the accepted prefix of each window (0 to 4 tokens) runs again
    # from the same cached state and writes the new state in place.  The
    # committed state equals the state after that many single decode steps,
    # bitwise, and the replayed outputs equal the verification outputs of
    # the accepted tokens, bitwise.
    import torch
    import chunked_kda_prefill_amd as kda
    users, win, H = 16, 4, 12
    w = wl.decode_step(users, win, H)
    log("[case] verify -> replay")
    t = wl.to_torch(w, dev)
    cache = t["initial_state"].clone()
    o_ver, none = kda.decode_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                 initial_state=cache, scale=w.scale, output_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(cache, t["initial_state"])           # the cache is untouched
    # verification outputs against the oracle over the whole window
    from oracle import max_abs_err, rel_fro_err
    o_ref, _ = run_oracle(w)
    ov = wl.bf16_tensor_to_f32(o_ver).astype(np.float64)
    log(f"[parity] verify window: o_maxabs={max_abs_err(ov, o_ref):.3e} "
        f"o_relF={rel_fro_err(ov, o_ref):.3e}")
    assert max_abs_err(ov, o_ref) <= 2e-2 and rel_fro_err(ov, o_ref) <= 5e-3

    accepted = np.random.default_rng(73).integers(0, win + 1, size=users)
    accepted[0], accepted[1] = 0, win                         # both extremes present
    rows = np.concatenate([np.arange(u * win, u * win + a) for u, a in enumerate(accepted)])
    idx = torch.from_numpy(rows.astype(np.int64)).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(accepted)]).astype(np.int32)).to(dev)
    sel = {k: t[k][idx].contiguous() for k in ("q", "k", "v", "g", "beta")}
    o_rep, committed = kda.decode_fwd(sel["q"], sel["k"], sel["v"], sel["g"], sel["beta"], cu,
                                      initial_state=cache, final_state=cache, scale=w.scale)
    torch.cuda.synchronize()
    assert committed.data_ptr() == cache.data_ptr()
    assert torch.equal(o_rep.view(torch.int16), o_ver[idx].view(torch.int16))

    # the same commit by single decode steps: user u takes accepted[u] steps
    st = t["initial_state"].clone()
    for j in range(win):
        active = [u for u in range(users) if accepted[u] > j]
        lens = np.array([1 if accepted[u] > j else 0 for u in range(users)])
        r = torch.tensor([u * win + j for u in active], dtype=torch.int64, device=dev)
        cu1 = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
        _, st = kda.decode_fwd(t["q"][r].contiguous(), t["k"][r].contiguous(),
                               t["v"][r].contiguous(), t["g"][r].contiguous(),
                               t["beta"][r].contiguous(), cu1, initial_state=st,
                               final_state=st, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(cache, st)
    # and against the oracle run over the accepted prefixes only
    wa = wl.Workload(name="accepted", seed=0, q=w.q[rows], k=w.k[rows], v=w.v[rows],
                     g=w.g[rows], beta=w.beta[rows], initial_state=w.initial_state,
                     cu_seqlens=cu.cpu().numpy(), scale=w.scale)
    parity(wl.bf16_tensor_to_f32(o_rep).astype(np.float64),
           cache.cpu().numpy().astype(np.float64), *run_oracle(wa), "replay commit")
