"""End-to-end parity of kda_chunk_fwd against the fp64 oracle, on every
named workload and on edge cases, plus the varlen bit-exactness contract:
a sequence's outputs are bitwise the same alone or packed at any offset, in
any order; empty sequences copy the state; a NULL initial state equals
explicit zeros; results are deterministic run to run."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


@pytest.mark.parametrize("scale", [None, 1.0], ids=["scale_rsqrt128", "scale_1"])
def test_tiny(dev, scale):
    w = wl.tiny()
    log(f"[case] tiny scale={scale}")
    o, f = run_gpu(w, dev, scale=scale)
    o_ref, f_ref = run_oracle(w, scale=scale)
    parity(o, f, o_ref, f_ref, f"tiny scale={scale}")


EDGE = [1, 8, 15, 16, 17, 63, 64, 65, 130, 210]


@pytest.mark.parametrize("pinned", [0.0, 1.0], ids=["random_g", "g_at_lower_bound"])
def test_edge_lengths(dev, pinned):
    w = wl.small(EDGE, H=2, seed=41, pinned_fraction=pinned, scale=1.0)
    log(f"[case] edge lengths pinned={pinned}")
    o, f = run_gpu(w, dev)
    o_ref, f_ref = run_oracle(w)
    parity(o, f, o_ref, f_ref, f"edge pinned={pinned}")


def test_heads_1_8_and_32(dev):
    # H = 32 also gives 96 chains, where the recurrence splits each chain
    # over two workgroups instead of four
    for H in (1, 8, 32):
        w = wl.small([100, 64, 3], H=H, seed=42)
        log(f"[case] H={H}")
        o, f = run_gpu(w, dev)
        parity(o, f, *run_oracle(w), f"H={H}")


def test_sampled_lengths(dev):
    # the eight sampled sequence lengths of the KDA TPU report's correctness
    # section: short, sub-subblock, exact multiples of 16 and 64, and long
    w = wl.make_workload("sampled8", [53, 14, 13, 33, 16, 480, 512, 77], H=4, seed=45,
                         h0="normal")
    log("[case] sampled lengths")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), "sampled lengths")


def test_headline(dev):
    w = wl.headline()
    log("[case] headline 4x2048 H=16")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), "headline")


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_batch(dev, B):
    w = wl.batch(B)
    heads = [0, 7, 15]
    log(f"[case] batch B={B} (oracle on heads {heads})")
    o, f = run_gpu(w, dev)
    o_ref, f_ref = run_oracle(w, heads=heads)
    parity(o[:, heads], f[:, heads], o_ref, f_ref, f"batch{B}")


def test_sharegpt_like(dev):
    w = wl.sharegpt_like()
    heads = [3, 12]
    log(f"[case] sharegpt-like T={w.T} chunks={w.num_chunks()} (oracle on heads {heads})")
    o, f = run_gpu(w, dev)
    o_ref, f_ref = run_oracle(w, heads=heads)
    parity(o[:, heads], f[:, heads], o_ref, f_ref, "sharegpt_like")


def test_long_single_sequence(dev):
    w = wl.long_single()
    heads = [0, 47, 95]
    log(f"[case] long T=16384 H=96 (oracle on heads {heads})")
    o, f = run_gpu(w, dev)
    o_ref, f_ref = run_oracle(w, heads=heads)
    parity(o[:, heads], f[:, heads], o_ref, f_ref, "long")


def test_e2e_4x32k(dev):
    # the KDA TPU report's end-to-end varlen shape (correctness section):
    # 4 x 32,768 tokens, 512 chunks per chain, with a nonzero initial state
    w = wl.e2e_4x32k()
    heads = [2, 13]
    log(f"[case] e2e 4x32768 H=16 (oracle on heads {heads})")
    o, f = run_gpu(w, dev)
    o_ref, f_ref = run_oracle(w, heads=heads)
    parity(o[:, heads], f[:, heads], o_ref, f_ref, "e2e_4x32k")


@pytest.mark.parametrize("gmul", [0.0, 0.01], ids=["g_zero", "weak_decay"])
@pytest.mark.parametrize("shape", ["headline", "long"])
def test_weak_and_no_decay_full_size(dev, shape, gmul):
    # little or no decay at full length: the state carries the whole history
    # (16,384 tokens in one chain for the long shape), at scale 1 where the
    # max-abs bar bites; checked on sampled heads
    w = wl.by_name(shape)
    w.g = (w.g * np.float32(gmul)).astype(np.float32)
    heads = [0, 47, 95] if shape == "long" else [0, 9]
    log(f"[case] {shape} decay scaled by {gmul}, scale 1 (oracle on heads {heads})")
    o, f = run_gpu(w, dev, scale=1.0)
    o_ref, f_ref = run_oracle(w, scale=1.0, heads=heads)
    parity(o[:, heads], f[:, heads], o_ref, f_ref, f"{shape} g*{gmul} scale 1")


@pytest.mark.parametrize("N", [1024, 1100], ids=["N1024_table_in_intra", "N1100_table_kernel"])
def test_many_sequences(dev, N):
    # up to 1024 sequences the intra-chunk kernel builds the chunk table
    # itself; past that a separate table kernel does: both sides of the switch
    lens = list(np.random.default_rng(5).integers(0, 140, size=N))
    w = wl.make_workload(f"many_N{N}", lens, H=2, seed=44, h0="normal")
    log(f"[case] many sequences N={N} T={w.T} chunks={w.num_chunks()}")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), f"many N={N}")


# ---------------------------------------------------------------------------
# varlen bit-exactness
# ---------------------------------------------------------------------------
def _sub(w, order):
    """Repack a workload with its sequences in `order` (a permutation or a
    subset), as a new Workload with the same per-sequence data."""
    cu = w.cu_seqlens
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order]).astype(np.int64)
    lens = [int(cu[s + 1] - cu[s]) for s in order]
    ncu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    h0 = None if w.initial_state is None else np.ascontiguousarray(w.initial_state[list(order)])
    return wl.Workload(name=w.name + "_sub", seed=w.seed, q=w.q[idx], k=w.k[idx], v=w.v[idx],
                       g=w.g[idx], beta=w.beta[idx], initial_state=h0, cu_seqlens=ncu,
                       scale=w.scale)


def test_varlen_bit_exact(dev):
    w = wl.small([130, 0, 64, 17, 200, 1, 0, 95], H=3, seed=43)
    log("[case] varlen bit-exact")
    o, f = run_gpu(w, dev)
    cu = w.cu_seqlens
    # each sequence alone
    for s in range(w.N):
        ws = _sub(w, [s])
        os_, fs = run_gpu(ws, dev)
        assert np.array_equal(os_, o[cu[s]:cu[s + 1]]), s
        assert np.array_equal(fs[0], f[s]), s
    # permuted packing order
    perm = [4, 7, 0, 3, 1, 6, 2, 5]
    wp = _sub(w, perm)
    op, fp = run_gpu(wp, dev)
    for new, s in enumerate(perm):
        a, b = wp.cu_seqlens[new], wp.cu_seqlens[new + 1]
        assert np.array_equal(op[a:b], o[cu[s]:cu[s + 1]])
        assert np.array_equal(fp[new], f[s])
    # empty sequences: final = initial, bitwise
    for s in (1, 6):
        assert np.array_equal(f[s], w.initial_state[s].astype(np.float64))
    # run-to-run determinism
    o2, f2 = run_gpu(w, dev)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


@pytest.mark.parametrize("H", [8, 16, 32], ids=["one_wave_parts8", "two_waves_parts4",
                                                  "four_waves_parts2"])
def test_short_chains_in_each_launch_configuration(dev, H):
    # 4 sequences of 2, 1, 1 and 3 chunks: 32, 64 and 128 chains put the
    # recurrence in its one-, two- and four-compute-wave configurations (8, 4
    # and 2 workgroups per chain), where the copy waves' block copies and L2
    # touches run out after one to three chunks.  Against the oracle, and
    # bitwise against each sequence alone (H chains: the one-wave
    # configuration), since the per-column arithmetic does not depend on how
    # the value tiles are grouped.
    w = wl.small([100, 64, 3, 150], H=H, seed=46, h0="normal")
    log(f"[case] short chains H={H} ({4 * H} chains)")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), f"short chains H={H}")
    cu = w.cu_seqlens
    for s in range(w.N):
        os_, fs = run_gpu(_sub(w, [s]), dev)
        assert np.array_equal(os_, o[cu[s]:cu[s + 1]]), (H, s)
        assert np.array_equal(fs[0], f[s]), (H, s)


@pytest.mark.parametrize("bval", [0.0, 1.0], ids=["beta_0", "beta_1"])
def test_degenerate_beta(dev, bval):
    # beta = 0: L = 0, T = I, W = U = 0, so v_new = 0, the state only decays
    # and o reads the decayed initial state; beta = 1 on every token: the
    # strongest correction the delta rule applies.  Ragged lengths, a normal
    # initial state, g down to its lower bound.
    base = wl.small([130, 64, 17, 200], H=4, seed=47, h0="normal", pinned_fraction=0.5)
    beta = np.full_like(base.beta, bval)
    w = wl.Workload(name=base.name + f"_beta{bval:g}", seed=base.seed, q=base.q, k=base.k,
                    v=base.v, g=base.g, beta=beta, initial_state=base.initial_state,
                    cu_seqlens=base.cu_seqlens, scale=base.scale)
    log(f"[case] beta = {bval:g}")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), f"beta={bval:g}")


def test_null_initial_state_equals_zeros(dev):
    w = wl.small([100, 37], H=2, seed=44, h0="zeros")
    log("[case] NULL initial_state vs zeros")
    oz, fz = run_gpu(w, dev)
    on, fn = run_gpu(w, dev, with_h0=False)
    assert np.array_equal(oz, on) and np.array_equal(fz, fn)


def test_in_place_state_update(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([90, 64], H=2, seed=45)
    log("[case] final_state aliasing initial_state")
    o_ref, f_ref = run_gpu(w, dev)
    t = wl.to_torch(w, dev)
    st = t["initial_state"].clone()
    o, f = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                         initial_state=st, final_state=st, scale=w.scale)
    torch.cuda.synchronize()
    assert f.data_ptr() == st.data_ptr()
    assert np.array_equal(st.cpu().numpy().astype(np.float64), f_ref)
    assert np.array_equal(wl.bf16_tensor_to_f32(o).astype(np.float64), o_ref)


def test_split_equals_chain(dev):
    # running [A; B] equals running A, then B from A's final state (up to the
    # fp32 hand-over of the state, which the single call never rounds)
    w = wl.small([300], H=2, seed=46)
    log("[case] split = chain")
    o, f = run_gpu(w, dev)
    cut = 128                                  # a chunk boundary: same chunking
    wa = wl.Workload(name="a", seed=0, q=w.q[:cut], k=w.k[:cut], v=w.v[:cut], g=w.g[:cut],
                     beta=w.beta[:cut], initial_state=w.initial_state,
                     cu_seqlens=np.array([0, cut], np.int32), scale=w.scale)
    oa, fa = run_gpu(wa, dev)
    wb = wl.Workload(name="b", seed=0, q=w.q[cut:], k=w.k[cut:], v=w.v[cut:], g=w.g[cut:],
                     beta=w.beta[cut:], initial_state=fa.astype(np.float32),
                     cu_seqlens=np.array([0, 300 - cut], np.int32), scale=w.scale)
    ob, fb = run_gpu(wb, dev)
    assert np.array_equal(oa, o[:cut])
    assert np.array_equal(ob, o[cut:]) and np.array_equal(fb, f)


def test_intra_then_recurrence_equals_fwd(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([150, 64, 3, 0, 77], H=3, seed=47)
    log("[case] intra + recurrence == fwd (bitwise)")
    t = wl.to_torch(w, dev)
    o1, f1 = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                           initial_state=t["initial_state"], scale=w.scale)
    ws = kda.chunk_intra(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                         scale=w.scale)
    o2, f2 = kda.chunk_recurrence(ws, w.T, w.N, w.H, initial_state=t["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1, f2)


def test_workspace_contents_do_not_matter(dev):
    # The workspace is scratch: whatever it holds on entry (zeros, all ones,
    # random bytes, an earlier call's table and intermediates), the outputs
    # are bitwise those of a fresh workspace, and the flags word reports no
    # malformed input.  Full-size (4 x 2048 tokens x 16 heads, several units
    # per workgroup of the intra-chunk kernel).
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.headline()
    log("[case] workspace contents on entry")
    o_ref, f_ref = run_gpu(w, dev)
    parity(o_ref[:, [5]], f_ref[:, [5]], *run_oracle(w, heads=[5]), "headline head 5")
    t = wl.to_torch(w, dev)
    ws = kda.new_workspace(w.T, w.N, w.H, dev)
    gen = torch.Generator(device="cpu").manual_seed(5)
    fills = [("zeros", lambda: ws.zero_()),
             ("ones", lambda: ws.fill_(0xFF)),
             ("random", lambda: ws.copy_(torch.randint(0, 256, ws.shape, generator=gen,
                                                      dtype=torch.uint8).to(dev))),
             ("as left", lambda: None)]
    for name, fill in fills:
        fill()
        o, f = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                             initial_state=t["initial_state"], scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0, name
        assert np.array_equal(wl.bf16_tensor_to_f32(o).astype(np.float64), o_ref), name
        assert np.array_equal(f.cpu().numpy().astype(np.float64), f_ref), name


@pytest.mark.parametrize("gmul", [0.0, 0.01], ids=["g_zero", "weak_decay"])
def test_weak_and_no_decay(dev, gmul):
    # with little or no decay the state carries the whole history, the
    # hardest case for the bf16 rounding budget
    w = wl.small([700, 130, 64], H=2, seed=48, scale=1.0)
    w.g = (w.g * np.float32(gmul)).astype(np.float32)
    log(f"[case] decay scaled by {gmul}")
    o, f = run_gpu(w, dev)
    parity(o, f, *run_oracle(w), f"g*{gmul}")
