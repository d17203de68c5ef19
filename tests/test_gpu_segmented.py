"""kda_chunk_fwd_segmented (chunk-parallel state passing) against the fp64
oracle: each chain cut into `segments` runs, segment maps composed as
h' = M h + b.  Cases: the batch-1 shape at several segment counts, varlen
chains shorter than the segment count (empty segments), the long shape,
weak decay at scale 1, segments = 1 against kda_chunk_fwd (bitwise), and a
sequence's bits alone and packed with others at the same segment count."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def run_seg(w, dev, segments, scale=None, **kw):
    import torch
    import chunked_kda_prefill_amd as kda
    t = wl.to_torch(w, dev)
    o, f = kda.chunk_fwd_segmented(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                   segments, initial_state=t["initial_state"],
                                   scale=w.scale if scale is None else scale, **kw)
    torch.cuda.synchronize()
    return wl.bf16_tensor_to_f32(o).astype(np.float64), (
        None if f is None else f.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("segments", [2, 4, 8, 32])
def test_batch1_segments(dev, segments):
    w = wl.batch(1)
    heads = [0, 15]
    log(f"[case] batch 1 with {segments} segments (oracle on heads {heads})")
    o, f = run_seg(w, dev, segments)
    parity(o[:, heads], f[:, heads], *run_oracle(w, heads=heads), f"batch1 segments={segments}")


@pytest.mark.parametrize("segments", [3, 8])
def test_varlen_short_chains(dev, segments):
    # chains of 0, 1, 2, 3 and 33 chunks: segments with no chunks compose as
    # the identity
    w = wl.small([130, 0, 64, 17, 2048, 1, 700, 150], H=3, seed=91)
    log(f"[case] varlen with {segments} segments")
    o, f = run_seg(w, dev, segments)
    parity(o, f, *run_oracle(w), f"varlen segments={segments}")


def test_long_shape_segments(dev):
    w = wl.long_single()
    heads = [0, 47, 95]
    log(f"[case] long with 4 segments (oracle on heads {heads})")
    o, f = run_seg(w, dev, 4)
    parity(o[:, heads], f[:, heads], *run_oracle(w, heads=heads), "long segments=4")


@pytest.mark.parametrize("gmul", [0.0, 0.01], ids=["g_zero", "weak_decay"])
def test_weak_decay_segments(dev, gmul):
    # little decay: the maps M stay far from zero, and every composed entry
    # state carries the whole history
    w = wl.batch(1)
    w.g = (w.g * np.float32(gmul)).astype(np.float32)
    heads = [3, 11]
    log(f"[case] batch 1, decay x {gmul}, scale 1, 8 segments")
    o, f = run_seg(w, dev, 8, scale=1.0)
    parity(o[:, heads], f[:, heads], *run_oracle(w, scale=1.0, heads=heads),
           f"batch1 g*{gmul} segments=8")


def test_one_segment_is_chunk_fwd(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([300, 64, 5], H=2, seed=92)
    log("[case] segments = 1 is kda_chunk_fwd")
    t = wl.to_torch(w, dev)
    o1, f1 = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                           initial_state=t["initial_state"], scale=w.scale)
    o2, f2 = kda.chunk_fwd_segmented(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                     t["cu_seqlens"], 1, initial_state=t["initial_state"],
                                     scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)


def test_segments_bitwise_alone_and_packed(dev):
    # the segment length depends on the chain's own chunk count: a sequence's
    # results are the same bits alone or packed with others
    w = wl.small([900, 0, 64, 333, 1500], H=2, seed=93)
    log("[case] segments: alone vs packed")
    o, f = run_seg(w, dev, 4)
    cu = w.cu_seqlens
    for s in range(w.N):
        a, b = int(cu[s]), int(cu[s + 1])
        ws = wl.Workload(name="one", seed=0, q=w.q[a:b], k=w.k[a:b], v=w.v[a:b], g=w.g[a:b],
                         beta=w.beta[a:b], initial_state=w.initial_state[s:s + 1],
                         cu_seqlens=np.array([0, b - a], np.int32), scale=w.scale)
        o1, f1 = run_seg(ws, dev, 4)
        assert np.array_equal(o1, o[a:b]), s
        assert np.array_equal(f1[0], f[s]), s
    # without a final state
    o2, f2 = run_seg(w, dev, 4, output_final_state=False)
    assert f2 is None and np.array_equal(o2, o)
