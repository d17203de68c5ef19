"""The entry points inside a captured HIP graph: they allocate nothing,
record no memset and never synchronise, so a capture of one call replays
to the eager result, bitwise.  Each graph is replayed several times, with
eager work (overwriting the outputs) and synchronisations between replays."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def _bf(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def _capture_and_replay(call, outs, eager, label):
    """call(): launches into the preallocated `outs`; eager: their expected
    contents.  Warm up on a side stream, capture, then replay 4 times."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for o in outs:                       # eager work between replays
            o.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e), \
                (label, rep)
    log(f"[graph] {label}: 4 replays bitwise equal to eager")


def test_chunk_fwd_in_graph(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([130, 64, 210, 0, 17], H=4, seed=90, h0="normal")
    t = wl.to_torch(w, dev)
    ws = kda.new_workspace(w.T, w.N, w.H, dev)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"])
    o_e, f_e = kda.chunk_fwd(*args, initial_state=t["initial_state"], scale=w.scale,
                             workspace=ws)
    torch.cuda.synchronize()
    o = torch.empty_like(o_e)
    f = torch.empty_like(f_e)
    call = lambda: kda.chunk_fwd(*args, initial_state=t["initial_state"], scale=w.scale,
                                 workspace=ws, o=o, final_state=f)
    _capture_and_replay(call, [o, f], [o_e, f_e], "chunk_fwd")


def test_fused_paths_in_graph(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([130, 64, 3], H=2, seed=91, h0="normal")
    rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 305)
    t = wl.to_torch(w, dev)
    q, k, b = _bf(rq, dev), _bf(rk, dev), _bf(bfull, dev)[:, pre:pre + w.H]
    ws = kda.new_workspace(w.T, w.N, w.H, dev)
    o_e, f_e = kda.chunk_fwd_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"],
                                   initial_state=t["initial_state"], workspace=ws)
    torch.cuda.synchronize()
    o, f = torch.empty_like(o_e), torch.empty_like(f_e)
    _capture_and_replay(
        lambda: kda.chunk_fwd_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"],
                                    initial_state=t["initial_state"], workspace=ws, o=o,
                                    final_state=f),
        [o, f], [o_e, f_e], "chunk_fwd_fused")

    d = wl.decode_step(16, 1, 12)
    rq, rk, bfull, pre = wl.raw_prologue_inputs(d, 306)
    t = wl.to_torch(d, dev)
    q, k, b = _bf(rq, dev), _bf(rk, dev), _bf(bfull, dev)[:, pre:pre + d.H]
    z = torch.randn((d.T, d.H, 128), device=dev).to(torch.bfloat16)
    nw = torch.rand(128, device=dev)
    o_e, y_e, f_e = kda.decode_step_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"], z, nw,
                                          initial_state=t["initial_state"])
    torch.cuda.synchronize()
    o, y, f = torch.empty_like(o_e), torch.empty_like(y_e), torch.empty_like(f_e)
    _capture_and_replay(
        lambda: kda.decode_step_fused(q, k, t["v"], t["g"], b, t["cu_seqlens"], z, nw,
                                      initial_state=t["initial_state"], o=o, y=y,
                                      final_state=f),
        [o, y, f], [o_e, y_e, f_e], "decode_step_fused")
