"""kda_chunk_fwd_noalloc on the GPU: the entry point that allocates nothing
(its workspace is the library's own per-GPU array) gives bitwise the
results of kda_chunk_fwd, on two calls in a row (the second smaller, so
the array holds the first call's contents on entry), and is within the
parity bar of the fp64 oracle."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log, parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def test_noalloc_equals_chunk_fwd_on_two_calls(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    for w, heads in ((wl.headline(), [3]), (wl.small([130, 0, 64, 17, 200], H=3, seed=81), None)):
        log(f"[case] noalloc {w.name} T={w.T} N={w.N} H={w.H}")
        t = wl.to_torch(w, dev)
        o_ref, f_ref = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                     initial_state=t["initial_state"], scale=w.scale)
        o = torch.full_like(o_ref, float("nan"))
        f = torch.full_like(f_ref, float("nan"))
        kda.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], o,
                              final_state=f, initial_state=t["initial_state"], scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(f, f_ref)
        og = wl.bf16_tensor_to_f32(o).astype(np.float64)
        fg = f.cpu().numpy().astype(np.float64)
        if heads is None:
            parity(og, fg, *run_oracle(w), f"noalloc {w.name}")
        else:
            parity(og[:, heads], fg[:, heads], *run_oracle(w, heads=heads), f"noalloc {w.name}")


def test_noalloc_rejects_sizes_beyond_its_array(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([16384], H=96, seed=82)
    t = wl.to_torch(w, dev)
    o = torch.empty((w.T, w.H, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(kda.KDAError) as err:
        kda.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], o,
                              initial_state=t["initial_state"], scale=w.scale)
    assert err.value.status == 3
