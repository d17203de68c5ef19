"""Helpers shared by the GPU tests."""

import sys

import numpy as np

import oracle
from chunked_kda_prefill_amd import workloads as wl

# The parity bar for o and final_state, per tensor: max |x - ref| <= 2e-2 and
# ||x - ref||_F / ||ref||_F <= 5e-3, computed in fp64 against the fp64 oracle.
MAX_ABS = 2e-2
REL_FRO = 5e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(w: wl.Workload, dev, scale=None, with_h0=True, **kw):
    import chunked_kda_prefill_amd as kda
    t = wl.to_torch(w, dev)
    o, f = kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                         initial_state=t["initial_state"] if with_h0 else None,
                         scale=w.scale if scale is None else scale, **kw)
    import torch
    torch.cuda.synchronize()
    return wl.bf16_tensor_to_f32(o).astype(np.float64), f.cpu().numpy().astype(np.float64)


def run_oracle(w: wl.Workload, scale=None, heads=None):
    return oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.initial_state,
                          scale=w.scale if scale is None else scale, heads=heads)


def parity(o, f, o_ref, f_ref, label):
    r = {"o_maxabs": oracle.max_abs_err(o, o_ref), "o_relF": oracle.rel_fro_err(o, o_ref),
         "f_maxabs": oracle.max_abs_err(f, f_ref), "f_relF": oracle.rel_fro_err(f, f_ref)}
    log(f"[parity] {label}: " + " ".join(f"{k}={v:.3e}" for k, v in r.items()))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f)), label
    assert r["o_maxabs"] <= MAX_ABS and r["o_relF"] <= REL_FRO, (label, r)
    assert r["f_maxabs"] <= MAX_ABS and r["f_relF"] <= REL_FRO, (label, r)
    return r
