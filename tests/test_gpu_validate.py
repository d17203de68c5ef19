"""kda_validate_inputs: the opt-in check of the device-content contracts.
The inputs here are only read by the validator; none of them is passed to
a forward entry point."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def test_valid_inputs_pass(dev):
    import chunked_kda_prefill_amd as kda
    for w in (wl.headline(), wl.by_name("long"), wl.small([0, 1, 63, 64, 65, 0], H=3, seed=80)):
        t = wl.to_torch(w, dev)
        log(f"[case] validate {w.name}")
        # the long workload pins channels at exactly -5: the bound is inclusive
        assert kda.validate_inputs(t["g"], t["beta"], t["cu_seqlens"]) == set()
        assert kda.validate_inputs(t["g"], None, t["cu_seqlens"]) == set()


def test_each_contract_is_reported(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small([100, 64, 3, 130], H=2, seed=81)
    base = wl.to_torch(w, dev)
    T = w.T

    def check(g=None, beta=None, cu=None):
        return kda.validate_inputs(base["g"] if g is None else g,
                                   base["beta"] if beta is None else beta,
                                   base["cu_seqlens"] if cu is None else cu)

    log("[case] validate planted violations")
    for val in (-5.0001, 0.0001, float("nan"), float("-inf")):
        g = base["g"].clone()
        g[T - 1, 1, 127] = val                    # the very last element
        assert check(g=g) == {"g"}, val
    g = base["g"].clone()
    g[0, 0, 0] = 1.0
    assert check(g=g) == {"g"}
    for val in (1.5, -0.25, float("nan")):
        b = base["beta"].clone()
        b[37, 0] = val
        assert check(beta=b) == {"beta"}, val
    cu = base["cu_seqlens"].clone()
    cu[2], cu[3] = cu[3].item(), cu[2].item()     # not monotone
    assert check(cu=cu) == {"cu_seqlens"}
    cu = base["cu_seqlens"].clone()
    cu[-1] = T - 1                                # does not end at T
    assert check(cu=cu) == {"cu_seqlens"}
    cu = base["cu_seqlens"].clone()
    cu[0] = 1                                     # does not start at 0
    assert check(cu=cu) == {"cu_seqlens"}
    g = base["g"].clone()
    g[5, 0, 5] = 2.0
    b = base["beta"].clone()
    b[0, 1] = -1.0
    assert check(g=g, beta=b, cu=cu) == {"g", "beta", "cu_seqlens"}
    # the word is cleared by every call
    assert check() == set()
