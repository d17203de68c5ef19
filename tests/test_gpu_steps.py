"""Step-level GPU checks: chunk table (bit-exact), chunk-local gate cumsum,
and the intra-chunk kernel's intermediates against the fp64 chunk form."""

import numpy as np
import pytest

import oracle
from chunked_kda_prefill_amd import workloads as wl

from gpu_util import log
from ws_decode import BLOCK, decode_block

pytestmark = pytest.mark.gpu

CU_CASES = [
    [70, 130],                        # the TPU report's worked example
    [0, 64, 0, 128, 1, 0],            # empty sequences and exact multiples
    [1, 8, 15, 16, 17, 63, 64, 65, 130, 210],
    [5000],
    list(np.random.default_rng(3).integers(0, 400, size=300)),  # > 256 sequences
]


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@pytest.mark.parametrize("lens", CU_CASES, ids=lambda x: f"N{len(x)}")
def test_chunk_table_bit_exact(dev, lens):
    import torch
    import chunked_kda_prefill_amd as kda
    cu = _cu(lens)
    T = int(cu[-1])
    log(f"[chunk_table] N={len(lens)} T={T}")
    first, info, flags = kda.chunk_table(torch.from_numpy(cu).to(dev), T)
    torch.cuda.synchronize()
    rows = oracle.chunk_table(cu)
    first = first.cpu().numpy()
    info = info.cpu().numpy()
    assert int(flags.cpu()[0]) == 0
    nc = len(rows)
    assert first[-1] == nc
    counts = [(int(L) + 63) // 64 for L in lens]
    assert list(first) == list(np.concatenate([[0], np.cumsum(counts)]))
    exp = np.array([[r["start"], r["length"], r["seq"], r["local"]] for r in rows],
                   dtype=np.int32).reshape(-1, 4)
    assert np.array_equal(info[:nc], exp)
    assert np.all(info[nc:] == np.array([0, 0, -1, -1]))


def test_chunk_table_clamps_malformed_offsets(dev):
    import torch
    import chunked_kda_prefill_amd as kda
    # decreasing offsets and a last offset past T: clamped, flagged, in bounds
    cu = np.array([0, 100, 40, 300], dtype=np.int32)
    T = 200
    log("[chunk_table] malformed cu")
    first, info, flags = kda.chunk_table(torch.from_numpy(cu).to(dev), T)
    torch.cuda.synchronize()
    assert int(flags.cpu()[0]) == 1
    info = info.cpu().numpy()
    nc = int(first.cpu()[-1])
    nc_max = (T + 63 * 3) // 64
    assert nc <= nc_max
    assert np.all(info[:nc, 0] >= 0) and np.all(info[:nc, 0] + info[:nc, 1] <= T)


@pytest.mark.parametrize("lens", CU_CASES + [list(np.random.default_rng(6).integers(0, 90, size=n))
                                             for n in (1024, 1025)],
                         ids=lambda x: f"N{len(x)}")
def test_chunk_table_in_workspace(dev, lens):
    # the table the forward pass leaves in its workspace (built inside the
    # intra-chunk kernel for up to 1024 sequences, by its own kernel above)
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.make_workload(f"table_N{len(lens)}", lens, H=1, seed=34)
    log(f"[workspace table] N={w.N} T={w.T}")
    t = wl.to_torch(w, dev)
    ws = kda.new_workspace(w.T, w.N, w.H, dev).fill_(0xA5)    # no stale table to pass on
    kda.chunk_intra(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                    scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    lay = kda.workspace_layout(w.T, w.N, w.H)
    raw = ws.cpu().numpy()
    flags = raw[lay["flags"]:lay["flags"] + 4].view(np.int32)
    first = raw[lay["chunk_first"]:lay["chunk_first"] + 4 * (w.N + 1)].view(np.int32)
    info = raw[lay["chunk_info"]:lay["chunk_info"] + 16 * lay["nc_max"]].view(np.int32)
    info = info.reshape(-1, 4)
    rows = oracle.chunk_table(w.cu_seqlens)
    nc = len(rows)
    assert int(flags[0]) == 0
    counts = [(int(L) + 63) // 64 for L in lens]
    assert list(first) == list(np.concatenate([[0], np.cumsum(counts)]))
    exp = np.array([[r["start"], r["length"], r["seq"], r["local"]] for r in rows],
                   dtype=np.int32).reshape(-1, 4)
    assert np.array_equal(info[:nc], exp)
    assert np.all(info[nc:] == np.array([0, 0, -1, -1]))


def test_chunk_table_in_workspace_clamps_malformed_offsets(dev):
    # the same clamping when the intra-chunk kernel builds the table
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.make_workload("table_malformed", [100, 100], H=1, seed=35)
    t = wl.to_torch(w, dev)
    cu = torch.tensor([0, 100, 40, 300], dtype=torch.int32, device=dev)
    T, N = 200, 3
    log("[workspace table] malformed cu")
    ws = kda.new_workspace(T, N, 1, dev).fill_(0xA5)
    kda.chunk_intra(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    lay = kda.workspace_layout(T, N, 1)
    raw = ws.cpu().numpy()
    assert int(raw[lay["flags"]:lay["flags"] + 4].view(np.int32)[0]) == 1
    first = raw[lay["chunk_first"]:lay["chunk_first"] + 4 * (N + 1)].view(np.int32)
    info = raw[lay["chunk_info"]:lay["chunk_info"] + 16 * lay["nc_max"]].view(np.int32)
    info = info.reshape(-1, 4)
    nc = int(first[-1])
    assert nc <= lay["nc_max"]
    assert np.all(info[:nc, 0] >= 0) and np.all(info[:nc, 0] + info[:nc, 1] <= T)


@pytest.mark.parametrize("lens", [[256], [70, 130, 1, 64], [3, 200]], ids=str)
def test_gate_cumsum(dev, lens):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small(lens, H=3, seed=31, pinned_fraction=0.1)
    log(f"[gate_cumsum] lens={lens}")
    t = wl.to_torch(w, dev)
    G = kda.gate_cumsum(t["g"], t["cu_seqlens"])
    torch.cuda.synchronize()
    G = G.cpu().numpy().astype(np.float64)
    ref = np.zeros_like(G)
    for r in oracle.chunk_table(w.cu_seqlens):
        a, n = r["start"], r["length"]
        ref[a:a + n] = np.cumsum(w.g[a:a + n].astype(np.float64), axis=0)
    err = np.abs(G - ref)
    log(f"[gate_cumsum] max abs err {err.max():.3e} (|G| <= {np.abs(ref).max():.1f})")
    assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(ref)) * 64)
    for r in oracle.chunk_table(w.cu_seqlens):          # first row of a chunk is g itself
        assert np.array_equal(G[r["start"]], w.g[r["start"]].astype(np.float64))


@pytest.mark.parametrize("lens,scale", [([130, 64, 37], None), ([64], 1.0)], ids=["varlen", "s1"])
def test_intra_intermediates(dev, lens, scale):
    import torch
    import chunked_kda_prefill_amd as kda
    w = wl.small(lens, H=2, seed=32, pinned_fraction=0.1, scale=scale)
    log(f"[intra] lens={lens} scale={w.scale}")
    t = wl.to_torch(w, dev)
    ws = kda.chunk_intra(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                         scale=w.scale)
    torch.cuda.synchronize()
    lay = kda.workspace_layout(w.T, w.N, w.H)
    raw = ws.cpu().numpy()
    q, k, v = (wl.bf16_bits_to_f32(x) for x in (w.q, w.k, w.v))
    worst = {}
    for c, r in enumerate(oracle.chunk_table(w.cu_seqlens)):
        a, n = r["start"], r["length"]
        for h in range(w.H):
            off = lay["blocks"] + (h * lay["nc_max"] + c) * lay["block_bytes"]
            got = decode_block(raw[off:off + BLOCK])
            ref = oracle.chunk_terms(q[a:a + n, h], k[a:a + n, h], v[a:a + n, h],
                                     w.g[a:a + n, h], w.beta[a:a + n, h], w.scale)
            for name in ("W", "U", "qg", "kg", "Aqk"):
                x = got[name]
                rr = np.zeros_like(x)
                rr[:n, :ref[name].shape[1]] = ref[name]
                e = oracle.rel_fro_err(x, rr)
                worst[name] = max(worst.get(name, 0.0), e)
                # rows past a partial chunk's end are exactly zero
                assert not np.any(x[n:]), (name, c, h)
            # gamma = exp(G_last) underflows fp32 for long strong decays:
            # absolute error everywhere, relative where it is representable
            ga, gr = got["gamma"], ref["gamma"]
            big = gr > 1e-30
            eg = max(float(np.max(np.abs(ga - gr))),
                     float(np.max(np.abs(ga[big] / gr[big] - 1.0))) if big.any() else 0.0)
            worst["gamma"] = max(worst.get("gamma", 0.0), eg)
    log("[intra] worst relF " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    # bf16 storage of one rounding: ~2^-9 relative per element
    for name in ("W", "U", "qg", "kg"):
        assert worst[name] < 4e-3, (name, worst[name])
    # Aqk: bf16 strip operands (one rounding each side), then bf16 storage
    assert worst["Aqk"] < 8e-3
    assert worst["gamma"] < 1e-4
