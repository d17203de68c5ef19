"""Host side of the C ABI (no GPU needed): the library loads, exports every
function include/kda.h declares, sizes its workspace, and rejects bad
arguments before launching anything."""

import ctypes
import os
import re

import pytest

import chunked_kda_prefill_amd as kda
from chunked_kda_prefill_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", src)))


def test_header_declarations_are_exported():
    lib = kda.load_library()
    names = declared_functions()
    assert names, "no declarations parsed"
    assert sorted(names) == sorted(_binding.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = kda.load_library()
    for code, name in _binding.STATUS_NAMES.items():
        assert lib.kda_status_string(code).decode() == name
    assert lib.kda_status_string(99).decode() == "KDA_ERR_UNKNOWN"


def test_workspace_size_and_layout():
    T, N, H = 8192, 4, 16
    lay = kda.workspace_layout(T, N, H)
    assert lay["nc_max"] == (T + 63 * N) // 64
    assert lay["block_bytes"] == 72192
    for key in ("chunk_first", "chunk_info", "blocks"):
        assert lay[key] % 256 == 0
    assert lay["chunk_info"] >= lay["chunk_first"] + 4 * (N + 1)
    assert lay["blocks"] >= lay["chunk_info"] + 16 * lay["nc_max"]
    assert kda.workspace_size(T, N, H) == lay["blocks"] + H * lay["nc_max"] * 72192
    assert kda.workspace_size(0, 1, 1) > 0
    for bad in [(-1, 1, 1), (10, 0, 1), (10, 1, 0)]:
        assert kda.workspace_size(*bad) == 0
    assert kda.workspace_size(2**31, 1, 1) == 0          # beyond int32 tokens
    assert kda.workspace_size(10, 1, 70000) == 0         # beyond the head limit


def _fwd(lib, **over):
    """Call kda_chunk_fwd with fake, aligned, non-null host addresses: every
    call here must be rejected by host-side validation before any launch."""
    A = 1 << 20
    args = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, h0=None, cu=6 * A, T=128, N=1,
                H=2, scale=1.0, o=7 * A, hT=8 * A, ws=9 * A, ws_bytes=0, stream=None)
    args.update(over)
    return lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"],
                             args["h0"], args["cu"], args["T"], args["N"], args["H"],
                             args["scale"], args["o"], args["hT"], args["ws"],
                             args["ws_bytes"], args["stream"])


def test_invalid_arguments_are_rejected_before_launch():
    lib = kda.load_library()
    INV, UNS, WS = 1, 2, 3
    assert _fwd(lib, q=None) == INV
    assert _fwd(lib, cu=None) == INV
    assert _fwd(lib, o=None) == INV
    assert _fwd(lib, ws=None, ws_bytes=10**9) == INV
    assert _fwd(lib, T=-1) == INV
    assert _fwd(lib, N=0) == INV
    assert _fwd(lib, H=0) == INV
    assert _fwd(lib, H=70000) == UNS
    assert _fwd(lib, T=2**31) == UNS
    assert _fwd(lib, q=(1 << 20) + 8) == INV                 # misaligned
    assert _fwd(lib, beta=(5 << 20) + 2) == INV
    assert _fwd(lib, ws=(9 << 20) + 16, ws_bytes=10**9) == INV  # workspace not 256-aligned
    assert _fwd(lib) == WS                                    # workspace too small
    need = kda.workspace_size(128, 1, 2)
    assert _fwd(lib, ws_bytes=need - 1) == WS
    # o aliasing an input, and overlapping (not identical) state buffers
    assert _fwd(lib, o=(1 << 20) + 64, ws_bytes=need) == INV
    assert _fwd(lib, h0=8 << 20, hT=(8 << 20) + 256, ws_bytes=need) == INV
    # o overlapping the workspace
    assert _fwd(lib, o=(9 << 20) + 4096, ws_bytes=need) == INV
    A = 1 << 20
    # the workspace is written while every input is still being read: an
    # overlap with any of them is rejected
    for name in ("q", "k", "v", "g", "beta", "cu"):
        assert _fwd(lib, ws=9 * A, ws_bytes=need, **{name: 9 * A + 4096}) == INV, name
    assert _fwd(lib, ws=9 * A, ws_bytes=need, h0=9 * A + 8192) == INV
    # o overlapping cu_seqlens or the initial state; final_state overlapping
    # an input other than the initial state
    assert _fwd(lib, ws_bytes=need, cu=7 * A + 256) == INV
    assert _fwd(lib, ws_bytes=need, h0=7 * A + 4096) == INV
    for name in ("q", "k", "v", "g", "beta", "cu"):
        assert _fwd(lib, ws_bytes=need, **{name: 8 * A + 512}) == INV, name
    # ... while final_state == initial_state (in place) is accepted by the
    # host checks (a launch is never reached with these fake addresses only
    # because the workspace check comes first in this call)
    assert _fwd(lib, h0=8 * A, hT=8 * A) == 3


def test_step_entry_points_reject_bad_arguments():
    lib = kda.load_library()
    P = 1 << 20
    assert lib.kda_chunk_table(None, 10, 1, P, P, P, None) == 1
    assert lib.kda_chunk_table(P, 10, 0, P, P, P, None) == 1
    assert lib.kda_gate_cumsum(P, P, 10, 1, 1, 2 * P, 4 * P, 0, None) == 3
    assert lib.kda_gate_cumsum(P, P, 10, 1, 1, P, 4 * P, 10**9, None) == 1  # G aliases g
    assert lib.kda_chunk_intra(P, P, P, P, P, P, 10, 1, 1, 1.0, None, 10**9, None) == 1
    # a workspace over an input of the intra step, or of the gate cumsum
    W = 64 * P
    assert lib.kda_chunk_intra(P, 2 * P, 3 * P, 4 * P, 5 * P, W + 512, 10, 1, 1, 1.0,
                               W, 10**9, None) == 1
    assert lib.kda_chunk_intra(W + 4096, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 10, 1, 1, 1.0,
                               W, 10**9, None) == 1
    assert lib.kda_gate_cumsum(W + 4096, P, 10, 1, 1, 2 * P, W, 10**9, None) == 1
    assert lib.kda_gate_cumsum(P, W + 256, 10, 1, 1, 2 * P, W, 10**9, None) == 1
    assert lib.kda_gate_cumsum(P, 2 * P + 64, 10, 1, 1, 2 * P, W, 10**9, None) == 1  # G over cu
    out = (ctypes.c_int64 * 5)()
    assert lib.kda_workspace_layout(-5, 1, 1, out) == 1


def test_decode_entry_rejects_bad_arguments():
    # host-checked argument errors of kda_decode_fwd (no launch is reached)
    lib = kda.load_library()
    A = 1 << 20
    def dec(**over):
        a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, h0=None, cu=6 * A, T=128, N=1,
                 H=2, scale=1.0, o=7 * A, hT=8 * A, stream=None)
        a.update(over)
        return lib.kda_decode_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                  a["T"], a["N"], a["H"], a["scale"], a["o"], a["hT"], a["stream"])
    INV, UNS = 1, 2
    assert dec(q=None) == INV
    assert dec(cu=None) == INV
    assert dec(o=None) == INV
    assert dec(T=-1) == INV
    assert dec(N=0) == INV
    assert dec(H=70000) == UNS
    assert dec(k=(2 << 20) + 8) == INV                     # misaligned
    assert dec(o=(3 << 20) + 64) == INV                    # o aliases v
    assert dec(h0=8 << 20, hT=(8 << 20) + 256) == INV     # partly overlapping states
    # every workgroup reads cu_seqlens while others write o and the state
    assert dec(cu=7 * A + 128) == INV                      # o over cu_seqlens
    assert dec(h0=7 * A + 4096) == INV                     # o over the initial state
    for name in ("q", "k", "v", "g", "beta", "cu"):
        assert dec(**{name: 8 * A + 512}) == INV, name    # final_state over an input


def test_fused_entries_reject_bad_arguments():
    # host-checked argument errors of the fused entry points (no launch is reached)
    lib = kda.load_library()
    A = 1 << 20
    def call(fn, **over):
        a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, bs=2, eps=1e-6, h0=None, cu=6 * A,
                 T=128, N=1, H=2, scale=1.0, o=7 * A, hT=8 * A)
        a.update(over)
        head = (a["q"], a["k"], a["v"], a["g"], a["b"], a["bs"], a["eps"], a["h0"], a["cu"],
                a["T"], a["N"], a["H"], a["scale"], a["o"], a["hT"])
        if fn == "chunk":
            return lib.kda_chunk_fwd_fused(*head, 9 * A, 64 * A, None)
        return lib.kda_decode_fwd_fused(*head, None)
    INV = 1
    for fn in ("chunk", "decode"):
        assert call(fn, b=None) == INV                     # logits required when T > 0
        assert call(fn, eps=float("nan")) == INV
        assert call(fn, bs=1) == INV                       # row stride below H
        assert call(fn, bs=1 << 25) == INV                 # row stride beyond 2^24
        assert call(fn, b=(5 << 20) + 1) == INV            # misaligned logits
        assert call(fn, o=(5 << 20) + 64) == INV           # o overlaps the logits


def test_gated_rmsnorm_rejects_bad_arguments():
    # host-checked argument errors of kda_gated_rmsnorm (no launch is reached)
    lib = kda.load_library()
    A = 1 << 20
    def call(**over):
        a = dict(x=A, xs=256, z=2 * A, zs=256, w=3 * A, eps=1e-6, act=0, T=16, H=2, y=4 * A)
        a.update(over)
        return lib.kda_gated_rmsnorm(a["x"], a["xs"], a["z"], a["zs"], a["w"], a["eps"],
                                     a["act"], a["T"], a["H"], a["y"], None)
    INV, UNS = 1, 2
    assert call(T=0, x=None, y=None) == 0                 # empty: no-op
    assert call(x=None) == INV
    assert call(w=None) == INV
    assert call(act=2) == INV
    assert call(eps=-1.0) == INV
    assert call(eps=float("nan")) == INV
    assert call(eps=float("inf")) == INV
    assert call(xs=255) == INV                            # below H * 128
    assert call(zs=260) == INV                            # not a multiple of 8
    assert call(xs=(1 << 31) + 8) == INV                  # stride beyond 2^31
    assert call(z=2 * A + 8) == INV                       # misaligned
    assert call(y=A + 512) == INV                         # y overlaps x (not in place)
    assert call(y=2 * A) == INV                           # y is the gate
    assert call(H=70000, xs=70000 * 128, zs=70000 * 128) == UNS


def test_decode_step_rejects_bad_arguments():
    # host-checked argument errors of kda_decode_step_fused (no launch is reached)
    lib = kda.load_library()
    A = 1 << 20
    def call(**over):
        a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, bs=2, eps=1e-6, h0=None, cu=6 * A,
                 T=16, N=1, H=2, scale=1.0, z=7 * A, zs=256, nw=8 * A, neps=1e-6, act=0,
                 o=9 * A, y=10 * A, hT=11 * A)
        a.update(over)
        return lib.kda_decode_step_fused(a["q"], a["k"], a["v"], a["g"], a["b"], a["bs"],
                                         a["eps"], a["h0"], a["cu"], a["T"], a["N"], a["H"],
                                         a["scale"], a["z"], a["zs"], a["nw"], a["neps"],
                                         a["act"], a["o"], a["y"], a["hT"], None)
    INV = 1
    assert call(y=None) == INV                      # y required when T > 0
    assert call(b=None) == INV
    assert call(z=None) == INV
    assert call(nw=None) == INV
    assert call(act=5) == INV
    assert call(neps=-1.0) == INV
    assert call(neps=float("nan")) == INV
    assert call(zs=255) == INV                      # below H * 128
    assert call(zs=(1 << 31) + 8) == INV            # beyond 2^31
    assert call(z=7 * A + 1) == INV                 # misaligned gate
    assert call(nw=8 * A + 2) == INV                # misaligned weight
    assert call(y=9 * A + 64) == INV                # y overlaps o
    assert call(y=7 * A) == INV                     # y is the gate
    assert call(y=11 * A) == INV                    # y overlaps the state


def test_validate_rejects_bad_arguments():
    # host-checked argument errors of kda_validate_inputs (no launch is reached)
    lib = kda.load_library()
    A = 1 << 20
    def call(**over):
        a = dict(g=A, beta=2 * A, cu=3 * A, T=16, N=1, H=2, flags=4 * A)
        a.update(over)
        return lib.kda_validate_inputs(a["g"], a["beta"], a["cu"], a["T"], a["N"], a["H"],
                                       a["flags"], None)
    INV = 1
    assert call(flags=None) == INV
    assert call(cu=None) == INV
    assert call(g=None) == INV
    assert call(g=A + 4) == INV                     # g not 16-byte aligned
    assert call(flags=A + 64) == INV                # flags inside g
    assert call(N=0) == INV


def test_python_wrapper_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load_library()


def test_noalloc_entry_checks_before_any_device_call():
    # kda_chunk_fwd_noalloc rejects sizes whose workspace exceeds its
    # library-owned array, and bad arguments, before it looks at any device
    lib = kda.load_library()
    A = 1 << 20

    def call(**over):
        a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, h0=None, cu=6 * A, T=128, N=1,
                 H=2, scale=1.0, o=7 * A, hT=8 * A)
        a.update(over)
        return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"],
                                         a["cu"], a["T"], a["N"], a["H"], a["scale"], a["o"],
                                         a["hT"], None)
    INV, WS = 1, 3
    limit = kda.NOALLOC_WORKSPACE_BYTES
    assert kda.workspace_size(8192, 4, 16) <= limit          # the headline shape fits
    assert kda.workspace_size(16384, 1, 96) > limit          # the long shape does not
    assert call(T=16384, N=1, H=96) == WS
    assert call(q=None) == INV
    assert call(T=-1) == INV
    assert call(o=(1 << 20) + 64) == INV                      # o over q


def test_segmented_entry_rejects_bad_arguments():
    lib = kda.load_library()
    A = 1 << 20
    assert lib.kda_chunk_fwd_segmented_workspace_size(2048, 1, 16, 0) == 0
    assert lib.kda_chunk_fwd_segmented_workspace_size(2048, 1, 16, 65) == 0
    plain = kda.workspace_size(2048, 1, 16)
    need = lib.kda_chunk_fwd_segmented_workspace_size(2048, 1, 16, 4)
    # segment 0's exit state and two maps (M, b) per chain for the middle segments
    assert need >= plain + 16 * (1 + 2 * 2) * 128 * 128 * 4
    assert lib.kda_chunk_fwd_segmented_workspace_size(2048, 1, 16, 1) >= plain

    def call(segments=4, ws_bytes=0, **over):
        a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, h0=None, cu=6 * A, T=128, N=1, H=2,
                 o=7 * A, hT=8 * A, ws=64 * A)
        a.update(over)
        return lib.kda_chunk_fwd_segmented(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"],
                                           a["cu"], a["T"], a["N"], a["H"], 1.0, segments,
                                           a["o"], a["hT"], a["ws"], ws_bytes, None)
    assert call(segments=0) == 1
    assert call(segments=65) == 1
    assert call(q=None) == 1
    assert call() == 3                                         # workspace too small
    small = lib.kda_chunk_fwd_segmented_workspace_size(128, 1, 2, 4)
    assert call(ws_bytes=small - 1) == 3
    assert call(ws_bytes=small, cu=64 * A + 256) == 1          # workspace over an input
