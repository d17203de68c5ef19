"""ctypes binding of libkda.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kda.h.  PyTorch provides device
memory and the current HIP stream.  If the library is missing, every entry
point raises -- there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_OK = 0
HEAD_DIM = 128
CHUNK = 64
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
                3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}

# Every symbol include/kda.h declares.
EXPORTED = ("kda_status_string", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd",
            "kda_chunk_table", "kda_gate_cumsum", "kda_chunk_intra",
            "kda_workspace_layout", "kda_chunk_recurrence", "kda_decode_fwd",
            "kda_chunk_fwd_fused", "kda_decode_fwd_fused", "kda_gated_rmsnorm",
            "kda_decode_step_fused", "kda_validate_inputs", "kda_chunk_fwd_noalloc",
            "kda_chunk_fwd_segmented", "kda_chunk_fwd_segmented_workspace_size")
VALIDATION_BITS = {1: "cu_seqlens", 2: "g", 4: "beta"}
ACTIVATIONS = {"sigmoid": 0, "silu": 1}


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def load_library():
    """Load libkda.so (built in-tree by chunked_kda_prefill_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m chunked_kda_prefill_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_float, ctypes.c_size_t)
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_size.argtypes = [I64, I32, I32]
    lib.kda_chunk_fwd_workspace_size.restype = SZ
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F32, P, P, P, SZ, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_segmented.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F32, I32, P, P,
                                            P, SZ, P]
    lib.kda_chunk_fwd_segmented.restype = ctypes.c_int
    lib.kda_chunk_fwd_segmented_workspace_size.argtypes = [I64, I32, I32, I32]
    lib.kda_chunk_fwd_segmented_workspace_size.restype = SZ
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F32, P, P, P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_decode_fwd.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F32, P, P, P]
    lib.kda_decode_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_fused.argtypes = [P, P, P, P, P, I64, F32, P, P, I64, I32, I32, F32, P, P, P,
                                        SZ, P]
    lib.kda_chunk_fwd_fused.restype = ctypes.c_int
    lib.kda_decode_fwd_fused.argtypes = [P, P, P, P, P, I64, F32, P, P, I64, I32, I32, F32, P, P, P]
    lib.kda_decode_fwd_fused.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [P, I64, P, I64, P, F32, I32, I64, I32, P, P]
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_decode_step_fused.argtypes = [P, P, P, P, P, I64, F32, P, P, I64, I32, I32, F32,
                                          P, I64, P, F32, I32, P, P, P, P]
    lib.kda_decode_step_fused.restype = ctypes.c_int
    lib.kda_validate_inputs.argtypes = [P, P, P, I64, I32, I32, P, P]
    lib.kda_validate_inputs.restype = ctypes.c_int
    lib.kda_chunk_table.argtypes = [P, I64, I32, P, P, P, P]
    lib.kda_chunk_table.restype = ctypes.c_int
    lib.kda_gate_cumsum.argtypes = [P, P, I64, I32, I32, P, P, SZ, P]
    lib.kda_gate_cumsum.restype = ctypes.c_int
    lib.kda_chunk_intra.argtypes = [P, P, P, P, P, P, I64, I32, I32, F32, P, SZ, P]
    lib.kda_chunk_intra.restype = ctypes.c_int
    lib.kda_chunk_recurrence.argtypes = [P, I64, I32, I32, P, P, P, SZ, P]
    lib.kda_chunk_recurrence.restype = ctypes.c_int
    lib.kda_workspace_layout.argtypes = [I64, I32, I32, ctypes.POINTER(ctypes.c_int64)]
    lib.kda_workspace_layout.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != KDA_OK:
        raise KDAError(fn, status)


def workspace_size(T: int, N: int, H: int) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(T, N, H))


def workspace_layout(T: int, N: int, H: int) -> dict:
    out = (ctypes.c_int64 * 5)()
    _check("kda_workspace_layout", load_library().kda_workspace_layout(T, N, H, out))
    return {"flags": out[0], "chunk_first": out[1], "chunk_info": out[2],
            "blocks": out[3], "block_bytes": out[4],
            "nc_max": (T + (CHUNK - 1) * N) // CHUNK}


# ---------------------------------------------------------------------------
# torch-facing helpers (torch is imported lazily: the CPU tests that only
# exercise the host side of the ABI do not need a GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _expect(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _check_inputs(q, k, v, g, beta, cu_seqlens):
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [T, H, {HEAD_DIM}]")
    T, H = int(q.shape[0]), int(q.shape[1])
    _expect(q, "q", torch.bfloat16)
    _expect(k, "k", torch.bfloat16, (T, H, HEAD_DIM))
    _expect(v, "v", torch.bfloat16, (T, H, HEAD_DIM))
    _expect(g, "g", torch.float32, (T, H, HEAD_DIM))
    if beta is not None:
        _expect(beta, "beta", torch.float32, (T, H))
    _expect(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = int(cu_seqlens.shape[0]) - 1
    return T, N, H


def new_workspace(T: int, N: int, H: int, device):
    torch = _torch()
    nbytes = workspace_size(T, N, H)
    if nbytes == 0:
        raise ValueError(f"invalid sizes T={T} N={N} H={H}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def chunk_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, scale: Optional[float] = None,
              output_final_state: bool = True, workspace=None, o=None,
              final_state=None) -> Tuple[object, object]:
    """KDA chunked prefill forward on the GPU (kda_chunk_fwd).

    q, k, v: bf16 [T, H, 128]; g: fp32 [T, H, 128] in [-5, 0]; beta: fp32
    [T, H]; cu_seqlens: int32 [N + 1]; initial_state: fp32 [N, H, 128, 128]
    or None.  Returns (o bf16 [T, H, 128], final_state fp32 [N, H, 128, 128]
    or None).  Runs on the current stream of q's device.
    """
    torch = _torch()
    T, N, H = _check_inputs(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if o is None:
        o = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _expect(o, "o", torch.bfloat16, (T, H, HEAD_DIM))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _expect(final_state, "final_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if workspace is None:
        workspace = new_workspace(T, N, H, dev)
    st = load_library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(o), _ptr(final_state), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check("kda_chunk_fwd", st)
    return o, final_state


def chunk_fwd_segmented(q, k, v, g, beta, cu_seqlens, segments: int, initial_state=None,
                        scale: Optional[float] = None, output_final_state: bool = True,
                        workspace=None, o=None, final_state=None):
    """kda_chunk_fwd_segmented: the chunked forward with chunk-parallel state
    passing, each chain cut into `segments` runs.  Returns (o, final_state)."""
    torch = _torch()
    T, N, H = _check_inputs(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if o is None:
        o = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _expect(o, "o", torch.bfloat16, (T, H, HEAD_DIM))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _expect(final_state, "final_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    lib = load_library()
    if workspace is None:
        nbytes = lib.kda_chunk_fwd_segmented_workspace_size(T, N, H, int(segments))
        if nbytes == 0:
            raise ValueError(f"invalid sizes T={T} N={N} H={H} segments={segments}")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_fwd_segmented(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), int(segments), _ptr(o), _ptr(final_state), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check("kda_chunk_fwd_segmented", st)
    return o, final_state


NOALLOC_WORKSPACE_BYTES = 160 << 20


def chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, o, final_state=None, initial_state=None,
                      scale: Optional[float] = None):
    """kda_chunk_fwd_noalloc: the chunked forward with the library's own
    per-GPU workspace.  The caller passes the outputs (o bf16 [T, H, 128],
    final_state fp32 [N, H, 128, 128] or None); nothing is allocated.
    Calls that overlap in time on one GPU race."""
    torch = _torch()
    T, N, H = _check_inputs(q, k, v, g, beta, cu_seqlens)
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    _expect(o, "o", torch.bfloat16, (T, H, HEAD_DIM))
    if final_state is not None:
        _expect(final_state, "final_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load_library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(o), _ptr(final_state), _stream(q.device))
    _check("kda_chunk_fwd_noalloc", st)
    return o, final_state


def decode_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, scale: Optional[float] = None,
               output_final_state: bool = True, o=None, final_state=None) -> Tuple[object, object]:
    """Token-serial KDA forward for decode steps and speculative verification
    windows (kda_decode_fwd): the same arguments and results as chunk_fwd,
    without a workspace; meant for a few tokens per sequence.  Pass
    final_state=initial_state to update the state in place."""
    torch = _torch()
    T, N, H = _check_inputs(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if o is None:
        o = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _expect(o, "o", torch.bfloat16, (T, H, HEAD_DIM))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _expect(final_state, "final_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    st = load_library().kda_decode_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(o), _ptr(final_state), _stream(dev))
    _check("kda_decode_fwd", st)
    return o, final_state


def _fused_outputs(q, cu_seqlens, initial_state, o, final_state, output_final_state, T, N, H):
    torch = _torch()
    dev = q.device
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    if o is None:
        o = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _expect(o, "o", torch.bfloat16, (T, H, HEAD_DIM))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _expect(final_state, "final_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    return o, final_state


def _beta_logits(b, T: int, H: int):
    """b: a bf16 [T, W] tensor or a column slice of one (W >= H); returns its
    row stride in elements."""
    torch = _torch()
    if b.dtype != torch.bfloat16 or b.dim() != 2 or b.shape[0] != T or b.shape[1] != H \
            or b.stride(1) != 1 or (T > 1 and b.stride(0) < H):
        raise ValueError("b must be a bf16 [T, H] tensor with unit column stride (a column "
                         "slice of a row-major projection output is fine)")
    return int(b.stride(0)) if T > 1 else H


def chunk_fwd_fused(q, k, v, g, b, cu_seqlens, initial_state=None, scale: Optional[float] = None,
                    qk_eps: Optional[float] = 1e-6, output_final_state: bool = True,
                    workspace=None, o=None, final_state=None):
    """chunk_fwd with the prologue fused in (kda_chunk_fwd_fused): beta =
    sigmoid(b) from bf16 logits b [T, H] (a strided column slice is fine),
    and, unless qk_eps is None, q and k L2-normalised per (token, head) as
    x / sqrt(sum x^2 + qk_eps)."""
    T, N, H = _check_inputs(q, k, v, g, None, cu_seqlens)
    stride = _beta_logits(b, T, H)
    o, final_state = _fused_outputs(q, cu_seqlens, initial_state, o, final_state,
                                    output_final_state, T, N, H)
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if workspace is None:
        workspace = new_workspace(T, N, H, q.device)
    st = load_library().kda_chunk_fwd_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), stride,
        -1.0 if qk_eps is None else float(qk_eps), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(o), _ptr(final_state), _ptr(workspace), workspace.numel(),
        _stream(q.device))
    _check("kda_chunk_fwd_fused", st)
    return o, final_state


def decode_fwd_fused(q, k, v, g, b, cu_seqlens, initial_state=None, scale: Optional[float] = None,
                     qk_eps: Optional[float] = 1e-6, output_final_state: bool = True, o=None,
                     final_state=None):
    """decode_fwd with the prologue fused in (kda_decode_fwd_fused); b and
    qk_eps as in chunk_fwd_fused."""
    T, N, H = _check_inputs(q, k, v, g, None, cu_seqlens)
    stride = _beta_logits(b, T, H)
    o, final_state = _fused_outputs(q, cu_seqlens, initial_state, o, final_state,
                                    output_final_state, T, N, H)
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load_library().kda_decode_fwd_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), stride,
        -1.0 if qk_eps is None else float(qk_eps), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(o), _ptr(final_state), _stream(q.device))
    _check("kda_decode_fwd_fused", st)
    return o, final_state


def _rows(x, name: str):
    """x: bf16 [T, H, 128] whose (head, channel) block is contiguous; returns
    its token stride in elements."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dtype != torch.bfloat16 or x.dim() != 3 or x.shape[2] != HEAD_DIM \
            or x.stride(2) != 1 or x.stride(1) != HEAD_DIM:
        raise ValueError(f"{name} must be a bf16 [T, H, 128] tensor with contiguous heads and "
                         "channels (a token-strided view, e.g. a column slice, is fine)")
    return int(x.stride(0)) if x.shape[0] > 1 else x.shape[1] * HEAD_DIM


def gated_rmsnorm(x, gate, weight, eps: float = 1e-6, activation: str = "sigmoid", out=None):
    """Gated RMSNorm after the operation (kda_gated_rmsnorm): per (token,
    head) row, y = weight * x / sqrt(mean(x^2) + eps) * act(gate), act =
    sigmoid or silu.  x, gate: bf16 [T, H, 128] (token-strided views are
    fine); weight: fp32 [128].  Returns y, bf16 [T, H, 128]; out=x updates
    x in place (x contiguous)."""
    torch = _torch()
    xs, zs = _rows(x, "x"), _rows(gate, "gate")
    T, H = int(x.shape[0]), int(x.shape[1])
    if tuple(gate.shape) != tuple(x.shape) or gate.device != x.device:
        raise ValueError("gate must match x in shape and device")
    _expect(weight, "weight", torch.float32, (HEAD_DIM,))
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    if out is None:
        out = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
    else:
        _expect(out, "out", torch.bfloat16, (T, H, HEAD_DIM))
    st = load_library().kda_gated_rmsnorm(
        _ptr(x), xs, _ptr(gate), zs, _ptr(weight), float(eps), ACTIVATIONS[activation], T, H,
        _ptr(out), _stream(x.device))
    _check("kda_gated_rmsnorm", st)
    return out


def decode_step_fused(q, k, v, g, b, cu_seqlens, gate, norm_weight, initial_state=None,
                      scale: Optional[float] = None, qk_eps: Optional[float] = 1e-6,
                      norm_eps: float = 1e-6, activation: str = "sigmoid",
                      output_final_state: bool = True, o=None, y=None, final_state=None):
    """A whole decode step in one kernel (kda_decode_step_fused):
    decode_fwd_fused, then gated_rmsnorm(o, gate, norm_weight) on o's fp32
    rows.  gate: bf16 [T, H, 128] (token-strided views are fine).  Returns
    (o, y, final_state)."""
    torch = _torch()
    T, N, H = _check_inputs(q, k, v, g, None, cu_seqlens)
    stride = _beta_logits(b, T, H)
    zs = _rows(gate, "gate")
    if tuple(gate.shape) != (T, H, HEAD_DIM):
        raise ValueError(f"gate must have shape {(T, H, HEAD_DIM)}")
    _expect(norm_weight, "norm_weight", torch.float32, (HEAD_DIM,))
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    o, final_state = _fused_outputs(q, cu_seqlens, initial_state, o, final_state,
                                    output_final_state, T, N, H)
    if y is None:
        y = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    else:
        _expect(y, "y", torch.bfloat16, (T, H, HEAD_DIM))
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load_library().kda_decode_step_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), stride,
        -1.0 if qk_eps is None else float(qk_eps), _ptr(initial_state), _ptr(cu_seqlens),
        T, N, H, float(scale), _ptr(gate), zs, _ptr(norm_weight), float(norm_eps),
        ACTIVATIONS[activation], _ptr(o), _ptr(y), _ptr(final_state), _stream(q.device))
    _check("kda_decode_step_fused", st)
    return o, y, final_state


def validate_inputs(g, beta, cu_seqlens):
    """Opt-in check of the device-content contracts (kda_validate_inputs):
    returns the set of failed checks, a subset of {"cu_seqlens", "g",
    "beta"} (empty when all hold).  beta may be None.  Synchronises the
    current stream to read the result."""
    torch = _torch()
    _expect(cu_seqlens, "cu_seqlens", torch.int32)
    _expect(g, "g", torch.float32)
    if g.dim() != 3 or g.shape[2] != HEAD_DIM:
        raise ValueError("g must be fp32 [T, H, 128]")
    T, H = int(g.shape[0]), int(g.shape[1])
    if beta is not None:
        _expect(beta, "beta", torch.float32, (T, H))
    N = int(cu_seqlens.shape[0]) - 1
    flags = torch.empty(1, dtype=torch.int32, device=g.device)
    st = load_library().kda_validate_inputs(_ptr(g), _ptr(beta), _ptr(cu_seqlens), T, N, H,
                                            _ptr(flags), _stream(g.device))
    _check("kda_validate_inputs", st)
    word = int(flags.item())
    return {name for bit, name in VALIDATION_BITS.items() if word & bit}


def chunk_table(cu_seqlens, T: int):
    """Device chunk table (kda_chunk_table): (chunk_first [N+1], chunk_info
    [NCmax, 4], flags [1]), all int32 on cu_seqlens' device."""
    torch = _torch()
    _expect(cu_seqlens, "cu_seqlens", torch.int32)
    N = int(cu_seqlens.shape[0]) - 1
    nc_max = (T + (CHUNK - 1) * N) // CHUNK
    dev = cu_seqlens.device
    first = torch.empty(N + 1, dtype=torch.int32, device=dev)
    info = torch.empty((max(nc_max, 1), 4), dtype=torch.int32, device=dev)
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    st = load_library().kda_chunk_table(_ptr(cu_seqlens), T, N, _ptr(first), _ptr(info),
                                        _ptr(flags), _stream(dev))
    _check("kda_chunk_table", st)
    return first, info[:nc_max], flags


def gate_cumsum(g, cu_seqlens):
    """Chunk-local inclusive cumsum of g (kda_gate_cumsum), fp32 like g."""
    torch = _torch()
    _expect(g, "g", torch.float32)
    T, H = int(g.shape[0]), int(g.shape[1])
    _expect(cu_seqlens, "cu_seqlens", torch.int32)
    N = int(cu_seqlens.shape[0]) - 1
    G = torch.empty_like(g)
    ws = new_workspace(T, N, H, g.device)
    st = load_library().kda_gate_cumsum(_ptr(g), _ptr(cu_seqlens), T, N, H, _ptr(G), _ptr(ws),
                                        ws.numel(), _stream(g.device))
    _check("kda_gate_cumsum", st)
    return G


def chunk_intra(q, k, v, g, beta, cu_seqlens, scale: Optional[float] = None, workspace=None):
    """Chunk table + intra-chunk kernel (kda_chunk_intra); returns the
    workspace holding the intermediate blocks."""
    T, N, H = _check_inputs(q, k, v, g, beta, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if workspace is None:
        workspace = new_workspace(T, N, H, q.device)
    st = load_library().kda_chunk_intra(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), T, N, H,
        float(scale), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check("kda_chunk_intra", st)
    return workspace


def chunk_recurrence(workspace, T: int, N: int, H: int, initial_state=None, o=None,
                     final_state=None, output_final_state: bool = True, device=None):
    """Recurrence + output (kda_chunk_recurrence) on a workspace that
    chunk_intra has just filled; returns (o, final_state)."""
    torch = _torch()
    dev = workspace.device if device is None else device
    if o is None:
        o = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    if initial_state is not None:
        _expect(initial_state, "initial_state", torch.float32, (N, H, HEAD_DIM, HEAD_DIM))
    st = load_library().kda_chunk_recurrence(
        _ptr(initial_state), T, N, H, _ptr(o), _ptr(final_state), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check("kda_chunk_recurrence", st)
    return o, final_state
