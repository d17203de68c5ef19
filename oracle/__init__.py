"""KDA forward oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and it
never calls the GPU library; the two share no code.  The only common module
is the seeded input generator, which holds none of the method's arithmetic
(and which this package does not import: it takes plain arrays).

Contents
--------
``kda_fwd``        fp64 token-by-token recurrence (C, OpenMP over independent
                   (sequence, head) pairs).  The definition of the result.
``brute_force``    the same recurrence with explicit dense K x K transition
                   matrices M_t = (I - beta_t k_t k_t^T) Diag(exp g_t), for
                   tiny inputs (an independent check of ``kda_fwd``).
``decay_closed_form``  beta = 0: o_t = scale (q_t * exp(G_t))^T S_0 and
                   final = Diag(exp G_T) S_0 with G the in-sequence cumsum.
``linear_attention``   g = 0, orthonormal keys, S_0 = 0: causal linear
                   attention o_t = scale sum_{s<=t} beta_s (q_t.k_s) v_s.
``chunked_fwd``    the chunk (WY/UT) form in fp64 with BT-token chunks.
``chunk_terms``    the per-chunk quantities of that form (W, U, Aqk, ...).
``chunk_table``    per-chunk (sequence, local chunk, start, length, flags).
``strip_exponents``  largest |exponent| the subblock-midpoint strip factors
                   need, in nats.

Citations are to the pages: "KDA TPU report" is the Chinese-language report
on accelerating Kimi K3 KDA prefill on TPU (junyi.dev); "MI355X serving
post" is the Russian translation of the Kimi K3 on AMD Instinct article.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_double, P, P, ctypes.c_int32]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = ctypes.c_int32
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def widen(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exactly; fp32/fp64 pass through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x


def _f32(x):
    return np.ascontiguousarray(widen(x), dtype=np.float32)


def kda_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=None,
            heads: Optional[Sequence[int]] = None, nthreads: int = 0):
    """fp64 token recurrence.  Returns (o [T,H,dv] fp64, final [N,H,dk,dv]).

    ``q, k, v`` may be bf16 bit patterns (uint16) or float arrays; ``g``,
    ``beta`` and ``initial_state`` are float.  Every input enters the C
    recurrence as fp32 (then widened to fp64 there): bf16 and fp32 inputs
    pass exactly, while fp64 inputs (e.g. the output of ``prologue``) are
    rounded to fp32 first, a relative change of at most 2^-24 per element,
    far below the parity tolerances.  ``heads`` restricts the run to
    a subset of heads (the outputs then have len(heads) heads, in that
    order); heads are independent, so this is exact sampling.
    """
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    beta = _f32(beta)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    h0 = None if initial_state is None else _f32(initial_state)
    if heads is not None:
        idx = np.asarray(list(heads), dtype=np.int64)
        q, k, v, g = (np.ascontiguousarray(a[:, idx]) for a in (q, k, v, g))
        beta = np.ascontiguousarray(beta[:, idx])
        if h0 is not None:
            h0 = np.ascontiguousarray(h0[:, idx])
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _load().kda_oracle_fwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                                ptr(h0), ptr(cu), T, N, H, dk, dv,
                                float(scale), ptr(o), ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError(f"kda_oracle_fwd failed with code {rc}")
    return o, fin


def prologue(q, k, b, qk_eps=None):
    """The steps fused in front of the recurrence, in fp64 ("Kimi K3 Prefill
    PP16" notes, third throughput section, KDA switch table: beta from a bf16
    slice of the projection output through a sigmoid; KDA TPU report,
    section 8: q and k L2-normalised per token as the model does).  ``b`` holds the beta logits
    [T, H] (bf16 bit patterns or float); beta = 1 / (1 + exp(-b)).  With
    ``qk_eps`` given, each (token, head) row x of q and of k becomes
    x / sqrt(sum x^2 + qk_eps).  Returns (q, k, beta), fp64."""
    q, k, b = (widen(a).astype(np.float64) for a in (q, k, b))
    beta = 1.0 / (1.0 + np.exp(-b))
    if qk_eps is not None:
        q, k = _unit_rows(q, qk_eps), _unit_rows(k, qk_eps)
    return q, k, beta


def _unit_rows(x, eps):
    # x / sqrt(|x|^2 + eps); an all-zero row with eps = 0 (0/0) is read as
    # zero, the limit of the eps > 0 case
    d = np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)
    return np.divide(x, d, out=np.zeros_like(x), where=d > 0)


def gated_rmsnorm(x, gate, weight, eps, act="sigmoid"):
    """The gated RMSNorm that follows the operation, in fp64 ("Kimi K3
    Prefill PP16" notes, third throughput section, KDA switch table: the
    KDA output tail; RMSNorm as defined by Zhang and Sennrich, whom the KDA
    TPU report cites).  Per (token, head) row x of 128 channels, with gate
    row z and weight w [128]:  y = w * x / sqrt(mean(x^2) + eps) * act(z),
    act(z) = 1 / (1 + exp(-z)) ("sigmoid") or z / (1 + exp(-z)) ("silu").
    An all-zero row with eps = 0 (0/0) is read as zero.  ``x`` and ``gate``
    are [T, H, 128] (bf16 bit patterns or float); returns y, fp64."""
    x, z = widen(x).astype(np.float64), widen(gate).astype(np.float64)
    w = np.asarray(weight, dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-z))
    a = {"sigmoid": sig, "silu": z * sig}[act]
    d = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    xn = np.divide(x, d, out=np.zeros_like(x), where=d > 0)
    return w * xn * a


def _seq_ranges(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[s]), int(cu[s + 1])) for s in range(cu.shape[0] - 1)]


def brute_force(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=None):
    """Dense-transition form of the recurrence (KDA TPU report, section 2:
    the gated delta rule S_t = (I - beta k k^T) Diag(exp g) S_{t-1} +
    beta k v^T; o_t = scale S_t^T q_t).  Builds each K x K transition matrix
    explicitly.  Meant for T <= 32 and small heads."""
    q, k, v, g = (widen(a).astype(np.float64) for a in (q, k, v, g))
    beta = widen(beta).astype(np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = dk ** -0.5
    ranges = _seq_ranges(cu_seqlens)
    o = np.zeros((T, H, dv))
    fin = np.zeros((len(ranges), H, dk, dv))
    eye = np.eye(dk)
    for s, (a, b) in enumerate(ranges):
        for h in range(H):
            S = (np.zeros((dk, dv)) if initial_state is None else
                 widen(initial_state)[s, h].astype(np.float64))
            for t in range(a, b):
                kt = k[t, h][:, None]
                M = (eye - beta[t, h] * (kt @ kt.T)) @ np.diag(np.exp(g[t, h]))
                S = M @ S + beta[t, h] * (kt @ v[t, h][None, :])
                o[t, h] = scale * (S.T @ q[t, h])
            fin[s, h] = S
    return o, fin


def decay_closed_form(q, g, cu_seqlens, initial_state, scale=None):
    """beta = 0 freezes the write path: the state only decays.  With G_t the
    inclusive in-sequence cumsum of g, S_t = Diag(exp G_t) S_0, so
    o_t = scale (q_t * exp(G_t))^T S_0 and final = Diag(exp G_L) S_0."""
    q, g = widen(q).astype(np.float64), widen(g).astype(np.float64)
    S0 = widen(initial_state).astype(np.float64)
    T, H, dk = q.shape
    dv = S0.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    ranges = _seq_ranges(cu_seqlens)
    o = np.zeros((T, H, dv))
    fin = np.zeros((len(ranges), H, dk, dv))
    for s, (a, b) in enumerate(ranges):
        G = np.cumsum(g[a:b], axis=0)                      # [L, H, dk]
        for h in range(H):
            o[a:b, h] = scale * (q[a:b, h] * np.exp(G[:, h])) @ S0[s, h]
            Gl = G[-1, h] if b > a else np.zeros(dk)
            fin[s, h] = np.exp(Gl)[:, None] * S0[s, h]
    return o, fin


def linear_attention(q, k, v, beta, scale=None):
    """Causal linear attention with per-token write strength beta:
    o_t = scale * sum_{s<=t} beta_s (q_t . k_s) v_s, one sequence.  The
    delta rule reduces to this when g = 0, S_0 = 0 and the keys are
    orthonormal, because then S_{t-1}^T k_t = 0 for every t."""
    q, k, v = (widen(a).astype(np.float64) for a in (q, k, v))
    beta = widen(beta).astype(np.float64)
    T, H, dk = q.shape
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((T, H, v.shape[2]))
    for h in range(H):
        A = np.tril(q[:, h] @ k[:, h].T) * beta[None, :, h]
        o[:, h] = scale * A @ v[:, h]
    return o


def chunk_table(cu_seqlens, bt: int = 64):
    """Per-chunk bookkeeping of the flat packed-chunk grid (KDA TPU report,
    section 6.5): chunks are taken relative to each sequence's start, a
    sequence of length L has ceil(L/bt) chunks, and each chunk carries its
    sequence id, a start flag (load the entry state) and an end flag (write
    the final state).  Zero-length sequences own no chunk.

    Returns a list of dicts with keys seq, local, start (packed token
    offset), length, start_flag, end_flag, aligned_start (the offset the
    same chunk would have if each sequence were padded to a multiple of bt,
    which is chunk_id * bt, section 6.4)."""
    rows = []
    cid = 0
    for s, (a, b) in enumerate(_seq_ranges(cu_seqlens)):
        L = b - a
        n = (L + bt - 1) // bt
        for j in range(n):
            rows.append(dict(seq=s, local=j, start=a + j * bt,
                             length=min(bt, L - j * bt),
                             start_flag=int(j == 0), end_flag=int(j == n - 1),
                             aligned_start=cid * bt))
            cid += 1
    return rows


def chunk_terms(Q, K, V, g, beta, scale):
    """fp64 per-chunk quantities of the chunk form for one (sequence, head)
    chunk of n rows (KDA TPU report, section 4 for L, the inverse and the
    fused right-hand side [beta v | beta k 2^G]; section 6.2 for what the
    recurrence consumes).  With G the inclusive cumsum of g over the chunk
    and Gam = exp(G):

        L   = strictly-lower( diag(beta) (K*Gam)(K/Gam)^T )
        Tm  = (I + L)^-1
        U   = Tm (beta * V);   W = Tm (beta * K * Gam)
        Aqk = scale lower-incl-diag( (Q*Gam)(K/Gam)^T )
        qg  = scale Q * Gam;   kg = K * exp(G_{n-1} - G);   gamma = exp(G_{n-1})
    """
    Q, K, V, g = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, g))
    bet = np.asarray(beta, dtype=np.float64)
    n = Q.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Kp, Km = K * Gam, K * np.exp(-G)
    L = np.tril(bet[:, None] * (Kp @ Km.T), -1)
    Tm = np.linalg.solve(np.eye(n) + L, np.eye(n))
    return dict(G=G, L=L, T=Tm,
                U=Tm @ (bet[:, None] * V), W=Tm @ (bet[:, None] * Kp),
                Aqk=scale * np.tril((Q * Gam) @ Km.T), qg=scale * Q * Gam,
                kg=K * np.exp(G[-1][None, :] - G), gamma=np.exp(G[-1]))


def chunked_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=None,
                bt: int = 64):
    """The chunk (WY/UT) form of the same recurrence, fp64.

    Per sequence, head and chunk of n <= bt rows with entry state h (KDA TPU
    report, section 6.2 for the per-chunk dependencies), using
    ``chunk_terms``:

        v_new = U - W h
        o     = qg h + Aqk v_new
        h    <- Diag(gamma) h + kg^T v_new

    o reads the entry state h, never the updated one (section 6.2).
    """
    q, k, v, g = (widen(a).astype(np.float64) for a in (q, k, v, g))
    beta = widen(beta).astype(np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = dk ** -0.5
    ranges = _seq_ranges(cu_seqlens)
    o = np.zeros((T, H, dv))
    fin = np.zeros((len(ranges), H, dk, dv))
    for s, (a, b) in enumerate(ranges):
        for hh in range(H):
            hst = (np.zeros((dk, dv)) if initial_state is None else
                   widen(initial_state)[s, hh].astype(np.float64).copy())
            for c0 in range(a, b, bt):
                c1 = min(c0 + bt, b)
                t = chunk_terms(q[c0:c1, hh], k[c0:c1, hh], v[c0:c1, hh],
                                g[c0:c1, hh], beta[c0:c1, hh], scale)
                vnew = t["U"] - t["W"] @ hst
                o[c0:c1, hh] = t["qg"] @ hst + t["Aqk"] @ vnew
                hst = t["gamma"][:, None] * hst + t["kg"].T @ vnew
            fin[s, hh] = hst
    return o, fin


def strip_exponents(g_chunk, sb: int = 16, ref: int = 7):
    """Largest |exponent| (nats) the subblock-midpoint factors need inside
    one chunk (KDA TPU report, section 4: each SB=16 subblock is
    re-referenced at its midpoint so the bf16 strip-GEMM factors stay within
    (SB/2)|lower_bound|/ln 2 bits).  g_chunk: [n, dk] log-decays.  Row i of
    subblock b uses exp(G_i - G_r), r = min(sb*b + ref, n-1)."""
    g_chunk = np.asarray(g_chunk, dtype=np.float64)
    n = g_chunk.shape[0]
    G = np.cumsum(g_chunk, axis=0)
    worst = 0.0
    for b0 in range(0, n, sb):
        r = min(b0 + ref, n - 1)
        blk = G[b0:min(b0 + sb, n)]
        worst = max(worst, float(np.max(np.abs(blk - G[r][None, :]))))
    return worst


def max_abs_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)))


def rel_fro_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
