"""Seeded synthetic inputs for KDA chunked prefill.

This module only draws random numbers and packs them into arrays.  It holds
none of the method's arithmetic: both the fp64 CPU oracle and the HIP path are
fed from here, and neither one imports the other.

Every workload is drawn from NumPy's PCG64 (``default_rng(seed)``) in a fixed
order -- lengths, q, k, v, g, beta, initial_state, pinned channels -- in fp32,
and the bf16 tensors are then rounded to nearest even.

Distributions (the pages' KDA prefill workloads, KDA TPU report, sections 1
and 8.1; the varlen packing follows its section 6.5 flat packed-chunk grid):

* q ~ N(0,1)/sqrt(128), k ~ N(0,1) L2-normalised per (token, head),
  v ~ N(0,1); all bf16 [T, H, 128] (token-major, model-native layout);
* g = -5 * sigmoid(N(0,1)), fp32 [T, H, 128], i.e. a log-decay in (-5, 0)
  (the bounded gate, lower_bound = -5);
* beta = sigmoid(N(0,1)), fp32 [T, H];
* initial_state fp32 [N, H, 128, 128]: zeros, or N(0, 0.1) (0.1 is the
  standard deviation) to stand in for a cached prefix;
* cu_seqlens int32 [N+1] for the packed varlen batch.

The ShareGPT-like length mix is a seeded lognormal stand-in (median 600,
sigma = sqrt(2 ln(108.20/28)), the mean/median ratio of the report's
ShareGPT-derived prompt lengths), clipped to [16, 8192] and nudged off
multiples of 64.  No dataset item is used.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DK = 128
DV = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    q: np.ndarray            # uint16 (bf16 bits) [T, H, DK]
    k: np.ndarray            # uint16 (bf16 bits) [T, H, DK]
    v: np.ndarray            # uint16 (bf16 bits) [T, H, DV]
    g: np.ndarray            # float32 [T, H, DK]
    beta: np.ndarray         # float32 [T, H]
    initial_state: Optional[np.ndarray]  # float32 [N, H, DK, DV] or None
    cu_seqlens: np.ndarray   # int32 [N+1]
    scale: float

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    def num_chunks(self, bt: int = 64) -> int:
        return int(sum((int(L) + bt - 1) // bt for L in self.lengths))

    def describe(self) -> dict:
        return {"workload": self.name, "seed": self.seed, "T": self.T,
                "N": self.N, "H": self.H, "K": DK, "V": DV,
                "chunks": self.num_chunks(),
                "initial_state": self.initial_state is not None}


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x, dtype=np.float32))).astype(np.float32)


def make_workload(name: str, lengths, H: int, seed: int, *,
                  h0: str = "zeros", pinned_fraction: float = 0.0,
                  scale: Optional[float] = None,
                  rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw one packed varlen workload.

    ``h0``: "none" (no initial_state tensor), "zeros" (explicit zero tensor)
    or "normal" (N(0, 0.1)).  ``pinned_fraction``: per head, that share of
    the key channels (rounded) has g = -5 exactly at every token.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    N = int(lengths.shape[0])
    T = int(lengths.sum())
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)

    q32 = _normal(rng, (T, H, DK)) * np.float32(1.0 / math.sqrt(DK))
    q = f32_to_bf16_bits(q32)
    del q32
    k32 = _normal(rng, (T, H, DK))
    nrm = np.sqrt(np.sum(k32.astype(np.float64) ** 2, axis=-1, keepdims=True))
    nrm = np.maximum(nrm, 1e-12).astype(np.float32)
    k = f32_to_bf16_bits(k32 / nrm)
    del k32, nrm
    v = f32_to_bf16_bits(_normal(rng, (T, H, DV)))
    g = (np.float32(-5.0) * _sigmoid(_normal(rng, (T, H, DK)))).astype(np.float32)
    beta = _sigmoid(_normal(rng, (T, H)))
    if h0 == "none":
        init = None
    elif h0 == "zeros":
        init = np.zeros((N, H, DK, DV), dtype=np.float32)
    elif h0 == "normal":
        init = (np.float32(0.1) * _normal(rng, (N, H, DK, DV))).astype(np.float32)
    else:
        raise ValueError(f"unknown h0 mode {h0!r}")
    if pinned_fraction > 0.0:
        npin = int(round(pinned_fraction * DK))
        for h in range(H):
            ch = rng.choice(DK, size=npin, replace=False)
            g[:, h, ch] = np.float32(-5.0)
    if scale is None:
        scale = 1.0 / math.sqrt(DK)
    return Workload(name=name, seed=seed, q=q, k=k, v=v, g=g, beta=beta,
                    initial_state=init, cu_seqlens=cu, scale=float(scale))


SHAREGPT_SIGMA = math.sqrt(2.0 * math.log(108.20 / 28.0))


def sharegpt_like_lengths(rng: np.random.Generator, n: int = 64,
                          median: float = 600.0, lo: int = 16,
                          hi: int = 8192) -> np.ndarray:
    L = np.rint(rng.lognormal(mean=math.log(median), sigma=SHAREGPT_SIGMA,
                              size=n)).astype(np.int64)
    L = np.clip(L, lo, hi)
    L = np.where(L % 64 == 0, L - 1, L)
    return L


# Named workloads.  Sizes: Tiny 1x256 tokens at H=2; Headline 4x2048 at H=16;
# Batch sweep Bx2048 at H=16 with a nonzero initial state; ShareGPT-like 64
# lognormal lengths at H=16; Long 1x16384 at H=96 with 10% of key channels
# pinned at the lower bound.
BATCH_SIZES = (1, 2, 4, 8, 16, 32, 64)


def tiny() -> Workload:
    return make_workload("tiny_T256_H2", [256], H=2, seed=0, h0="zeros")


def headline() -> Workload:
    return make_workload("headline_4x2048_H16", [2048] * 4, H=16, seed=1,
                         h0="zeros")


def batch(B: int) -> Workload:
    if B not in BATCH_SIZES:
        raise ValueError(f"batch size {B} not in {BATCH_SIZES}")
    return make_workload(f"batch_{B}x2048_H16", [2048] * B, H=16,
                         seed=100 + B, h0="normal")


def sharegpt_like(n: int = 64) -> Workload:
    rng = np.random.default_rng(2)
    L = sharegpt_like_lengths(rng, n)
    return make_workload(f"sharegpt_like_{n}seq_H16", L, H=16, seed=2,
                         h0="zeros", rng=rng)


def long_single() -> Workload:
    return make_workload("long_1x16384_H96", [16384], H=96, seed=3,
                         h0="normal", pinned_fraction=0.10)


def e2e_4x32k() -> Workload:
    """The end-to-end varlen shape of the KDA TPU report's correctness
    section: four packed sequences of 32,768 tokens (512-chunk chains), here
    at the headline's 16 heads with a cached-prefix state ~N(0, 0.1)."""
    return make_workload("e2e_4x32768_H16", [32768] * 4, H=16, seed=4, h0="normal")


def decode_step(users: int, tokens: int, H: int) -> Workload:
    """A decode step (tokens = 1) or a speculative-verification window
    (tokens = 4) for `users` sequences with cached states, ~N(0, 0.1)."""
    return make_workload(f"decode_{users}x{tokens}_H{H}", [tokens] * users, H=H,
                         seed=200 + 10 * tokens + users % 10, h0="normal")


def raw_prologue_inputs(w: Workload, seed: int, pre: int = 5, post: int = 3):
    """Inputs for the fused-prologue entry points, next to workload ``w``: q
    and k drawn N(0,1) (not normalised; k scaled by 4 so that its rows are
    far from unit norm) and beta logits N(0,1), all bf16, the logits as
    columns [pre, pre + H) of a [T, pre + H + post] row-major tensor (the
    strided slice of a projection output).  Returns (q, k, b_full, pre) as
    bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    T, H = w.T, w.H
    q = f32_to_bf16_bits(_normal(rng, (T, H, DK)))
    k = f32_to_bf16_bits(4.0 * _normal(rng, (T, H, DK)))
    b = f32_to_bf16_bits(_normal(rng, (T, pre + H + post)))
    return q, k, b, pre


def small(lengths, H: int = 2, seed: int = 7, h0: str = "normal",
          pinned_fraction: float = 0.0, scale: Optional[float] = None) -> Workload:
    """A small ad-hoc workload for parity and edge-case tests."""
    return make_workload(f"small_{'-'.join(str(int(x)) for x in lengths)}_H{H}",
                         lengths, H=H, seed=seed, h0=h0,
                         pinned_fraction=pinned_fraction, scale=scale)


def by_name(name: str) -> Workload:
    if name == "tiny":
        return tiny()
    if name == "headline":
        return headline()
    if name.startswith("batch"):
        return batch(int(name[len("batch"):]))
    if name == "sharegpt":
        return sharegpt_like()
    if name == "long":
        return long_single()
    if name == "e2e4x32k":
        return e2e_4x32k()
    if name.startswith("decode"):  # decodeUxT_hH, e.g. decode16x1_h12
        ut, hh = name[len("decode"):].split("_h")
        u, t = ut.split("x")
        return decode_step(int(u), int(t), int(hh))
    raise ValueError(f"unknown workload {name!r}")


def algorithmic_bytes(w: Workload) -> int:
    """Bytes the method must move: q,k,v bf16 + g fp32 + beta fp32 read and
    o bf16 written per (token, head); final_state fp32 written per
    (sequence, head); initial_state read when a tensor is passed."""
    per_tok_head = 3 * DK * 2 + DK * 4 + 4 + DV * 2
    b = w.T * w.H * per_tok_head + w.N * w.H * DK * DV * 4
    if w.initial_state is not None:
        b += w.N * w.H * DK * DV * 4
    return int(b)


def algorithmic_flops(w: Workload) -> int:
    """FLOP of the chunked method (BT=64) per (token, head): 154,624."""
    return int(w.T * w.H * 154624)


def to_torch(w: Workload, device="cuda") -> dict:
    """Device copies of a workload's tensors (bf16 stays bit-identical)."""
    import torch

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(
            torch.bfloat16)

    def f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    return {"q": bf(w.q), "k": bf(w.k), "v": bf(w.v), "g": f32(w.g), "beta": f32(w.beta),
            "cu_seqlens": torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(device),
            "initial_state": None if w.initial_state is None else f32(w.initial_state)}


def bf16_tensor_to_f32(t) -> np.ndarray:
    """A bf16 torch tensor (any device) as exact fp32 numpy values."""
    import torch
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16).astype(
        np.uint32).__lshift__(16).view(np.float32)
