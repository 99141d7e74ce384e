"""Seeded synthetic inputs for the Qwen3 attention block.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the block's arithmetic, so both the CPU oracle (through the
tests) and the HIP path consume exactly the same values without sharing any
computation.

Shapes and value distributions follow the pages' model shapes:
  * Qwen3-0.6B: d=1024, 16 query heads, 8 KV heads, head dim 128
    (page "Assembling a large model from scratch", shape table; page
    "Qwen3 Architecture Layer-by-Layer", config values).
  * Qwen3-4B: d=2560, 32 query heads, 8 KV heads, head dim 128 (page
    "Hand-Writing a Vision-Language Model, Part 1", key numbers).
  * The worked example of page "Qwen 3 From Scratch": d=4096, 64 query heads,
    4 KV heads, head dim 128.

Recipe (std, not variance, for every normal draw):
  hidden ~ N(0,1); q/k/v/o weights ~ 0.02*N(0,1), no biases;
  q_norm / k_norm gains ~ 1 + 0.1*N(0,1).
Draw order from numpy's PCG64 seeded with ``1000 + config index``:
  X, Wq, Wk, Wv, Wo, gq, gk; for decode then the cache lengths.
bf16 workloads are drawn in float32 and rounded once to bf16
(round-to-nearest-even); the rounded values are what both sides see.
"""
from __future__ import annotations

import dataclasses
import numpy as np

EPS = 1e-6
ROPE_THETA = 1.0e6
D_HEAD = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str          # "prefill" or "decode"
    dtype: str         # "f32" or "bf16"
    d: int
    n_q: int
    n_kv: int
    dh: int = D_HEAD
    B: int = 1         # prefill batch, or number of decode sequences
    T: int = 1         # prefill length (1 for decode)
    len_lo: int = 0    # decode: cache length range (inclusive)
    len_hi: int = 0
    cap: int = 0       # decode: cache capacity in tokens

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    1: Workload(1, "qwen3-0.6B-tiny-prefill-f32-B1-T128", "prefill", "f32",
                d=1024, n_q=16, n_kv=8, B=1, T=128),
    2: Workload(2, "qwen3-0.6B-prefill-bf16-B2-T2048", "prefill", "bf16",
                d=1024, n_q=16, n_kv=8, B=2, T=2048),
    3: Workload(3, "qwen3-4B-prefill-bf16-B1-T4096", "prefill", "bf16",
                d=2560, n_q=32, n_kv=8, B=1, T=4096),
    4: Workload(4, "wide-gqa-64q4kv-prefill-bf16-B1-T8192", "prefill", "bf16",
                d=4096, n_q=64, n_kv=4, B=1, T=8192),
    5: Workload(5, "qwen3-0.6B-decode-bf16-N64-L1024..32768", "decode", "bf16",
                d=1024, n_q=16, n_kv=8, B=64, T=1, len_lo=1024, len_hi=32768,
                cap=32832),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly representable float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 draw to the storage dtype; returns float32 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(round_to_bf16_bits(x32))
    return np.ascontiguousarray(x32, dtype=np.float32)


def make_block_inputs(rng: np.random.Generator, *, rows: int, d: int, n_q: int,
                      n_kv: int, dh: int, dtype: str, hidden_shape=None) -> dict:
    """Hidden states, the four projection weights ([out, in]) and two gains."""
    f32 = np.float32
    hq, hkv = n_q * dh, n_kv * dh
    X = rng.standard_normal((rows, d), dtype=f32)
    Wq = 0.02 * rng.standard_normal((hq, d), dtype=f32)
    Wk = 0.02 * rng.standard_normal((hkv, d), dtype=f32)
    Wv = 0.02 * rng.standard_normal((hkv, d), dtype=f32)
    Wo = 0.02 * rng.standard_normal((d, hq), dtype=f32)
    gq = 1.0 + 0.1 * rng.standard_normal(dh, dtype=f32)
    gk = 1.0 + 0.1 * rng.standard_normal(dh, dtype=f32)
    out = dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, gq=gq, gk=gk)
    out = {k: _store(v.astype(f32), dtype) for k, v in out.items()}
    if hidden_shape is not None:
        out["X"] = out["X"].reshape(hidden_shape)
    return out


def prefill_inputs(w: Workload, *, seed: int | None = None, B: int | None = None,
                   T: int | None = None) -> dict:
    """Inputs of a prefill workload (optionally at a reduced B or T).

    Returns float32 arrays holding values exactly representable in the
    workload's dtype, plus int32 positions 0..T-1 per sequence.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = make_block_inputs(rng, rows=B * T, d=w.d, n_q=w.n_q, n_kv=w.n_kv,
                            dh=w.dh, dtype=w.dtype, hidden_shape=(B, T, w.d))
    out["positions"] = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    return out


def decode_inputs(w: Workload, *, seed: int | None = None, N: int | None = None,
                  len_lo: int | None = None, len_hi: int | None = None) -> dict:
    """Hidden states, weights and cache lengths of a decode workload.

    The cache contents are drawn separately (``decode_cache_host`` on the
    host, or on the device by the caller) because at full size they are
    several GB.
    """
    N = w.B if N is None else N
    lo = w.len_lo if len_lo is None else len_lo
    hi = w.len_hi if len_hi is None else len_hi
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = make_block_inputs(rng, rows=N, d=w.d, n_q=w.n_q, n_kv=w.n_kv,
                            dh=w.dh, dtype=w.dtype)
    out["lengths"] = rng.integers(lo, hi, size=N, endpoint=True).astype(np.int32)
    out["positions"] = out["lengths"].copy()
    return out


def decode_cache_host(w: Workload, lengths: np.ndarray, cap: int, *,
                      seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Host-drawn caches [N, n_kv, cap, dh] (float32 values of the dtype).

    Rows at and beyond each sequence's length are zero.  Entries ~ N(0,1);
    sequence s draws K then V from PCG64 seeded with (seed, s).
    """
    base = (w.seed if seed is None else seed) + 7919
    N = len(lengths)
    kc = np.zeros((N, w.n_kv, cap, w.dh), np.float32)
    vc = np.zeros_like(kc)
    for s, L in enumerate(lengths):
        rng = np.random.default_rng([base, s])
        kc[s, :, :L] = _store(rng.standard_normal((w.n_kv, L, w.dh), dtype=np.float32), w.dtype)
        vc[s, :, :L] = _store(rng.standard_normal((w.n_kv, L, w.dh), dtype=np.float32), w.dtype)
    return kc, vc
