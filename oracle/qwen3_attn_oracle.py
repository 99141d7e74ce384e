"""CPU oracle for the Qwen3 self-attention block -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it imports nothing
from the product path: the two share no code.

It is the plain, slow, obviously correct definition of what the block
computes, in float64 by default (a ``dtype`` argument runs the same code in
float32 for the CPU timing baseline).  Library primitives (a matmul, exp,
sqrt, cos/sin) serve as steps; there is no blocking, fusion or reordering
beyond the definition.  Every function cites the passage it follows.  Pages
are cited by title and section:

  [VLM1]  "Hand-Writing a Vision-Language Model, Part 1: Qwen3-4B's Attention
          Stack" (scott-k.dev)
  [BUILD] "Assembling a large model from scratch" (AI-infra handbook,
          anrans.github.io)
  [FROM]  "Qwen 3 From Scratch" (fanout.sharathchenna.top)
  [ANAT]  "Learning 10 - what each tensor is, and how we know"
          (curtisalexander.github.io)
  [HF]    "Qwen3 Architecture Layer-by-Layer - Reading the HuggingFace
          Implementation" (supercharleszhu.github.io)

Readings where the pages are silent or disagree (each also listed in the
design notes):
  * RoPE pairs dimension i with i + dh/2 (the rotate_half construction in all
    three code listings), not adjacent dimensions as one sentence of [HF]
    "apply_rotary_pos_emb" says.
  * The RoPE base is the ``theta`` argument (1e6 for Qwen3).
  * The attention is causal by token index: a query that is the i-th of T new
    tokens over S keys sees keys 0 .. S-T+i ([BUILD] "The complete code",
    the tril(diagonal=S-T) mask).  Positions drive RoPE only.
  * A sliding-window layer of window W ([HF] "Layer 1 - Qwen3Model" and
    "Layer 3 - Qwen3Attention": the per-layer sliding_window attribute and
    the sliding-window causal mask) keeps the W most recent keys, the query's
    own included: query i of the tril mask above sees keys j with
    S-T+i-W < j <= S-T+i.  The cache still holds every key.
  * cos/sin are not multiplied by any attention_scaling factor (default RoPE).
  * eps sits inside the square root; a zero head vector maps to zero.
  * The oracle is the exact math on the given inputs; it does not emulate the
    intermediate bf16 roundings of the PyTorch listings.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against closed forms, invariants, brute force and torch's own CPU routines.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# Projections -- [VLM1] "Attention: Grouped-Query Attention"; [BUILD] "The
# complete code" (Attention.forward); [ANAT] "Part 2 - tensor by tensor"
# (weights stored [out, in]); [HF] "Layer 3 - Qwen3Attention" (no biases).
# ----------------------------------------------------------------------------
def linear(x: np.ndarray, w: np.ndarray, dtype=np.float64) -> np.ndarray:
    """y = x @ w^T for a weight stored [out, in]; no bias."""
    return np.asarray(x, dtype) @ np.asarray(w, dtype).T


def split_heads(u: np.ndarray, dh: int) -> np.ndarray:
    """[..., heads*dh] -> [..., heads, dh] (head h owns columns h*dh .. h*dh+dh-1)."""
    return u.reshape(*u.shape[:-1], u.shape[-1] // dh, dh)


def merge_heads(a: np.ndarray) -> np.ndarray:
    """[..., heads, dh] -> [..., heads*dh], the inverse of split_heads."""
    return a.reshape(*a.shape[:-2], a.shape[-2] * a.shape[-1])


# ----------------------------------------------------------------------------
# QK-Norm -- [VLM1] "RMSNorm"; [BUILD] "The complete code" (RMSNorm);
# [FROM] "The idea" and "In code"; [HF] "Primitives - Qwen3RMSNorm".
# ----------------------------------------------------------------------------
def rms_norm(u: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * u / sqrt(mean(u^2) + eps) over the last axis (no mean subtraction)."""
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return np.asarray(g, u.dtype) * (u / np.sqrt(ms + eps))


# ----------------------------------------------------------------------------
# RoPE -- [VLM1] "RotaryEmbedding (RoPE)"; [BUILD] "The complete code"
# (rope_cos_sin, rotate_half, apply_rope); [HF] "apply_rotary_pos_emb" and
# "Primitives - Qwen3RotaryEmbedding" (inv_freq formula).
# ----------------------------------------------------------------------------
def rope_inv_freq(dh: int, theta: float, dtype=np.float64) -> np.ndarray:
    """omega_i = theta^(-2i/dh), i = 0 .. dh/2-1."""
    i = np.arange(dh // 2, dtype=np.float64)
    return (theta ** (-2.0 * i / dh)).astype(dtype)


def rope(u: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate head vectors u[..., T, H, dh] by their token positions[..., T].

    Dimension i (< dh/2) and i + dh/2 form one 2-D pair rotated by the angle
    p * omega_i:  out_i = u_i cos - u_{i+dh/2} sin,
                  out_{i+dh/2} = u_{i+dh/2} cos + u_i sin.
    """
    dh = u.shape[-1]
    half = dh // 2
    omega = rope_inv_freq(dh, theta, u.dtype)
    ang = np.asarray(positions, u.dtype)[..., None, None] * omega   # [..., T, 1, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ----------------------------------------------------------------------------
# Causal grouped-query attention -- [VLM1] "Attention: Grouped-Query
# Attention" (repeat_kv, query head h uses KV head h // n_rep); [BUILD] "The
# complete code" (repeat_interleave, tril(diagonal=S-T) mask, fp32 softmax);
# [FROM] "Worked example" (scores divided by sqrt(dh)); [HF] "The attention
# dispatch".
# ----------------------------------------------------------------------------
def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis; -inf entries get probability 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window=None) -> np.ndarray:
    """Causal GQA for one sequence.

    q: [T, n_q, dh] queries (the last T of S positions);
    k, v: [S, n_kv, dh] keys/values for positions 0 .. S-1 (S >= T).
    Returns [T, n_q, dh].  Query head h reads KV head h // (n_q // n_kv);
    query i sees keys j <= S - T + i, and with a sliding window W (None or
    0: no window) only those with j > S - T + i - W.
    """
    T, n_q, dh = q.shape
    S, n_kv, _ = k.shape
    n_rep = n_q // n_kv
    last = (S - T + np.arange(T))[:, None]                                  # [T, 1]
    visible = np.arange(S)[None, :] <= last                                 # [T, S]
    if window:
        visible &= np.arange(S)[None, :] > last - window
    out = np.empty_like(q)
    for h in range(n_q):
        g = h // n_rep
        scores = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(dh)
        scores = np.where(visible, scores, -np.inf)
        out[:, h, :] = softmax(scores) @ v[:, g, :]
    return out


# ----------------------------------------------------------------------------
# The whole block.
# ----------------------------------------------------------------------------
def project_norm_rope(x, wq, wk, wv, gq, gk, positions, *, n_q, n_kv, dh, eps,
                      theta, dtype=np.float64):
    """Steps before attention for tokens x[..., T, d] at positions[..., T].

    Returns (q~, k~, v) with shapes [..., T, heads, dh]: projections, per-head
    RMSNorm of q and k with their own gains, then RoPE on q and k only ([VLM1]
    "Attention: Grouped-Query Attention", order of operations; [HF]
    "Forward: the four-step dance").
    """
    q = split_heads(linear(x, wq, dtype), dh)
    k = split_heads(linear(x, wk, dtype), dh)
    v = split_heads(linear(x, wv, dtype), dh)
    assert q.shape[-2] == n_q and k.shape[-2] == n_kv
    q = rms_norm(q, np.asarray(gq, dtype), eps)
    k = rms_norm(k, np.asarray(gk, dtype), eps)
    q = rope(q, positions, theta)
    k = rope(k, positions, theta)
    return q, k, v


def prefill(x, wq, wk, wv, wo, gq, gk, positions, *, n_q, n_kv, dh=128,
            eps=1e-6, theta=1e6, dtype=np.float64, window=None) -> dict:
    """Block forward over B sequences of T new tokens with an empty cache
    (window: the sliding window of the layer, None for full attention).

    x: [B, T, d]; positions: [B, T].  Returns a dict with
      Y  [B, T, d]        block output,
      Q  [B, T, n_q, dh]  post-norm post-RoPE queries,
      Kc [B, n_kv, T, dh] post-norm post-RoPE keys in cache layout,
      Vc [B, n_kv, T, dh] values in cache layout,
      A  [B, T, n_q*dh]   merged attention output (o_proj input).
    """
    q, k, v = project_norm_rope(x, wq, wk, wv, gq, gk, positions, n_q=n_q,
                                n_kv=n_kv, dh=dh, eps=eps, theta=theta, dtype=dtype)
    B = q.shape[0]
    a = np.stack([gqa_attention(q[b], k[b], v[b], window) for b in range(B)])
    A = merge_heads(a)
    Y = linear(A, wo, dtype)
    return dict(Y=Y, Q=q, Kc=np.transpose(k, (0, 2, 1, 3)),
                Vc=np.transpose(v, (0, 2, 1, 3)), A=A)


def decode(x, wq, wk, wv, wo, gq, gk, positions, k_cache, v_cache, *, n_q, n_kv,
           dh=128, eps=1e-6, theta=1e6, dtype=np.float64, window=None) -> dict:
    """One new token per sequence on top of an existing cache.

    x: [N, d]; positions[s] = L_s, the number of cached tokens of sequence s;
    k_cache, v_cache: [N, n_kv, >=L_s, dh] holding post-norm post-RoPE keys
    and values of positions 0 .. L_s-1.  The new token sits at position L_s
    and sees all L_s + 1 keys ([BUILD] "The complete code": the cache update
    then the tril(diagonal=S-T) mask with T=1; the generate loop), or the
    last `window` of them.
    Returns Y [N, d], the new k~ and v [N, n_kv, dh], and A [N, n_q*dh].
    """
    N = x.shape[0]
    pos = np.asarray(positions).reshape(N, 1)
    q, k, v = project_norm_rope(np.asarray(x)[:, None, :], wq, wk, wv, gq, gk, pos,
                                n_q=n_q, n_kv=n_kv, dh=dh, eps=eps, theta=theta,
                                dtype=dtype)
    A = np.empty((N, n_q * dh), dtype)
    for s in range(N):
        L = int(pos[s, 0])
        ks = np.concatenate([np.asarray(k_cache[s][:, :L], dtype).transpose(1, 0, 2), k[s]], axis=0)
        vs = np.concatenate([np.asarray(v_cache[s][:, :L], dtype).transpose(1, 0, 2), v[s]], axis=0)
        A[s] = merge_heads(gqa_attention(q[s], ks, vs, window))[0]
    Y = linear(A, wo, dtype)
    return dict(Y=Y, k_new=k[:, 0], v_new=v[:, 0], A=A, Q=q[:, 0])


def prefill_chunk(x, wq, wk, wv, wo, gq, gk, positions, past_len, k_cache, v_cache, *,
                  n_q, n_kv, dh=128, eps=1e-6, theta=1e6, dtype=np.float64,
                  window=None) -> dict:
    """A chunk of T new tokens per sequence appended to a non-empty cache.

    x: [B, T, d]; positions: [B, T]; past_len[b] = P_b cached tokens;
    k_cache, v_cache: [B, n_kv, >=P_b, dh] holding post-norm post-RoPE keys
    and values of the first P_b tokens.  The KV cache appends the chunk's keys
    and values after them, and chunk token t (key P_b + t) sees keys
    0 .. P_b + t: gqa_attention with S = P_b + T ([BUILD] "The complete code":
    KVCache.update, then the tril(diagonal=S-T) mask).  Returns Y [B, T, d],
    Q [B, T, n_q, dh], the chunk's Kc / Vc [B, n_kv, T, dh] (cache layout) and
    A [B, T, n_q*dh].
    """
    q, k, v = project_norm_rope(x, wq, wk, wv, gq, gk, positions, n_q=n_q,
                                n_kv=n_kv, dh=dh, eps=eps, theta=theta, dtype=dtype)
    B = q.shape[0]
    out = []
    for b in range(B):
        P = int(past_len[b])
        ks = np.concatenate([np.asarray(k_cache[b][:, :P], dtype).transpose(1, 0, 2), k[b]], axis=0)
        vs = np.concatenate([np.asarray(v_cache[b][:, :P], dtype).transpose(1, 0, 2), v[b]], axis=0)
        out.append(gqa_attention(q[b], ks, vs, window))
    A = merge_heads(np.stack(out))
    Y = linear(A, wo, dtype)
    return dict(Y=Y, Q=q, Kc=np.transpose(k, (0, 2, 1, 3)),
                Vc=np.transpose(v, (0, 2, 1, 3)), A=A)


def prefill_residual(x, g_in, wq, wk, wv, wo, gq, gk, positions, *, n_q, n_kv, dh=128,
                     eps=1e-6, theta=1e6, dtype=np.float64, window=None) -> dict:
    """The attention half of a decoder layer: x + block(RMSNorm(x) * g_in)
    ([BUILD] "The complete code": input_layernorm, self-attention, residual
    add).  Same arguments as prefill plus the input-norm gain g_in [d];
    returns prefill's dict with Y replaced by the layer output."""
    xd = np.asarray(x, dtype)
    out = prefill(rms_norm(xd, g_in, eps), wq, wk, wv, wo, gq, gk, positions, n_q=n_q,
                  n_kv=n_kv, dh=dh, eps=eps, theta=theta, dtype=dtype, window=window)
    out["Y"] = xd + out["Y"]
    return out


def decode_residual(x, g_in, wq, wk, wv, wo, gq, gk, positions, k_cache, v_cache, *, n_q,
                    n_kv, dh=128, eps=1e-6, theta=1e6, dtype=np.float64, window=None) -> dict:
    """decode() with the input RMSNorm and the residual add around the block."""
    xd = np.asarray(x, dtype)
    out = decode(rms_norm(xd, g_in, eps), wq, wk, wv, wo, gq, gk, positions, k_cache, v_cache,
                 n_q=n_q, n_kv=n_kv, dh=dh, eps=eps, theta=theta, dtype=dtype, window=window)
    out["Y"] = xd + out["Y"]
    return out


def prefill_rows(x, wq, wk, wv, wo, gq, gk, positions, rows, *, n_q, n_kv, dh=128,
                 eps=1e-6, theta=1e6, dtype=np.float64, window=None) -> dict:
    """The prefill output at selected tokens only, for full-size checks.

    rows: list of (b, t).  Same definition as ``prefill``: keys/values of
    tokens 0..t of sequence b, the query of token t, causal GQA over them,
    then o_proj.  Returns Y [len(rows), d], A [len(rows), n_q*dh], and the
    post-norm post-RoPE keys/values of every token up to the largest
    sampled t of each sampled sequence: Kc[b], Vc[b] as [n_kv, t_max+1, dh].
    """
    seqs = sorted({b for b, _ in rows})
    kv = {}
    for b in seqs:
        tmax = max(t for bb, t in rows if bb == b)
        # keys/values of the needed prefix; the query projection is not needed here
        _, k, v = project_norm_rope(x[b, :tmax + 1], wq[:0], wk, wv, gq, gk,
                                    positions[b, :tmax + 1], n_q=0, n_kv=n_kv, dh=dh,
                                    eps=eps, theta=theta, dtype=dtype)
        kv[b] = (k, v)
    A = np.empty((len(rows), n_q * dh), dtype)
    for i, (b, t) in enumerate(rows):
        q, _, _ = project_norm_rope(x[b, t:t + 1], wq, wk[:0], wv[:0], gq, gk,
                                    positions[b, t:t + 1], n_q=n_q, n_kv=0, dh=dh,
                                    eps=eps, theta=theta, dtype=dtype)
        k, v = kv[b]
        A[i] = merge_heads(gqa_attention(q, k[:t + 1], v[:t + 1], window))[0]
    Y = linear(A, wo, dtype)
    return dict(Y=Y, A=A, Kc={b: np.transpose(kv[b][0], (1, 0, 2)) for b in seqs},
                Vc={b: np.transpose(kv[b][1], (1, 0, 2)) for b in seqs})
