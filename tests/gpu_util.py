"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP block
through the C ABI binding, compare against the oracle with the pass bar."""
from __future__ import annotations

import sys

import numpy as np

import qwen3_gqa_attention_amd as q3
from workloads import EPS, ROPE_THETA

# Pass bar: fp32 max abs error <= 1e-4; bf16 max abs <= 2e-2 and rel L2 <= 1e-2.
# The bf16 absolute bar is stated for outputs of magnitude up to 4; above that
# the bf16 output format alone exceeds it (half an ulp is 2^-5 = 0.031 for
# |y| in [8, 16): the exact result of the 64-head / 4-KV-head workload,
# max|Y| = 8.95, rounded once to bf16 is already 0.0216 away).  So the
# absolute bar scales with the reference's magnitude beyond 4:
#   max abs <= 2e-2 * max(1, max|ref| / 4).
TOL = {"f32": dict(max_abs=1e-4, rel_l2=None, scale_above=None),
       "bf16": dict(max_abs=2e-2, rel_l2=1e-2, scale_above=4.0)}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(a, dtype):
    """Host float32 values (already representable in dtype) -> device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch_dtype(dtype)) if dtype != "f32" else t


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def block_from_inputs(inp, n_q, n_kv, dtype, **kw) -> q3.Qwen3Attention:
    """A handle over the workload's weights; kw: further Qwen3Attention options."""
    return q3.Qwen3Attention(dev(inp["Wq"], dtype), dev(inp["Wk"], dtype), dev(inp["Wv"], dtype),
                             dev(inp["Wo"], dtype), dev(inp["gq"], dtype), dev(inp["gk"], dtype),
                             n_q=n_q, n_kv=n_kv, eps=EPS, rope_theta=ROPE_THETA, **kw)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def max_abs_bar(ref, dtype) -> float:
    tol = TOL[dtype]
    if tol["scale_above"] is None:
        return tol["max_abs"]
    peak = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    return tol["max_abs"] * max(1.0, peak / tol["scale_above"])


def assert_close(got, ref, dtype, what):
    max_abs, rel = errors(got, ref)
    tol = TOL[dtype]
    bar = max_abs_bar(ref, dtype)
    print(f"  {what}: max_abs={max_abs:.3e} (bar {bar:.3e}) rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert max_abs <= bar, f"{what}: max abs {max_abs:.3e} > {bar:.3e}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: rel L2 {rel:.3e} > {tol['rel_l2']}"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_paged(kc, vc, lengths, bs, *, seed=0, spare=3):
    """Scatter contiguous host caches [S, n_kv, cap, dh] into pools
    [num_blocks, n_kv, bs, dh] under a random block table covering lengths[s]
    (+ the slots the call writes); unused blocks hold NaN."""
    S, n_kv, cap, dh = kc.shape
    need = [(int(L) + bs - 1) // bs for L in lengths]
    mb = max(max(need), 1)
    nb = sum(need) + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    table = np.zeros((S, mb), np.int32)
    kp = np.full((nb, n_kv, bs, dh), np.nan, np.float32)
    vp = np.full_like(kp, np.nan)
    nxt = 0
    for s in range(S):
        for i in range(need[s]):
            blk = int(perm[nxt]); nxt += 1
            table[s, i] = blk
            lo, hi = i * bs, min((i + 1) * bs, cap)
            kp[blk, :, : hi - lo] = kc[s, :, lo:hi]
            vp[blk, :, : hi - lo] = vc[s, :, lo:hi]
        table[s, need[s]:] = table[s, max(need[s] - 1, 0)]   # never reached
    return kp, vp, table


def from_paged(pool, table, s, L):
    bs = pool.shape[2]
    rows = [pool[table[s, p // bs], :, p % bs] for p in range(L)]
    return np.stack(rows, axis=1) if rows else np.zeros((pool.shape[1], 0, pool.shape[3]))
