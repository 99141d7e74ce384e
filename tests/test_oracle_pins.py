"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage or the closed form it checks.  None of them
re-types the oracle's formula: they use hand-worked values, invariants,
closed forms, brute force, or torch's own CPU routines (rms_norm and
scaled_dot_product_attention in float64), which the oracle does not call.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import WORKLOADS, prefill_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_block(seed, *, B=1, T=9, d=64, n_q=4, n_kv=2, dh=16, gain=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, d))
    wq = 0.1 * rng.standard_normal((n_q * dh, d))
    wk = 0.1 * rng.standard_normal((n_kv * dh, d))
    wv = 0.1 * rng.standard_normal((n_kv * dh, d))
    wo = 0.1 * rng.standard_normal((d, n_q * dh))
    gq = 1 + 0.1 * rng.standard_normal(dh) if gain else np.ones(dh)
    gk = 1 + 0.1 * rng.standard_normal(dh) if gain else np.ones(dh)
    pos = np.tile(np.arange(T), (B, 1))
    return dict(x=x, wq=wq, wk=wk, wv=wv, wo=wo, gq=gq, gk=gk, positions=pos,
                n_q=n_q, n_kv=n_kv, dh=dh)


def run_prefill(p, **kw):
    args = {k: p[k] for k in ("x", "wq", "wk", "wv", "wo", "gq", "gk", "positions")}
    return oracle.prefill(**args, n_q=p["n_q"], n_kv=p["n_kv"], dh=p["dh"], **kw)


# --- RoPE -------------------------------------------------------------------
def test_rope_inv_freq_endpoints_match_printed_formula():
    g = golden("rope_inv_freq_qwen3.json")
    w = oracle.rope_inv_freq(g["head_dim"], g["theta"])
    assert w.shape == (g["count"],)
    for i, v in g["values"].items():
        assert w[int(i)] == pytest.approx(v, rel=1e-14)
    assert np.all(np.diff(w) < 0)


def test_rope_hand_worked_rotate_half_example():
    g = golden("rope_rotate_half_example.json")
    for c in g["cases"]:
        u = np.array(c["x"], np.float64).reshape(1, 1, g["head_dim"])
        out = oracle.rope(u, np.array([c["position"]]), g["theta"])
        np.testing.assert_allclose(out.ravel(), c["out"], rtol=0, atol=1e-15)


def test_rope_preserves_head_norm():
    # Rotation keeps the norm of every head vector (From Scratch, "The idea").
    rng = np.random.default_rng(1)
    u = rng.standard_normal((3, 50, 4, 128))
    pos = rng.integers(0, 40960, size=(3, 50))
    r = oracle.rope(u, pos, 1e6)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    # <R_m q, R_n k> == <R_{m+c} q, R_{n+c} k> (VLM1, "RotaryEmbedding").
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for m, n, c in [(5, 3, 45), (50, 48, 1000), (4000, 17, 3333), (0, 0, 12345)]:
        s0 = np.sum(oracle.rope(q, np.array([m]), 1e6) * oracle.rope(k, np.array([n]), 1e6))
        s1 = np.sum(oracle.rope(q, np.array([m + c]), 1e6) * oracle.rope(k, np.array([n + c]), 1e6))
        assert s0 == pytest.approx(s1, rel=1e-9, abs=1e-9)


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((2, 7, 3, 128))
    np.testing.assert_array_equal(oracle.rope(u, np.zeros((2, 7)), 1e6), u)


# --- QK-Norm ------------------------------------------------------------------
def test_qk_norm_unit_rms_before_gain():
    # Each head has RMS sqrt(m/(m+eps)) before the gain (From Scratch, "Worked example").
    rng = np.random.default_rng(4)
    u = 0.3 * rng.standard_normal((5, 6, 128))
    eps = 1e-6
    r = oracle.rms_norm(u, np.ones(128), eps)
    ms = np.mean(u * u, axis=-1)
    rms = np.sqrt(np.mean(r * r, axis=-1))
    np.testing.assert_allclose(rms, np.sqrt(ms / (ms + eps)), rtol=1e-13)
    assert np.all(np.abs(rms - 1) < 1e-4)


def test_qk_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((4, 9, 128))
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = F.rms_norm(torch.from_numpy(u), (128,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(u, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_qk_norm_zero_vector_maps_to_zero():
    assert np.all(oracle.rms_norm(np.zeros((2, 128)), np.ones(128), 1e-6) == 0)


# --- attention core ---------------------------------------------------------------
@pytest.mark.parametrize("n_q,n_kv,T,S", [(4, 4, 10, 10), (8, 2, 13, 13), (16, 1, 5, 5),
                                          (6, 3, 4, 11), (2, 2, 1, 7)])
def test_attention_matches_torch_sdpa(n_q, n_kv, T, S):
    # Causal GQA == torch's SDPA with enable_gqa (repeat_kv semantics: h // n_rep).
    # S > T is the cached case: bottom-right aligned causal mask (tril(diagonal=S-T)).
    rng = np.random.default_rng(n_q * 100 + T)
    q = rng.standard_normal((T, n_q, 32))
    k = rng.standard_normal((S, n_kv, 32))
    v = rng.standard_normal((S, n_kv, 32))
    ours = oracle.gqa_attention(q, k, v)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2)[None] for a in (q, k, v))
    mask = torch.ones(T, S, dtype=torch.bool).tril(diagonal=S - T)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    np.testing.assert_allclose(ours, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def brute_force_attention(q, k, v):
    T, n_q, dh = q.shape
    S, n_kv, _ = k.shape
    out = np.zeros_like(q)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        for i in range(T):
            ws = []
            for j in range(S):
                if j <= S - T + i:
                    ws.append(sum(q[i, h, c] * k[j, g, c] for c in range(dh)) / dh ** 0.5)
            mx = max(ws)
            es = [np.exp(w - mx) for w in ws]
            tot = sum(es)
            for c in range(dh):
                out[i, h, c] = sum(es[j] / tot * v[j, g, c] for j in range(len(es)))
    return out


@pytest.mark.parametrize("T,S", [(1, 1), (5, 5), (8, 8), (3, 8)])
def test_attention_brute_force_tiny(T, S):
    rng = np.random.default_rng(T * 10 + S)
    q = rng.standard_normal((T, 4, 8))
    k = rng.standard_normal((S, 2, 8))
    v = rng.standard_normal((S, 2, 8))
    np.testing.assert_allclose(oracle.gqa_attention(q, k, v), brute_force_attention(q, k, v),
                               rtol=1e-12, atol=1e-12)


def test_chunked_lse_merge_equals_unsplit_softmax():
    # Split-K decode identity: per-chunk (max, sum, weighted sum) merged with
    # log-sum-exp weights gives the unsplit softmax-weighted sum.
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 16))
    k = rng.standard_normal((101, 1, 16))
    v = rng.standard_normal((101, 1, 16))
    full = oracle.gqa_attention(q, k, v)[0]
    parts = []
    for c0 in range(0, 101, 17):
        s = np.einsum("hd,jd->hj", q[0], k[c0:c0 + 17, 0]) / 4.0
        m = s.max(-1)
        e = np.exp(s - m[:, None])
        parts.append((m, e.sum(-1), e @ v[c0:c0 + 17, 0]))
    M = np.max([p[0] for p in parts], axis=0)
    L = sum(np.exp(p[0] - M) * p[1] for p in parts)
    O = sum(np.exp(p[0] - M)[:, None] * p[2] for p in parts) / L[:, None]
    np.testing.assert_allclose(O, full, rtol=1e-12, atol=1e-13)


# --- whole block --------------------------------------------------------------
def test_zero_query_weight_gives_prefix_mean_of_values():
    # Wq = 0 -> q~ = 0 -> uniform weights over the visible keys: A_t = mean(V_0..t).
    p = rand_block(7, B=2, T=11)
    p["wq"] = np.zeros_like(p["wq"])
    out = run_prefill(p)
    v = (p["x"] @ p["wv"].T).reshape(2, 11, p["n_kv"], p["dh"])
    pref = np.cumsum(v, axis=1) / np.arange(1, 12)[None, :, None, None]
    rep = p["n_q"] // p["n_kv"]
    for h in range(p["n_q"]):
        np.testing.assert_allclose(out["A"][..., h * 16:(h + 1) * 16], pref[:, :, h // rep],
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("which", ["gq", "gk"])
def test_zero_gain_gives_prefix_mean_of_values(which):
    # A zero q_norm (or k_norm) gain zeroes q~ (or k~): scores are uniform.
    # Pins which gain belongs to which side.
    p = rand_block(8, B=1, T=7)
    p[which] = np.zeros(p["dh"])
    out = run_prefill(p)
    v = (p["x"] @ p["wv"].T).reshape(1, 7, p["n_kv"], p["dh"])
    pref = np.cumsum(v, axis=1) / np.arange(1, 8)[None, :, None, None]
    rep = p["n_q"] // p["n_kv"]
    for h in range(p["n_q"]):
        np.testing.assert_allclose(out["A"][..., h * 16:(h + 1) * 16], pref[:, :, h // rep],
                                   rtol=1e-12, atol=1e-13)


def test_first_row_is_o_proj_of_own_values():
    # Token 0 sees only itself: Y_0 = Wo . concat_h V_{0, h // n_rep}.  Pins the
    # GQA map, the head merge order and Wo's [out, in] orientation.
    p = rand_block(9, B=2, T=5, d=48, n_q=6, n_kv=3)
    out = run_prefill(p)
    v0 = (p["x"][:, 0] @ p["wv"].T).reshape(2, 3, 16)
    cat = np.concatenate([v0[:, h // 2] for h in range(6)], axis=-1)
    np.testing.assert_allclose(out["Y"][:, 0], cat @ p["wo"].T, rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_duplicated_kv_weights():
    p = rand_block(10, B=2, T=9, n_q=8, n_kv=2)
    rep, dh = 4, p["dh"]
    q = dict(p)
    q["wk"] = np.concatenate([p["wk"][(h // rep) * dh:(h // rep + 1) * dh] for h in range(8)])
    q["wv"] = np.concatenate([p["wv"][(h // rep) * dh:(h // rep + 1) * dh] for h in range(8)])
    q["n_kv"] = 8
    np.testing.assert_allclose(run_prefill(p)["Y"], run_prefill(q)["Y"], rtol=1e-12, atol=1e-13)


def test_mha_case_matches_torch_composition():
    # n_kv = n_q: the block with torch's own routines for norm and attention.
    p = rand_block(11, B=1, T=12, n_q=4, n_kv=4)
    out = run_prefill(p)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    q = (t(p["x"]) @ t(p["wq"]).T).view(1, 12, 4, 16)
    k = (t(p["x"]) @ t(p["wk"]).T).view(1, 12, 4, 16)
    v = (t(p["x"]) @ t(p["wv"]).T).view(1, 12, 4, 16)
    q = F.rms_norm(q, (16,), weight=t(p["gq"]), eps=1e-6)
    k = F.rms_norm(k, (16,), weight=t(p["gk"]), eps=1e-6)
    # RoPE as a complex multiply of (u_i + i*u_{i+dh/2}) by exp(i*p*omega_i).
    omega = torch.tensor([1e6 ** (-2 * i / 16) for i in range(8)], dtype=torch.float64)
    rot = torch.polar(torch.ones(12, 8, dtype=torch.float64), torch.arange(12.0, dtype=torch.float64)[:, None] * omega)
    def rope_c(u):
        z = torch.complex(u[..., :8], u[..., 8:]) * rot[None, :, None, :]
        return torch.cat([z.real, z.imag], dim=-1)
    q, k = rope_c(q), rope_c(k)
    a = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True)
    y = a.transpose(1, 2).reshape(1, 12, 64) @ t(p["wo"]).T
    np.testing.assert_allclose(out["Y"], y.numpy(), rtol=1e-11, atol=1e-12)


def test_scaling_q_or_k_weights_leaves_output_unchanged():
    p = rand_block(12, B=1, T=8)
    base = run_prefill(p)["Y"]
    for key in ("wq", "wk"):
        q = dict(p)
        q[key] = 3.0 * p[key]
        np.testing.assert_allclose(run_prefill(q)["Y"], base, rtol=1e-5, atol=1e-6)


def test_causality_future_rows_do_not_change_past_outputs():
    p = rand_block(13, B=1, T=10)
    base = run_prefill(p)
    for t in (0, 4, 8):
        q = dict(p)
        x = p["x"].copy()
        x[:, t + 1:] += np.random.default_rng(t).standard_normal(x[:, t + 1:].shape)
        q["x"] = x
        out = run_prefill(q)
        np.testing.assert_array_equal(out["Y"][:, :t + 1], base["Y"][:, :t + 1])
        assert not np.allclose(out["Y"][:, t + 1:], base["Y"][:, t + 1:])


def test_batch_permutation_permutes_outputs():
    p = rand_block(14, B=3, T=6)
    base = run_prefill(p)
    perm = [2, 0, 1]
    q = dict(p)
    q["x"] = p["x"][perm]
    out = run_prefill(q)
    np.testing.assert_allclose(out["Y"], base["Y"][perm], rtol=1e-13, atol=1e-14)


def test_decode_equals_last_prefill_row():
    # Decoding token T-1 over the cache of tokens 0..T-2 equals row T-1 of a
    # full prefill (Assembling a large model, "The complete code": the cache
    # path and the tril(diagonal=S-T) mask).
    p = rand_block(15, B=2, T=9)
    full = run_prefill(p)
    cap = 12
    kc = np.zeros((2, p["n_kv"], cap, 16))
    vc = np.zeros_like(kc)
    kc[:, :, :8] = full["Kc"][:, :, :8]
    vc[:, :, :8] = full["Vc"][:, :, :8]
    dec = oracle.decode(p["x"][:, 8], p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"],
                        np.array([8, 8]), kc, vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    np.testing.assert_allclose(dec["Y"], full["Y"][:, 8], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["k_new"], full["Kc"][:, :, 8], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dec["v_new"], full["Vc"][:, :, 8], rtol=1e-13, atol=1e-14)


def chunk_args(p, lo, hi, past, kc, vc):
    return dict(x=p["x"][:, lo:hi], wq=p["wq"], wk=p["wk"], wv=p["wv"], wo=p["wo"], gq=p["gq"],
                gk=p["gk"], positions=p["positions"][:, lo:hi], past_len=past, k_cache=kc,
                v_cache=vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=p["dh"])


def test_chunked_prefill_equals_one_shot_prefill():
    # Prefilling tokens 0..P-1, then appending tokens P..P+T-1 as a chunk over
    # that cache, gives the same outputs and cache rows as one prefill of all
    # P+T tokens (Assembling a large model, "The complete code": KVCache
    # concatenates after the cached keys; tril(diagonal=S-T) with S = P+T).
    p = rand_block(21, B=2, T=14)
    full = run_prefill(p)
    for P in (1, 5, 9):
        head = run_prefill({**p, "x": p["x"][:, :P], "positions": p["positions"][:, :P]})
        ch = oracle.prefill_chunk(**chunk_args(p, P, 14, [P, P], head["Kc"], head["Vc"]))
        np.testing.assert_allclose(ch["Y"], full["Y"][:, P:], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ch["Kc"], full["Kc"][:, :, P:], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ch["Vc"], full["Vc"][:, :, P:], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ch["Q"], full["Q"][:, P:], rtol=1e-13, atol=1e-14)


def test_chunked_prefill_ragged_past_and_special_cases():
    # Different cached lengths per sequence are independent; P = 0 is the
    # plain prefill; a one-token chunk is a decode step.
    p = rand_block(22, B=3, T=10)
    past = [0, 3, 6]
    fulls = [run_prefill({**p, "x": p["x"][b:b + 1, :past[b] + 4],
                          "positions": p["positions"][b:b + 1, :past[b] + 4]}) for b in range(3)]
    kc = np.full((3, p["n_kv"], 12, 16), np.nan)
    vc = np.full_like(kc, np.nan)          # slots >= past must not be read
    for b, P in enumerate(past):
        kc[b, :, :P] = fulls[b]["Kc"][0, :, :P]
        vc[b, :, :P] = fulls[b]["Vc"][0, :, :P]
    x = np.stack([p["x"][b, past[b]:past[b] + 4] for b in range(3)])
    pos = np.stack([p["positions"][b, past[b]:past[b] + 4] for b in range(3)])
    ch = oracle.prefill_chunk(x, p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"], pos, past,
                              kc, vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    for b, P in enumerate(past):
        np.testing.assert_allclose(ch["Y"][b], fulls[b]["Y"][0, P:P + 4], rtol=1e-12, atol=1e-13)
    one = oracle.prefill_chunk(x[:, :1], p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"],
                               pos[:, :1], past, kc, vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    dec = oracle.decode(x[:, 0], p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"],
                        np.array(past), kc, vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    np.testing.assert_allclose(one["Y"][:, 0], dec["Y"], rtol=1e-12, atol=1e-13)
    zero = oracle.prefill_chunk(**chunk_args(p, 0, 10, [0, 0, 0], kc, vc))
    np.testing.assert_allclose(zero["Y"], run_prefill(p)["Y"], rtol=1e-12, atol=1e-13)


def residual_args(p):
    return {k: p[k] for k in ("x", "wq", "wk", "wv", "wo", "gq", "gk", "positions")}


def test_layer_residual_is_identity_when_o_proj_is_zero():
    # x + block(RMSNorm(x) g): with Wo = 0 the block adds nothing and the
    # layer returns its input exactly (Assembling a large model, "The
    # complete code": the residual add around the attention).
    p = rand_block(31, B=2, T=7)
    g_in = 1 + 0.1 * np.random.default_rng(1).standard_normal(p["x"].shape[-1])
    a = residual_args(p)
    a["wo"] = np.zeros_like(a["wo"])
    out = oracle.prefill_residual(a.pop("x"), g_in, **a, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    np.testing.assert_array_equal(out["Y"], p["x"])


def test_layer_block_sees_the_normalised_input():
    # The block's input is RMS-normalised: scaling x by c > 0 scales the
    # residual part only, so layer(c x) - c x = layer(x) - x (up to eps); and a
    # row of the normalised input has RMS sqrt(m / (m + eps)) before the gain.
    p = rand_block(32, B=1, T=6)
    g_in = 1 + 0.1 * np.random.default_rng(2).standard_normal(p["x"].shape[-1])
    a = residual_args(p)
    x = a.pop("x")
    base = oracle.prefill_residual(x, g_in, **a, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    big = oracle.prefill_residual(7.5 * x, g_in, **a, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    np.testing.assert_allclose(big["Y"] - 7.5 * x, base["Y"] - x, rtol=0, atol=1e-6)  # eps-level
    xn = oracle.rms_norm(x, np.ones(x.shape[-1]), 1e-6)
    m = np.mean(x ** 2, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(xn ** 2, axis=-1)), np.sqrt(m / (m + 1e-6)),
                               rtol=1e-13)
    # without the norm and residual, the same weights give a different output
    plain = oracle.prefill(x, **a, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    assert not np.allclose(base["Y"] - x, plain["Y"])


def test_layer_decode_equals_last_layer_prefill_row():
    p = rand_block(33, B=2, T=9)
    g_in = 1 + 0.1 * np.random.default_rng(3).standard_normal(p["x"].shape[-1])
    a = residual_args(p)
    full = oracle.prefill_residual(a.pop("x"), g_in, **a, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    kc = np.zeros((2, p["n_kv"], 12, 16))
    vc = np.zeros_like(kc)
    kc[:, :, :8] = full["Kc"][:, :, :8]
    vc[:, :, :8] = full["Vc"][:, :, :8]
    dec = oracle.decode_residual(p["x"][:, 8], g_in, p["wq"], p["wk"], p["wv"], p["wo"], p["gq"],
                                 p["gk"], np.array([8, 8]), kc, vc, n_q=p["n_q"], n_kv=p["n_kv"],
                                 dh=16)
    np.testing.assert_allclose(dec["Y"], full["Y"][:, 8], rtol=1e-12, atol=1e-13)


def _torch_input_norm(x, g_in, eps=1e-6):
    # torch's own RMSNorm with a weight, in float64 (the oracle's rms_norm is not used)
    t = torch.from_numpy(np.asarray(x, np.float64))
    return F.rms_norm(t, (t.shape[-1],), weight=torch.from_numpy(np.asarray(g_in, np.float64)),
                      eps=eps).numpy()


def test_layer_input_gain_closed_form_with_zero_query_weight():
    # Wq = 0: q~ = 0, every visible key gets the same weight, so the block's
    # attention output is the prefix mean of V = (RMSNorm(x) * g_in) Wv^T and
    # the layer returns y_t = x_t + Wo . concat_h mean_{j<=t} V_{j, h // n_rep}
    # ("Assembling a large model from scratch", section "The complete code":
    # input_layernorm with its weight, attention, residual add).  V depends on
    # the input gain g_in element by element, so a dropped, squared or
    # misplaced gain fails here.
    p = rand_block(34, B=2, T=9, d=48, n_q=6, n_kv=3)
    g_in = 1 + 0.3 * np.random.default_rng(4).standard_normal(48)
    a = residual_args(p)
    a["wq"] = np.zeros_like(a["wq"])
    x = a.pop("x")
    out = oracle.prefill_residual(x, g_in, **a, n_q=6, n_kv=3, dh=16)
    v = (_torch_input_norm(x, g_in) @ p["wv"].T).reshape(2, 9, 3, 16)
    pref = np.cumsum(v, axis=1) / np.arange(1, 10)[None, :, None, None]
    cat = np.concatenate([pref[:, :, h // 2] for h in range(6)], axis=-1)
    np.testing.assert_allclose(out["Y"], x + cat @ p["wo"].T, rtol=1e-12, atol=1e-12)


def test_layer_decode_input_gain_closed_form_with_zero_query_weight():
    # The same closed form for one decode step: the new token (position L)
    # weighs the L cached values and its own value V = (RMSNorm(x) * g_in) Wv^T
    # equally, y = x + Wo . concat_h mean(V_cache[0..L-1], V_new).
    rng = np.random.default_rng(5)
    p = rand_block(35, B=3, T=1, d=48, n_q=4, n_kv=2)
    g_in = 1 + 0.3 * rng.standard_normal(48)
    L = np.array([0, 3, 6])
    kc = rng.standard_normal((3, 2, 8, 16))
    vc = rng.standard_normal((3, 2, 8, 16))
    x = p["x"][:, 0]
    dec = oracle.decode_residual(x, g_in, np.zeros_like(p["wq"]), p["wk"], p["wv"], p["wo"],
                                 p["gq"], p["gk"], L, kc, vc, n_q=4, n_kv=2, dh=16)
    vnew = (_torch_input_norm(x, g_in) @ p["wv"].T).reshape(3, 2, 16)
    for s in range(3):
        allv = np.concatenate([vc[s][:, :L[s]], vnew[s][:, None]], axis=1)   # [n_kv, L+1, dh]
        mean = allv.mean(axis=1)
        cat = np.concatenate([mean[h // 2] for h in range(4)])
        np.testing.assert_allclose(dec["Y"][s], x[s] + p["wo"] @ cat, rtol=1e-12, atol=1e-12)


# --- sliding window ------------------------------------------------------
# A layer with sliding window W keeps the W most recent keys, the query's own
# included ("Qwen3 Architecture Layer-by-Layer", sections "Layer 1 -
# Qwen3Model" and "Layer 3 - Qwen3Attention": per-layer sliding_window and
# the sliding-window causal mask).
def test_window_one_attends_to_own_value_only():
    # W = 1: every token sees only itself, so A_t = concat_h V_{t, h // n_rep}
    # and Y_t = Wo . A_t (a window one key too wide or too narrow fails).
    p = rand_block(31, B=2, T=7, d=48, n_q=6, n_kv=3)
    out = run_prefill(p, window=1)
    v = (p["x"] @ p["wv"].T).reshape(2, 7, 3, 16)
    cat = np.concatenate([v[:, :, h // 2] for h in range(6)], axis=-1)
    np.testing.assert_allclose(out["A"], cat, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["Y"], cat @ p["wo"].T, rtol=1e-12, atol=1e-13)


def test_window_covering_the_sequence_is_full_attention():
    p = rand_block(32, B=2, T=9)
    full = run_prefill(p)
    for W in (9, 10, 100):
        np.testing.assert_array_equal(run_prefill(p, window=W)["Y"], full["Y"])
    assert not np.allclose(run_prefill(p, window=8)["Y"][:, 8], full["Y"][:, 8])
    np.testing.assert_array_equal(run_prefill(p, window=8)["Y"][:, :8], full["Y"][:, :8])


@pytest.mark.parametrize("W", [2, 3, 5])
def test_window_row_equals_full_prefill_of_the_window_slice(W):
    # RoPE scores depend on position differences only, so row t of a window-W
    # prefill equals the last row of a plain causal prefill of tokens
    # t-W+1 .. t that keep their own positions.
    p = rand_block(33 + W, B=1, T=10)
    win = run_prefill(p, window=W)
    for t in range(10):
        lo = max(0, t - W + 1)
        sl = run_prefill({**p, "x": p["x"][:, lo:t + 1], "positions": p["positions"][:, lo:t + 1]})
        np.testing.assert_allclose(win["Y"][:, t], sl["Y"][:, -1], rtol=1e-11, atol=1e-12)


def test_window_outputs_do_not_depend_on_tokens_outside_it():
    # Perturbing token j changes outputs j .. j+W-1 only; rows from j+W on are
    # bitwise unchanged (and rows before j by causality).
    p = rand_block(37, B=1, T=12)
    W = 4
    base = run_prefill(p, window=W)["Y"]
    for j in (0, 3, 7):
        x = p["x"].copy()
        x[:, j] += np.random.default_rng(j).standard_normal(x.shape[-1])
        out = run_prefill({**p, "x": x}, window=W)["Y"]
        np.testing.assert_array_equal(out[:, :j], base[:, :j])
        np.testing.assert_array_equal(out[:, j + W:], base[:, j + W:])
        for t in range(j, min(j + W, 12)):
            assert not np.allclose(out[:, t], base[:, t])


def test_window_matches_torch_sdpa_with_band_mask():
    rng = np.random.default_rng(38)
    T, S, W = 5, 11, 3
    q = rng.standard_normal((T, 8, 32))
    k = rng.standard_normal((S, 2, 32))
    v = rng.standard_normal((S, 2, 32))
    ours = oracle.gqa_attention(q, k, v, window=W)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2)[None] for a in (q, k, v))
    band = torch.ones(T, S, dtype=torch.bool)
    mask = band.tril(diagonal=S - T) & ~band.tril(diagonal=S - T - W)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    np.testing.assert_allclose(ours, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_window_chunk_and_decode_equal_one_shot_window_prefill():
    # The window is anchored at the key position P + t of a chunk token, not
    # at its index inside the chunk; decode is the one-token chunk.
    p = rand_block(39, B=2, T=13)
    W = 4
    full = run_prefill(p, window=W)
    for P in (2, 6, 12):
        head = run_prefill({**p, "x": p["x"][:, :P], "positions": p["positions"][:, :P]})
        ch = oracle.prefill_chunk(**chunk_args(p, P, 13, [P, P], head["Kc"], head["Vc"]),
                                  window=W)
        np.testing.assert_allclose(ch["Y"], full["Y"][:, P:], rtol=1e-12, atol=1e-13)
    head = run_prefill({**p, "x": p["x"][:, :12], "positions": p["positions"][:, :12]})
    dec = oracle.decode(p["x"][:, 12], p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"],
                        np.array([12, 12]), head["Kc"], head["Vc"], n_q=p["n_q"],
                        n_kv=p["n_kv"], dh=16, window=W)
    np.testing.assert_allclose(dec["Y"], full["Y"][:, 12], rtol=1e-12, atol=1e-13)


def test_decode_ragged_lengths_and_empty_cache():
    # Sequences with different cache lengths, including 0, are independent.
    p = rand_block(16, B=3, T=6)
    lens = [0, 3, 5]
    full = [run_prefill({**p, "x": p["x"][s:s + 1, :lens[s] + 1],
                         "positions": np.arange(lens[s] + 1)[None]}) for s in range(3)]
    kc = np.zeros((3, p["n_kv"], 8, 16))
    vc = np.zeros_like(kc)
    for s, L in enumerate(lens):
        kc[s, :, :L] = full[s]["Kc"][0, :, :L]
        vc[s, :, :L] = full[s]["Vc"][0, :, :L]
    xs = np.stack([p["x"][s, lens[s]] for s in range(3)])
    dec = oracle.decode(xs, p["wq"], p["wk"], p["wv"], p["wo"], p["gq"], p["gk"],
                        np.array(lens), kc, vc, n_q=p["n_q"], n_kv=p["n_kv"], dh=16)
    for s in range(3):
        np.testing.assert_allclose(dec["Y"][s], full[s]["Y"][0, -1], rtol=1e-12, atol=1e-13)


# --- the pages' worked numbers ----------------------------------------------------
def test_qwen3_0p6b_shape_table():
    g = golden("qwen3_0p6b_shapes.json")
    w = WORKLOADS[2]
    inp = prefill_inputs(w, T=4)
    for name, key in (("q_proj", "Wq"), ("k_proj", "Wk"), ("v_proj", "Wv"), ("o_proj", "Wo"),
                      ("q_norm", "gq"), ("k_norm", "gk")):
        assert list(inp[key].shape) == g["weights"][name]
    out = oracle.prefill(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                         inp["gk"], inp["positions"], n_q=w.n_q, n_kv=w.n_kv)
    B, T = 2, 4
    sub = lambda s: [B if i == 0 else (T if i == 1 else v) for i, v in enumerate(s)]
    a = g["activations"]
    assert list(out["Q"].shape) == sub(a["q_heads"])
    assert list(out["A"].shape) == sub(a["attn_merged"])
    assert list(out["Y"].shape) == sub(a["o_proj_out"])
    assert list(out["Kc"].shape) == [B, g["n_kv"], T, g["d_head"]]


def test_worked_example_wide_gqa_sizes_and_logit_scale():
    g = golden("worked_example_wide_gqa.json")
    w = WORKLOADS[4]
    assert (w.d, w.n_q, w.n_kv, w.dh) == (g["d_model"], g["n_q"], g["n_kv"], g["d_head"])
    assert [w.d, w.n_q * w.dh] == g["query_projection_in_out"]
    assert [w.d, w.n_kv * w.dh] == g["key_value_projection_in_out"]
    assert 2 * w.n_kv * w.dh == g["kv_cache_values_per_token_per_layer"]
    assert (2 * w.n_kv * w.dh) / (2 * w.n_q * w.dh) == g["kv_cache_fraction_of_mha"]
    # QK-Norm puts raw logits at RMS ~ sqrt(128) ~ 11.3 and scaled ones at ~1.
    rng = np.random.default_rng(17)
    d, T = 256, 64
    x = rng.standard_normal((1, T, d))
    wq = 0.02 * rng.standard_normal((8 * 128, d))
    wk = 0.02 * rng.standard_normal((2 * 128, d))
    wv = 0.02 * rng.standard_normal((2 * 128, d))
    q, k, _ = oracle.project_norm_rope(x, wq, wk, wv, np.ones(128), np.ones(128),
                                       np.zeros((1, T)), n_q=8, n_kv=2, dh=128,
                                       eps=1e-6, theta=1e6)
    raw = np.einsum("thd,shd->hts", q[0], np.repeat(k[0], 4, axis=1))
    rms = np.sqrt(np.mean(raw ** 2))
    assert rms == pytest.approx(g["raw_logit_rms_after_qk_norm"], rel=g["raw_logit_rms_rel_tolerance"])
    assert rms / np.sqrt(128) == pytest.approx(g["scaled_logit_rms"], rel=g["raw_logit_rms_rel_tolerance"])


# --- the seeded inputs -------------------------------------------------------------
def test_bf16_inputs_are_exactly_representable():
    inp = prefill_inputs(WORKLOADS[2], B=1, T=8)
    bits = inp["X"].view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    inp1 = prefill_inputs(WORKLOADS[1], T=8)
    assert np.any((inp1["X"].view(np.uint32) & 0xFFFF) != 0)


def test_inputs_are_seeded_and_reproducible():
    a = prefill_inputs(WORKLOADS[3], T=4)
    b = prefill_inputs(WORKLOADS[3], T=4)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_sampled_rows_equal_full_prefill():
    p = rand_block(18, B=2, T=13)
    full = run_prefill(p)
    rows = [(0, 0), (1, 12), (0, 7), (1, 5)]
    args = {k: p[k] for k in ("x", "wq", "wk", "wv", "wo", "gq", "gk", "positions")}
    r = oracle.prefill_rows(**args, rows=rows, n_q=p["n_q"], n_kv=p["n_kv"], dh=p["dh"])
    for i, (b, t) in enumerate(rows):
        np.testing.assert_allclose(r["Y"][i], full["Y"][b, t], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(r["Kc"][1], full["Kc"][1])
