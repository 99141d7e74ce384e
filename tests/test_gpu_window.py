"""GPU parity of sliding-window layers, through the C ABI, against the oracle.

A layer of window W lets each token see only its W most recent keys, its own
included ("Qwen3 Architecture Layer-by-Layer", sections "Layer 1 -
Qwen3Model" and "Layer 3 - Qwen3Attention": the per-layer sliding_window and
the sliding-window causal mask).  Cache slots that no window of a call
reaches hold NaN on the GPU side (the oracle gets the same caches without
them), so a kernel that read them would fail.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import (assert_close, block_from_inputs, dev, host, say, storage_floor_prefill,
                      storage_floor_rows, to_paged)
from workloads import (EPS, ROPE_THETA, WORKLOADS, decode_cache_host, decode_inputs,
                       prefill_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def weights(inp):
    return [inp[k] for k in ("Wq", "Wk", "Wv", "Wo", "gq", "gk")]


def okw(w, W):
    return dict(n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA, window=W)


def prefill_gpu(w, inp, B, T, W):
    import torch
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, sliding_window=W)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.full((B, w.n_kv, T + 16, 128), float("nan"), dtype=x.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    y = blk.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    out = dict(Y=host(y), Kc=host(kc), Vc=host(vc))
    blk.close()
    return out


WINDOW_PREFILL_CASES = [
    (1, 1, 128, 37),    # fp32 (32-key tiles), window edge inside a tile
    (1, 2, 200, 1),     # fp32, each token sees itself only
    (2, 2, 300, 1),     # bf16
    (2, 2, 300, 100),   # bf16, few query tiles: key ranges split over workgroups
    (2, 1, 700, 64),    # window = one key tile
    (2, 1, 700, 65),
    (3, 1, 520, 256),   # 4B shape (n_rep 4)
    (4, 1, 260, 70),    # wide GQA (n_rep 16)
]


@pytest.mark.parametrize("idx,B,T,W", WINDOW_PREFILL_CASES)
def test_window_prefill_parity(idx, B, T, W):
    w = WORKLOADS[idx]
    say(f"window prefill parity: {w.name} B={B} T={T} W={W}")
    inp = prefill_inputs(w, B=B, T=T)
    got = prefill_gpu(w, inp, B, T, W)
    ref = oracle.prefill(inp["X"], *weights(inp), inp["positions"], **okw(w, W))
    assert_close(got["Kc"][:, :, :T], ref["Kc"], w.dtype, "k cache")
    floor = storage_floor_prefill(inp, w, B, T, window=W) if w.dtype == "bf16" else None
    assert_close(got["Y"], ref["Y"], w.dtype, "windowed block output Y", floor=floor)


@pytest.mark.parametrize("n_q,n_kv,T,W", [(24, 8, 300, 50), (40, 8, 190, 33)])
def test_window_prefill_odd_group_sizes(n_q, n_kv, T, W):
    # n_rep 3 and 5: a wave's rows span tokens whose windows start in
    # different key tiles.
    w = dataclasses.replace(WORKLOADS[2], n_q=n_q, n_kv=n_kv)
    say(f"window prefill parity: n_q={n_q} n_kv={n_kv} T={T} W={W}")
    inp = prefill_inputs(w, B=1, T=T)
    got = prefill_gpu(w, inp, 1, T, W)
    ref = oracle.prefill(inp["X"], *weights(inp), inp["positions"], **okw(w, W))
    assert_close(got["Y"], ref["Y"], w.dtype, "Y")


def test_window_prefill_full_size_0p6b():
    # The 0.6B shape at full size (B=2, T=2048) with a 512-key window.
    w = WORKLOADS[2]
    W = 512
    say(f"window prefill full size: {w.name} W={W}")
    inp = prefill_inputs(w)
    got = prefill_gpu(w, inp, w.B, w.T, W)
    ref = oracle.prefill(inp["X"], *weights(inp), inp["positions"], **okw(w, W))
    assert_close(got["Y"], ref["Y"], w.dtype, "Y")


def test_window_prefill_wide_gqa_full_size_sampled_rows():
    # Wide GQA at T=8192 (many query tiles: the 4-wave workgroup variant)
    # with a 4096-key window; rows around the window's reach are sampled.
    w = WORKLOADS[4]
    W = 4096
    say(f"window prefill full size, sampled rows: {w.name} W={W}")
    inp = prefill_inputs(w)
    got = prefill_gpu(w, inp, w.B, w.T, W)
    ts = [0, 63, 64, 4094, 4095, 4096, 4097, 4160, 6000, 8190, 8191]
    ref = oracle.prefill_rows(inp["X"], *weights(inp), inp["positions"], [(0, t) for t in ts],
                              **okw(w, W))
    floor = storage_floor_rows(inp["X"][0], *weights(inp), inp["positions"][0], ts, n_q=w.n_q,
                               n_kv=w.n_kv, window=W)
    assert_close(np.stack([got["Y"][0, t] for t in ts]), ref["Y"], w.dtype, "Y at sampled rows",
                 floor=floor)


def test_window_covering_the_sequence_equals_full_attention_bitwise():
    w = WORKLOADS[2]
    T = 300
    inp = prefill_inputs(w, B=1, T=T)
    full = prefill_gpu(w, inp, 1, T, 0)
    for W in (T, 1 << 30):
        np.testing.assert_array_equal(prefill_gpu(w, inp, 1, T, W)["Y"], full["Y"])
    # one key short: only the last token loses a key
    short = prefill_gpu(w, inp, 1, T, T - 1)
    np.testing.assert_array_equal(short["Y"][:, :T - 1], full["Y"][:, :T - 1])
    assert not np.array_equal(short["Y"][:, T - 1], full["Y"][:, T - 1])


def nan_below(cache, lo):
    """Copy of cache [S, n_kv, cap, dh] with slots < lo[s] set to NaN."""
    c = cache.copy()
    for s, L in enumerate(lo):
        c[s, :, :int(L)] = np.nan
    return c


@pytest.mark.parametrize("idx,B,T,past,W", [
    (1, 1, 58, [70], 20),             # fp32
    (2, 2, 150, [37, 300], 100),      # window reaches into the cache of seq 1 only
    (2, 3, 1, [0, 64, 1000], 64),     # one-token chunks
    (4, 1, 65, [200], 128),           # wide GQA
])
def test_window_prefill_chunk_parity(idx, B, T, past, W):
    import torch
    w = WORKLOADS[idx]
    say(f"window chunked prefill parity: {w.name} B={B} T={T} past={past} W={W}")
    inp = prefill_inputs(w, B=B, T=T)
    past = np.asarray(past, np.int32)
    inp["positions"] = (past[:, None] + np.arange(T, dtype=np.int32)[None, :]).astype(np.int32)
    cap = int(past.max()) + T + 8
    kc, vc = decode_cache_host(w, past, cap, seed=w.seed + 1)
    # slots below the 64-key tile holding the chunk's first window start are never read
    unread = [max(0, int(P) - W + 1) // 64 * 64 for P in past]
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, sliding_window=W)
    kcd, vcd = dev(nan_below(kc, unread), w.dtype), dev(nan_below(vc, unread), w.dtype)
    y = blk.prefill_chunk(dev(inp["X"], w.dtype), torch.from_numpy(inp["positions"]).to("cuda"),
                          torch.from_numpy(past).to("cuda"), kcd, vcd)
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk(inp["X"], *weights(inp), inp["positions"], past, kc, vc,
                               **okw(w, W))
    assert_close(host(y), ref["Y"], w.dtype, "windowed chunk Y")
    kh = host(kcd)
    for b, P in enumerate(past):
        assert_close(kh[b, :, P:P + T], ref["Kc"][b], w.dtype, f"k cache chunk (seq {b})")
    blk.close()


DEC_LENS = np.array([0, 1, 99, 100, 511, 512, 513, 1030, 2047], np.int32)


@pytest.mark.parametrize("dtype,n_q,n_kv,W", [("bf16", 16, 8, 100), ("bf16", 16, 8, 1),
                                              ("f32", 16, 8, 600), ("bf16", 64, 4, 513),
                                              ("bf16", 40, 8, 17)])
def test_window_decode_parity(dtype, n_q, n_kv, W):
    import torch
    w = dataclasses.replace(WORKLOADS[5], dtype=dtype, n_q=n_q, n_kv=n_kv)
    say(f"window decode parity: dtype={dtype} n_q={n_q} n_kv={n_kv} W={W}")
    lens = DEC_LENS
    inp = decode_inputs(w, N=len(lens))
    inp["positions"] = lens
    kc, vc = decode_cache_host(w, lens, 2112)
    unread = np.maximum(0, lens + 1 - W)          # keys older than the window
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, sliding_window=W)
    kcd, vcd = dev(nan_below(kc, unread), w.dtype), dev(nan_below(vc, unread), w.dtype)
    y = blk.decode(dev(inp["X"], w.dtype), torch.from_numpy(lens).to("cuda"), kcd, vcd)
    torch.cuda.synchronize()
    ref = oracle.decode(inp["X"], *weights(inp), lens, kc, vc, **okw(w, W))
    assert_close(host(y), ref["Y"], w.dtype, "windowed decode Y")
    kh = host(kcd)
    assert_close(np.stack([kh[s, :, L] for s, L in enumerate(lens)]), ref["k_new"], w.dtype,
                 "new k in slot L")
    blk.close()


def test_window_decode_paged_parity():
    import torch
    w = WORKLOADS[5]
    W, bs = 300, 64
    say(f"window paged decode parity: W={W} block_size={bs}")
    lens = DEC_LENS
    inp = decode_inputs(w, N=len(lens))
    inp["positions"] = lens
    kc, vc = decode_cache_host(w, lens, 2112)
    unread = np.maximum(0, lens + 1 - W)
    kp, vp, table = to_paged(nan_below(kc, unread), nan_below(vc, unread), lens + 1, bs, seed=3)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, sliding_window=W)
    x, pos = dev(inp["X"], w.dtype), torch.from_numpy(lens).to("cuda")
    y_p = blk.decode_paged(x, pos, torch.from_numpy(table).to("cuda"), dev(kp, w.dtype),
                           dev(vp, w.dtype))
    y_c = blk.decode(x, pos, dev(kc, w.dtype), dev(vc, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.decode(inp["X"], *weights(inp), lens, kc, vc, **okw(w, W))
    assert_close(host(y_p), ref["Y"], w.dtype, "windowed paged decode Y")
    # at this size both calls take 512-key chunks, so they match bit for bit
    np.testing.assert_array_equal(host(y_p), host(y_c))
    blk.close()


def test_window_decode_full_size_sampled_sequences():
    # The 64-sequence decode workload (caches of 1024..32768) with a
    # 4096-key window; sampled sequences against the oracle.
    import torch
    w = WORKLOADS[5]
    W = 4096
    say(f"window decode full size: {w.name} W={W}")
    inp = decode_inputs(w)
    L = inp["positions"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 11)
    kc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda").to(torch.bfloat16)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, sliding_window=W)
    y = blk.decode(dev(inp["X"], w.dtype), torch.from_numpy(L).to("cuda"), kc, vc)
    torch.cuda.synchronize()
    Y = host(y)
    for s in sorted({int(np.argmin(L)), int(np.argmax(L)), 0, 42}):
        Ls = int(L[s])
        lo = max(0, Ls + 1 - W)
        # the oracle sees the window's keys only, at their own slots; older
        # slots are zero (masked by the window, never weighted)
        k_all = np.zeros((w.n_kv, Ls + 1, 128))
        v_all = np.zeros_like(k_all)
        k_all[:, lo:] = host(kc[s, :, lo:Ls + 1])
        v_all[:, lo:] = host(vc[s, :, lo:Ls + 1])
        sub = {k: (v[s:s + 1] if k in ("X", "positions") else v) for k, v in inp.items()}
        ref = oracle.decode(sub["X"], *weights(sub), sub["positions"], k_all[None, :, :Ls],
                            v_all[None, :, :Ls], **okw(w, W))
        assert_close(Y[s:s + 1], ref["Y"], w.dtype, f"decode Y seq {s} (L={Ls})")
        assert_close(k_all[:, Ls], ref["k_new"][0], w.dtype, f"new k seq {s}")
    blk.close()
    del kc, vc
    torch.cuda.empty_cache()
