"""Parity of the HIP block (through the C ABI) with the fp64 CPU oracle.

Reduced sizes span several 128-row / 64-key tiles and a ragged tail; the full
workload sizes run in the same launch configuration as the benchmark and are
checked on sampled rows (prefill) or sampled sequences (decode) that the
oracle computes one by one.  Pass bar: fp32 max abs <= 1e-4; bf16 max abs <=
2e-2 and relative L2 <= 1e-2.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from gpu_util import (assert_close, block_from_inputs, dev, from_paged, host, say,
                      storage_floor_prefill, storage_floor_rows, to_paged)
from workloads import (EPS, ROPE_THETA, WORKLOADS, bf16_bits_to_f32, decode_cache_host,
                       decode_inputs, prefill_inputs, round_to_bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


Q_WS_SCALE = float(np.float32(math.log2(math.e) / math.sqrt(128.0)))


def run_prefill_gpu(w, inp, B, T, *, cap_extra=64):
    import torch
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    cap = T + cap_extra
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.full((B, w.n_kv, cap, 128), float("nan"), dtype=x.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    ws = torch.empty(blk.workspace_size(False, B, T), dtype=torch.uint8, device="cuda")
    y = blk.prefill(x, pos, kc, vc, workspace=ws)
    torch.cuda.synchronize()
    es = 4 if w.dtype == "f32" else 2
    qt = ws[: B * T * w.n_q * 128 * es].view(x.dtype).view(B, T, w.n_q, 128)
    # The workspace holds q~ times log2(e)/sqrt(d_head) (fp32 factor).
    out = dict(Y=host(y), Kc=host(kc), Vc=host(vc), Q=host(qt) / Q_WS_SCALE)
    blk.close()
    return out


def oracle_prefill(inp, w):
    return oracle.prefill(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                          inp["gk"], inp["positions"], n_q=w.n_q, n_kv=w.n_kv, eps=EPS,
                          theta=ROPE_THETA)


PREFILL_CASES = [
    (1, 1, 128),   # the tiny fp32 workload at its full size
    (1, 2, 200),   # fp32, ragged over the 128-row and 32-key tiles
    (2, 2, 300),   # 0.6B shape, ragged over 128-row / 64-key tiles
    (3, 1, 520),   # 4B shape (n_rep 4)
    (4, 1, 260),   # wide GQA (n_rep 16)
    (2, 3, 1),     # one token per sequence
    (2, 1, 33),
    (2, 1, 64),
]


@pytest.mark.parametrize("idx,B,T", PREFILL_CASES)
def test_prefill_parity(idx, B, T):
    w = WORKLOADS[idx]
    say(f"prefill parity: workload {idx} ({w.name}) B={B} T={T}")
    inp = prefill_inputs(w, B=B, T=T)
    got = run_prefill_gpu(w, inp, B, T)
    ref = oracle_prefill(inp, w)
    assert_close(got["Q"], ref["Q"], w.dtype, "q~ (post-norm, post-RoPE)")
    assert_close(got["Kc"][:, :, :T], ref["Kc"], w.dtype, "k cache")
    assert_close(got["Vc"][:, :, :T], ref["Vc"], w.dtype, "v cache")
    assert np.all(np.isnan(got["Kc"][:, :, T:])), "cache slots >= T were written"
    assert np.all(np.isnan(got["Vc"][:, :, T:])), "cache slots >= T were written"
    floor = storage_floor_prefill(inp, w, B, T) if w.dtype == "bf16" else None
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y", floor=floor)


@pytest.mark.parametrize("dtype,gain", [("bf16", 1.71875), ("f32", 1.71875), ("bf16", 1.75),
                                        ("f32", 1.75)])
def test_prefill_scores_at_the_fixed_reference_limit(dtype, gain):
    # Over empty caches the attention takes the handle's score bound
    # 16.32 * max|g_q| * max|g_k| * (1 + 1/64) (log2 units) as a fixed softmax
    # reference while it is <= 50.  Constant gains of 1.71875 put it at 48.97,
    # just inside; 1.75 gives 50.77 and the running-max path.  With Wq = Wk
    # (16 query heads, 16 KV heads) each token's own score equals the
    # unmargined bound, 48.2, the largest a score can be, while others reach
    # down to about -48: probabilities from about 2^-97 to 1.
    w = dataclasses.replace(WORKLOADS[2], dtype=dtype, n_q=16, n_kv=16)
    B, T = 1, 300
    say(f"prefill at the fixed-reference limit: dtype={dtype} gains={gain}")
    inp = prefill_inputs(w, B=B, T=T)
    inp["Wk"] = inp["Wq"].copy()
    inp["gq"] = np.full(128, gain, np.float32)
    inp["gk"] = np.full(128, gain, np.float32)
    got = run_prefill_gpu(w, inp, B, T)
    ref = oracle_prefill(inp, w)
    assert_close(got["Kc"][:, :, :T], ref["Kc"], w.dtype, "k cache")
    floor = storage_floor_prefill(inp, w, B, T) if w.dtype == "bf16" else None
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y", floor=floor)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_full_size_0p6b(dtype):
    # The benchmark's workload, compared in full; in fp32 too, which takes the
    # same 256x256 q/k/v tiles (shared RoPE angles) through the fp32 MFMAs.
    w = dataclasses.replace(WORKLOADS[2], dtype=dtype)
    say(f"prefill parity full size: {w.name}")
    inp = prefill_inputs(w)
    got = run_prefill_gpu(w, inp, w.B, w.T)
    ref = oracle_prefill(inp, w)
    assert_close(got["Kc"][:, :, :w.T], ref["Kc"], w.dtype, "k cache")
    assert_close(got["Vc"][:, :, :w.T], ref["Vc"], w.dtype, "v cache")
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y")


@pytest.mark.parametrize("idx", [3, 4])
def test_prefill_full_size_sampled_rows(idx):
    w = WORKLOADS[idx]
    say(f"prefill parity full size, sampled rows: {w.name}")
    inp = prefill_inputs(w)
    got = run_prefill_gpu(w, inp, w.B, w.T)
    rng = np.random.default_rng(idx)
    ts = sorted({0, 1, 31, 63, 64, 127, 128, 129, w.T // 2, w.T - 2, w.T - 1,
                 *rng.integers(0, w.T, 6).tolist()})
    rows = [(0, t) for t in ts]
    ref = oracle.prefill_rows(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                              inp["gk"], inp["positions"], rows, n_q=w.n_q, n_kv=w.n_kv,
                              eps=EPS, theta=ROPE_THETA)
    assert_close(got["Kc"][0][:, :w.T], ref["Kc"][0], w.dtype, "k cache (all tokens)")
    assert_close(got["Vc"][0][:, :w.T], ref["Vc"][0], w.dtype, "v cache (all tokens)")
    floor = storage_floor_rows(inp["X"][0], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                               inp["gk"], inp["positions"][0], ts, n_q=w.n_q, n_kv=w.n_kv)
    assert_close(np.stack([got["Y"][0, t] for t in ts]), ref["Y"], w.dtype, "Y at sampled rows",
                 floor=floor)


@pytest.mark.parametrize("n_q,n_kv,B,T", [(8, 4, 2, 4100), (16, 4, 1, 4100), (6, 3, 1, 11008)])
def test_prefill_long_odd_tile_count_sampled_rows(n_q, n_kv, B, T):
    # 520 and 516 query tiles of 128 rows (two rounds of 8-wave workgroups),
    # an odd tile count per KV group and a ragged last tile; n_rep 2 and 4.
    # Rows at tile edges, the middle tiles and the ends are checked against
    # the oracle, the caches in full.  With 6/3 heads the q/k/v GEMM runs
    # 256x256 tiles (two heads each) and one tile pairs the last key head with
    # the first value head, so a value-head wave evaluates half of the key
    # head's RoPE angles.
    w = dataclasses.replace(WORKLOADS[2], n_q=n_q, n_kv=n_kv)
    say(f"prefill parity, long odd tile count: n_q={n_q} n_kv={n_kv} B={B} T={T}")
    inp = prefill_inputs(w, B=B, T=T)
    got = run_prefill_gpu(w, inp, B, T)
    rep = n_q // n_kv
    per_tile = 128 // rep                     # tokens per query tile
    tiles = (T * rep + 127) // 128
    mid = (tiles // 2) * per_tile
    ts = sorted({0, 1, per_tile - 1, per_tile, mid - 1, mid, mid + per_tile - 1, mid + per_tile,
                 T // 3, T - per_tile - 1, T - per_tile, T - 2, T - 1})
    rows = [(b, t) for b in range(B) for t in ts]
    ref = oracle.prefill_rows(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                              inp["gk"], inp["positions"], rows, n_q=n_q, n_kv=n_kv, eps=EPS,
                              theta=ROPE_THETA)
    for b in range(B):
        assert_close(got["Kc"][b][:, :T], ref["Kc"][b], w.dtype, f"k cache (all tokens, seq {b})")
        assert_close(got["Vc"][b][:, :T], ref["Vc"][b], w.dtype, f"v cache (all tokens, seq {b})")
    assert_close(np.stack([got["Y"][b, t] for b, t in rows]), ref["Y"], w.dtype, "Y at sampled rows")


def test_prefill_mha_case():
    # n_kv == n_q: standard multi-head attention (n_rep = 1).
    w = dataclasses.replace(WORKLOADS[2], n_q=8, n_kv=8)
    inp = prefill_inputs(w, B=1, T=150)
    got = run_prefill_gpu(w, inp, 1, 150)
    ref = oracle_prefill(inp, w)
    assert_close(got["Y"], ref["Y"], w.dtype, "Y (MHA)")


@pytest.mark.parametrize("n_q,n_kv,T", [(24, 8, 300), (40, 8, 190), (12, 4, 77), (48, 8, 100),
                                        (56, 8, 150)])
def test_prefill_odd_group_sizes(n_q, n_kv, T):
    # n_rep = 3, 5, 6 and 7: a wave's 32 packed rows cover a token range that
    # is not aligned to the 64-key tiles.
    w = dataclasses.replace(WORKLOADS[2], n_q=n_q, n_kv=n_kv)
    say(f"prefill parity: n_q={n_q} n_kv={n_kv} T={T}")
    inp = prefill_inputs(w, B=1, T=T)
    got = run_prefill_gpu(w, inp, 1, T)
    ref = oracle_prefill(inp, w)
    assert_close(got["Q"], ref["Q"], w.dtype, "q~")
    assert_close(got["Kc"][:, :, :T], ref["Kc"], w.dtype, "k cache")
    assert_close(got["Y"], ref["Y"], w.dtype, "Y")


def test_prefill_nonzero_positions():
    # Positions drive RoPE only; an offset start still uses the causal-by-index mask.
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=2, T=70)
    inp["positions"] = inp["positions"] + np.array([[5000], [31000]], np.int32)
    got = run_prefill_gpu(w, inp, 2, 70)
    ref = oracle_prefill(inp, w)
    assert_close(got["Kc"][:, :, :70], ref["Kc"], w.dtype, "k cache")
    assert_close(got["Y"], ref["Y"], w.dtype, "Y")


def test_prefill_positions_at_the_top_of_the_supported_range():
    # Positions up to 2^24 - 1 convert to fp32 exactly and the angle is reduced
    # exactly in revolutions, so fp32 q~ and K keep the 1e-4 bar there.
    w = WORKLOADS[1]
    inp = prefill_inputs(w, B=1, T=40)
    inp["positions"] = inp["positions"] + np.int32((1 << 24) - 40)
    say(f"prefill parity at positions {int(inp['positions'].min())}..{int(inp['positions'].max())}")
    got = run_prefill_gpu(w, inp, 1, 40)
    ref = oracle_prefill(inp, w)
    assert_close(got["Q"], ref["Q"], w.dtype, "q~")
    assert_close(got["Kc"][:, :, :40], ref["Kc"], w.dtype, "k cache")
    assert_close(got["Y"], ref["Y"], w.dtype, "Y")


def test_prefill_deterministic_and_causal():
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=1, T=200)
    a = run_prefill_gpu(w, inp, 1, 200)
    b = run_prefill_gpu(w, inp, 1, 200)
    np.testing.assert_array_equal(a["Y"], b["Y"])
    # Perturbing tokens after t leaves outputs 0..t bitwise unchanged.
    t = 77
    pert = dict(inp)
    x = inp["X"].copy()
    x[:, t + 1:] = prefill_inputs(w, B=1, T=200, seed=99)["X"][:, t + 1:]
    pert["X"] = x
    c = run_prefill_gpu(w, pert, 1, 200)
    np.testing.assert_array_equal(c["Y"][:, : t + 1], a["Y"][:, : t + 1])
    assert not np.array_equal(c["Y"][:, t + 1:], a["Y"][:, t + 1:])


# ---------------------------------------------------------------- chunked prefill
def chunk_case(idx, B, T, past, *, seed=None, cap_extra=40):
    w = WORKLOADS[idx]
    inp = prefill_inputs(w, B=B, T=T, seed=seed)
    past = np.asarray(past, np.int32)
    inp["positions"] = (past[:, None] + np.arange(T, dtype=np.int32)[None, :]).astype(np.int32)
    cap = int(past.max()) + T + cap_extra
    kc, vc = decode_cache_host(w, past, cap, seed=(w.seed if seed is None else seed) + 1)
    for b, P in enumerate(past):   # slots >= past hold NaN: written or never read
        kc[b, :, P:] = np.nan
        vc[b, :, P:] = np.nan
    return w, inp, past, kc, vc


def run_chunk_gpu(w, inp, past, kc_host, vc_host):
    import torch
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    pl = torch.from_numpy(past).to("cuda")
    kc, vc = dev(kc_host, w.dtype), dev(vc_host, w.dtype)
    y = blk.prefill_chunk(x, pos, pl, kc, vc)
    torch.cuda.synchronize()
    out = dict(Y=host(y), Kc=host(kc), Vc=host(vc))
    blk.close()
    return out


def oracle_chunk(w, inp, past, kc, vc):
    return oracle.prefill_chunk(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                                inp["gk"], inp["positions"], past, kc, vc, n_q=w.n_q, n_kv=w.n_kv,
                                eps=EPS, theta=ROPE_THETA)


CHUNK_CASES = [
    (1, 1, 58, [70]),            # fp32, past not a multiple of the 32-key tile
    (2, 2, 150, [37, 300]),      # 0.6B shape, ragged past lengths
    (2, 3, 1, [0, 64, 1000]),    # one-token chunks (decode-like), incl. an empty cache
    (3, 2, 64, [0, 129]),        # 4B shape (n_rep 4)
    (4, 1, 65, [200]),           # wide GQA (n_rep 16)
]


@pytest.mark.parametrize("idx,B,T,past", CHUNK_CASES)
def test_prefill_chunk_parity(idx, B, T, past):
    w, inp, past, kc, vc = chunk_case(idx, B, T, past)
    say(f"chunked prefill parity: workload {idx} ({w.name}) B={B} T={T} past={past.tolist()}")
    got = run_chunk_gpu(w, inp, past, kc, vc)
    ref = oracle_chunk(w, inp, past, kc, vc)
    for b, P in enumerate(past):
        # cached slots untouched, the chunk's slots written, the rest untouched
        np.testing.assert_array_equal(got["Kc"][b, :, :P], kc[b, :, :P])
        np.testing.assert_array_equal(got["Vc"][b, :, :P], vc[b, :, :P])
        assert_close(got["Kc"][b, :, P:P + T], ref["Kc"][b], w.dtype, f"k cache chunk (seq {b})")
        assert_close(got["Vc"][b, :, P:P + T], ref["Vc"][b], w.dtype, f"v cache chunk (seq {b})")
        assert np.all(np.isnan(got["Kc"][b, :, P + T:])), "slots past the chunk were written"
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y")


def test_prefill_chunk_after_prefill_equals_one_shot():
    # On the GPU: prefill of P tokens, then the next T tokens as a chunk over
    # the same caches, against one prefill of all P+T tokens.
    import torch
    w = WORKLOADS[2]
    P, T = 200, 137
    inp = prefill_inputs(w, B=2, T=P + T)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    cap = P + T + 8
    kc1 = torch.zeros((2, w.n_kv, cap, 128), dtype=x.dtype, device="cuda")
    vc1 = torch.zeros_like(kc1)
    y_full = blk.prefill(x, pos, kc1, vc1)
    kc2, vc2 = torch.zeros_like(kc1), torch.zeros_like(kc1)
    blk.prefill(x[:, :P].contiguous(), pos[:, :P].contiguous(), kc2, vc2)
    past = torch.full((2,), P, dtype=torch.int32, device="cuda")
    y_tail = blk.prefill_chunk(x[:, P:].contiguous(), pos[:, P:].contiguous(), past, kc2, vc2)
    torch.cuda.synchronize()
    assert_close(host(y_tail), host(y_full)[:, P:], w.dtype, "Y chunk vs one-shot")
    np.testing.assert_array_equal(host(kc2), host(kc1))
    np.testing.assert_array_equal(host(vc2), host(vc1))
    blk.close()


def test_prefill_chunk_full_size_0p6b():
    # The 0.6B shape: a 512-token chunk per sequence over 1536 cached tokens.
    w, inp, past, kc, vc = chunk_case(2, 2, 512, [1536, 1536], cap_extra=0)
    say("chunked prefill full size: 0.6B B=2 T=512 past=1536")
    got = run_chunk_gpu(w, inp, past, kc, vc)
    ref = oracle_chunk(w, inp, past, kc, vc)
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y")
    assert_close(got["Kc"][:, :, 1536:], ref["Kc"], w.dtype, "k cache chunk")


# fp32: a_j rises for the whole cache and the spike is 3000.  bf16: a_j
# stops after 4 steps and the spike sits 100 above it -- a score difference
# between two competing keys carries the bf16 rounding of q~ times their
# difference in a (relative 2^-9), which must stay well inside the bf16 bar.
RISE_CASES = [(1, None, 3000.0), (2, 4, 260.0)]


@pytest.mark.parametrize("idx,steps,spike", RISE_CASES)
def test_prefill_chunk_scores_rising_past_the_rescale_slack(idx, steps, spike):
    # The flash kernel keeps a reference max that may trail a query's running
    # max by up to 8 (log2 units) and rescales O and the sum only past that.
    # Cached keys k_j = a_j u_g + e_j, with a_j rising by 40 every 64 keys
    # (for `steps` steps) and one key at spike * u_g three slots before the
    # end of sequence 0, make a query's max jump by 40 (q.u) log2(e)/sqrt(d)
    # per 64 keys: past the slack for some queries, within it for others,
    # and again at the spike.  Queries with q.u < 0 keep their max in the
    # first tile, and the chunk's own keys dominate them.
    w, inp, past, kc, vc = chunk_case(idx, 2, 100, [1000, 700])
    rng = np.random.default_rng(7)
    store = (lambda a: bf16_bits_to_f32(round_to_bf16_bits(a.astype(np.float32)))) \
        if w.dtype == "bf16" else (lambda a: a.astype(np.float32))
    U = rng.standard_normal((2, w.n_kv, 128))
    U /= np.linalg.norm(U, axis=-1, keepdims=True)
    for b, P in enumerate(past):
        step = np.arange(P) // 64
        a = 40.0 * (step if steps is None else np.minimum(step, steps))
        kc[b, :, :P] = store(a[None, :, None] * U[b][:, None, :] + kc[b, :, :P])
    kc[0, :, past[0] - 3] = store(spike * U[0])
    say(f"chunked prefill, rising scores: workload {idx} ({w.name}) B=2 T=100 "
        f"past={past.tolist()} steps={steps} spike={spike}")
    got = run_chunk_gpu(w, inp, past, kc, vc)
    ref = oracle_chunk(w, inp, past, kc, vc)
    # both sides of the slack occur: per-64-key jumps above 8 and in (0, 8]
    rep = w.n_q // w.n_kv
    qu = np.einsum("bthd,bhd->bth", ref["Q"], np.repeat(U, rep, axis=1))
    jump = 40.0 * qu * Q_WS_SCALE
    assert np.mean(jump > 8) > 0.02 and np.mean((jump > 0) & (jump <= 8)) > 0.2
    assert_close(got["Y"], ref["Y"], w.dtype, "block output Y")


def test_prefill_chunk_argument_errors():
    import torch
    import qwen3_gqa_attention_amd as q3
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=1, T=8)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.zeros((1, w.n_kv, 16, 128), dtype=x.dtype, device="cuda")
    ws = torch.empty(blk.workspace_size(False, 1, 8), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    st = q3.qwen3_attn_forward_prefill_chunk(blk.handle, x.data_ptr(), pos.data_ptr(), None,
                                             kc.data_ptr(), kc.data_ptr(), 16, out.data_ptr(), 1, 8,
                                             ws.data_ptr(), ws.numel(), None)
    assert st == 1   # EINVAL: past_len missing
    blk.close()


# ------------------------------------------------------------------------- decode
def run_decode_gpu(w, inp, kc_host, vc_host, cap):
    import torch
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = dev(kc_host, w.dtype)
    vc = dev(vc_host, w.dtype)
    y = blk.decode(x, pos, kc, vc)
    torch.cuda.synchronize()
    out = dict(Y=host(y), kc=kc, vc=vc)
    blk.close()
    return out


def check_decode(w, inp, kc_host, vc_host, got):
    ref = oracle.decode(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"], inp["gk"],
                        inp["positions"], kc_host, vc_host, n_q=w.n_q, n_kv=w.n_kv, eps=EPS,
                        theta=ROPE_THETA)
    assert_close(got["Y"], ref["Y"], w.dtype, "decode Y")
    L = inp["positions"]
    kc = host(got["kc"])
    vc = host(got["vc"])
    k_new = np.stack([kc[s, :, L[s]] for s in range(len(L))])
    v_new = np.stack([vc[s, :, L[s]] for s in range(len(L))])
    assert_close(k_new, ref["k_new"], w.dtype, "new k in cache slot L")
    assert_close(v_new, ref["v_new"], w.dtype, "new v in cache slot L")
    # the cached prefix is untouched
    for s in range(len(L)):
        np.testing.assert_array_equal(kc[s, :, : L[s]], kc_host[s, :, : L[s]])


@pytest.mark.parametrize("dtype,n_q,n_kv", [("bf16", 16, 8), ("f32", 16, 8), ("bf16", 32, 8),
                                            ("bf16", 64, 4), ("bf16", 40, 8), ("bf16", 8, 8),
                                            ("bf16", 24, 8), ("bf16", 48, 8)])
def test_decode_parity_ragged(dtype, n_q, n_kv):
    w = dataclasses.replace(WORKLOADS[5], dtype=dtype, n_q=n_q, n_kv=n_kv)
    say(f"decode parity: dtype={dtype} n_q={n_q} n_kv={n_kv}")
    lens = np.array([0, 1, 127, 511, 512, 513, 1030, 2047], np.int32)
    inp = decode_inputs(w, N=len(lens))
    inp["positions"] = lens
    cap = 2112
    kc, vc = decode_cache_host(w, lens, cap)
    got = run_decode_gpu(w, inp, kc, vc, cap)
    check_decode(w, inp, kc, vc, got)


@pytest.mark.parametrize("N", [1, 64, 65])
def test_decode_batch_sizes_at_the_projection_path_edges(N):
    # N <= 64 runs the projections split-K (one 64-row tile, ragged for N < 64);
    # N = 65 is the smallest batch on the tiled path (a one-row second tile).
    w = WORKLOADS[5]
    say(f"decode batch-size edge: N={N}")
    lens = np.random.default_rng(100 + N).integers(0, 600, size=N).astype(np.int32)
    inp = decode_inputs(w, N=N)
    inp["positions"] = lens
    cap = 640
    kc, vc = decode_cache_host(w, lens, cap)
    got = run_decode_gpu(w, inp, kc, vc, cap)
    check_decode(w, inp, kc, vc, got)


def test_decode_full_size_sampled_sequences():
    # 64 sequences with caches of 1024..32768 tokens (several GB); the caches
    # are drawn on the device with torch's seeded generator, sampled
    # sequences are copied back and checked one by one.
    import torch
    w = WORKLOADS[5]
    say(f"decode parity full size: {w.name}")
    inp = decode_inputs(w)
    L = inp["positions"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    kc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    vc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    y = blk.decode(dev(inp["X"], w.dtype), torch.from_numpy(L).to("cuda"), kc, vc)
    torch.cuda.synchronize()
    Y = host(y)
    picks = sorted({int(np.argmin(L)), int(np.argmax(L)), 0, 17, 42, 63})
    for s in picks:
        Ls = int(L[s])
        k_all = host(kc[s, :, : Ls + 1])   # includes the new token's slot
        v_all = host(vc[s, :, : Ls + 1])
        sub = {k: (v[s:s + 1] if k in ("X", "positions") else v) for k, v in inp.items() if k != "lengths"}
        ref = oracle.decode(sub["X"], sub["Wq"], sub["Wk"], sub["Wv"], sub["Wo"], sub["gq"], sub["gk"],
                            sub["positions"], k_all[None, :, :Ls], v_all[None, :, :Ls], n_q=w.n_q,
                            n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA)
        assert_close(Y[s:s + 1], ref["Y"], w.dtype, f"decode Y seq {s} (L={Ls})")
        assert_close(k_all[:, Ls], ref["k_new"][0], w.dtype, f"new k seq {s}")
    blk.close()
    del kc, vc
    torch.cuda.empty_cache()


# ------------------------------------------------- input RMSNorm + residual fused
def layer_block(inp, w, g_in):
    import qwen3_gqa_attention_amd as q3m
    return q3m.Qwen3Attention(dev(inp["Wq"], w.dtype), dev(inp["Wk"], w.dtype), dev(inp["Wv"], w.dtype),
                              dev(inp["Wo"], w.dtype), dev(inp["gq"], w.dtype), dev(inp["gk"], w.dtype),
                              n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA,
                              input_norm=dev(g_in, w.dtype))


def input_gain(w, d, seed):
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    g = (1 + 0.1 * np.random.default_rng(seed).standard_normal(d)).astype(np.float32)
    return bf16_bits_to_f32(round_to_bf16_bits(g)) if w.dtype == "bf16" else g


@pytest.mark.parametrize("idx,B,T", [(1, 1, 128), (2, 2, 300), (4, 1, 100), (2, 1, 40)])
def test_layer_prefill_parity(idx, B, T):
    import torch
    w = WORKLOADS[idx]
    say(f"layer prefill parity (input norm + residual): {w.name} B={B} T={T}")
    inp = prefill_inputs(w, B=B, T=T)
    g_in = input_gain(w, w.d, 7 + idx)
    blk = layer_block(inp, w, g_in)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.full((B, w.n_kv, T + 8, 128), float("nan"), dtype=x.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    y = blk.prefill(x, pos, kc, vc)
    torch.cuda.synchronize()
    ref = oracle.prefill_residual(inp["X"], g_in, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                                  inp["gq"], inp["gk"], inp["positions"], n_q=w.n_q, n_kv=w.n_kv,
                                  eps=EPS, theta=ROPE_THETA)
    assert_close(host(kc)[:, :, :T], ref["Kc"], w.dtype, "k cache")
    assert_close(host(vc)[:, :, :T], ref["Vc"], w.dtype, "v cache")
    floor = storage_floor_prefill(inp, w, B, T, g_in=g_in) if w.dtype == "bf16" else None
    assert_close(host(y), ref["Y"], w.dtype, "layer output x + block(norm(x))", floor=floor)
    blk.close()


def test_layer_prefill_full_size_0p6b():
    # The 0.6B shape at full size: o_proj with the residual runs one 128x128
    # tile per CU, with the K range split over two wave groups.
    import torch
    w = WORKLOADS[2]
    say(f"layer prefill parity full size: {w.name}")
    inp = prefill_inputs(w)
    g_in = input_gain(w, w.d, 29)
    blk = layer_block(inp, w, g_in)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.empty((w.B, w.n_kv, w.T, 128), dtype=x.dtype, device="cuda")
    vc = torch.empty_like(kc)
    y = host(blk.prefill(x, pos, kc, vc))
    torch.cuda.synchronize()
    ref = oracle.prefill_residual(inp["X"], g_in, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                                  inp["gq"], inp["gk"], inp["positions"], n_q=w.n_q, n_kv=w.n_kv,
                                  eps=EPS, theta=ROPE_THETA)
    assert_close(host(kc), ref["Kc"], w.dtype, "k cache")
    assert_close(y, ref["Y"], w.dtype, "layer output x + block(norm(x))")
    blk.close()


def test_layer_prefill_full_size_4b_sampled_rows():
    # The 4B shape at full size (T=4096): the q/k/v GEMM with the fused input
    # norm on 256x128 tiles and o_proj with the residual on 256x256 tiles.
    import torch
    w = WORKLOADS[3]
    say(f"layer prefill parity full size, sampled rows: {w.name}")
    inp = prefill_inputs(w)
    g_in = input_gain(w, w.d, 23)
    blk = layer_block(inp, w, g_in)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.empty((1, w.n_kv, w.T, 128), dtype=x.dtype, device="cuda")
    vc = torch.empty_like(kc)
    y = host(blk.prefill(x, pos, kc, vc))
    torch.cuda.synchronize()
    ts = [0, 1, 255, 256, 2047, 4095]
    xn = oracle.rms_norm(inp["X"].astype(np.float64), g_in, EPS)
    ref = oracle.prefill_rows(xn, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"], inp["gk"],
                              inp["positions"], [(0, t) for t in ts], n_q=w.n_q, n_kv=w.n_kv,
                              eps=EPS, theta=ROPE_THETA)
    assert_close(host(kc)[0], ref["Kc"][0], w.dtype, "k cache (all tokens)")
    floor = storage_floor_rows(inp["X"][0], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                               inp["gk"], inp["positions"][0], ts, n_q=w.n_q, n_kv=w.n_kv,
                               g_in=g_in)
    assert_close(np.stack([y[0, t] for t in ts]),
                 ref["Y"] + inp["X"][0, ts].astype(np.float64), w.dtype, "layer Y at sampled rows",
                 floor=floor)
    blk.close()


@pytest.mark.parametrize("dtype,N", [("bf16", 8), ("f32", 8), ("bf16", 100)])
def test_layer_decode_parity(dtype, N):
    import torch
    w = dataclasses.replace(WORKLOADS[5], dtype=dtype)
    say(f"layer decode parity: dtype={dtype} N={N}")
    lens = (np.arange(N, dtype=np.int32) * 131) % 2000
    inp = decode_inputs(w, N=N)
    inp["positions"] = lens
    cap = 2048
    kc, vc = decode_cache_host(w, lens, cap)
    g_in = input_gain(w, w.d, 17)
    blk = layer_block(inp, w, g_in)
    kcd, vcd = dev(kc, w.dtype), dev(vc, w.dtype)
    y = blk.decode(dev(inp["X"], w.dtype), torch.from_numpy(lens).to("cuda"), kcd, vcd)
    torch.cuda.synchronize()
    ref = oracle.decode_residual(inp["X"], g_in, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                                 inp["gq"], inp["gk"], lens, kc, vc, n_q=w.n_q, n_kv=w.n_kv,
                                 eps=EPS, theta=ROPE_THETA)
    assert_close(host(y), ref["Y"], w.dtype, "layer decode output")
    kh = host(kcd)
    assert_close(np.stack([kh[s, :, lens[s]] for s in range(N)]), ref["k_new"], w.dtype, "new k")
    blk.close()


# --------------------------------------------------------------------- paged KV
@pytest.mark.parametrize("dtype,bs", [("bf16", 64), ("bf16", 256), ("f32", 128)])
def test_decode_paged_parity(dtype, bs):
    import torch
    w = dataclasses.replace(WORKLOADS[5], dtype=dtype)
    say(f"paged decode parity: dtype={dtype} block_size={bs}")
    lens = np.array([0, 1, 63, 64, 65, 511, 1030, 2047], np.int32)
    inp = decode_inputs(w, N=len(lens))
    inp["positions"] = lens
    cap = 2112
    kc, vc = decode_cache_host(w, lens, cap)
    kp, vp, table = to_paged(kc, vc, lens + 1, bs, seed=bs)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    kpd, vpd = dev(kp, w.dtype), dev(vp, w.dtype)
    y = blk.decode_paged(dev(inp["X"], w.dtype), torch.from_numpy(lens).to("cuda"),
                         torch.from_numpy(table).to("cuda"), kpd, vpd)
    torch.cuda.synchronize()
    kp_got, vp_got = host(kpd), host(vpd)
    ref = oracle.decode(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"], inp["gk"],
                        lens, kc, vc, n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA)
    assert_close(host(y), ref["Y"], w.dtype, "paged decode Y")
    for s, L in enumerate(lens):
        k_all = from_paged(kp_got, table, s, int(L) + 1)
        v_all = from_paged(vp_got, table, s, int(L) + 1)
        np.testing.assert_array_equal(k_all[:, :L], kc[s, :, :L])
        assert_close(k_all[:, L], ref["k_new"][s], w.dtype, f"new k seq {s}")
        assert_close(v_all[:, L], ref["v_new"][s], w.dtype, f"new v seq {s}")
    # the contiguous path gives the same result bit for bit
    got_c = run_decode_gpu(w, inp, kc, vc, cap)
    np.testing.assert_array_equal(host(y), got_c["Y"])
    used = set(table[s, i] for s in range(len(lens)) for i in range((int(lens[s]) + bs) // bs))
    for b in range(kp.shape[0]):
        if b not in used:
            assert np.all(np.isnan(kp_got[b])), "a block outside the tables was written"
    blk.close()


@pytest.mark.parametrize("dtype,bs,T,past", [("bf16", 64, 70, [0, 100, 300]),
                                             ("bf16", 128, 150, [37, 1000]),
                                             ("f32", 64, 58, [70])])
def test_prefill_paged_parity(dtype, bs, T, past):
    import torch
    idx = 1 if dtype == "f32" else 2
    w, inp, past, kc, vc = chunk_case(idx, len(past), T, past)
    say(f"paged chunked prefill parity: {w.name} block_size={bs} T={T} past={past.tolist()}")
    kp, vp, table = to_paged(kc, vc, past + T, bs, seed=T)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    kpd, vpd = dev(kp, w.dtype), dev(vp, w.dtype)
    y = blk.prefill_paged(dev(inp["X"], w.dtype), torch.from_numpy(inp["positions"]).to("cuda"),
                          torch.from_numpy(past).to("cuda"), torch.from_numpy(table).to("cuda"),
                          kpd, vpd)
    torch.cuda.synchronize()
    ref = oracle_chunk(w, inp, past, kc, vc)
    assert_close(host(y), ref["Y"], w.dtype, "paged chunked prefill Y")
    kp_got, vp_got = host(kpd), host(vpd)
    for b, P in enumerate(past):
        k_all = from_paged(kp_got, table, b, int(P) + T)
        v_all = from_paged(vp_got, table, b, int(P) + T)
        np.testing.assert_array_equal(k_all[:, :P], kc[b, :, :P])
        assert_close(k_all[:, P:], ref["Kc"][b], w.dtype, f"k chunk seq {b}")
        assert_close(v_all[:, P:], ref["Vc"][b], w.dtype, f"v chunk seq {b}")
    got_c = run_chunk_gpu(w, inp, past, kc, vc)
    np.testing.assert_array_equal(host(y), got_c["Y"])
    blk.close()


def test_decode_paged_full_size_matches_contiguous():
    # 64 sequences of 1024..32768 cached tokens in 64-token blocks laid out in
    # a shuffled pool, against the contiguous call on the same caches (that
    # path is checked against the oracle at this size above).  The two split
    # the keys into chunks of different lengths (512 over a paged pool, 2048
    # over a contiguous cache of this size), so their log-sum-exp merges add
    # the same terms in a different order: Y agrees to the bf16 bar, and the
    # new token's K/V rows, written by the same projection kernel, are
    # identical.
    import torch
    w = WORKLOADS[5]
    say(f"paged decode full size: {w.name}")
    inp = decode_inputs(w)
    L = inp["positions"]
    bs = 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 3)
    kc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((w.B, w.n_kv, w.cap, 128), generator=gen, device="cuda").to(torch.bfloat16)
    mb = w.cap // bs
    nb = w.B * mb
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(5)).to("cuda")
    table = perm.view(w.B, mb).to(torch.int32).contiguous()
    kp = torch.empty((nb, w.n_kv, bs, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    # block (s, i) of the contiguous cache -> pool[table[s, i]]
    kp[table.view(-1).long()] = kc.view(w.B, w.n_kv, mb, bs, 128).permute(0, 2, 1, 3, 4).reshape(nb, w.n_kv, bs, 128)
    vp[table.view(-1).long()] = vc.view(w.B, w.n_kv, mb, bs, 128).permute(0, 2, 1, 3, 4).reshape(nb, w.n_kv, bs, 128)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(L).to("cuda")
    y_p = blk.decode_paged(x, pos, table, kp, vp)
    y_c = blk.decode(x, pos, kc, vc)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(y_p)))
    assert_close(host(y_p), host(y_c), w.dtype, "paged vs contiguous Y")
    seq = torch.arange(w.B, device="cuda")
    posl = pos.long()
    phys = table[seq, posl // bs].long()
    for pool, cache, what in ((kp, kc, "k"), (vp, vc, "v")):
        new_p = pool[phys, :, posl % bs]             # [B, n_kv, 128]
        new_c = cache[seq, :, posl]
        assert torch.equal(new_p, new_c), f"new {what} rows differ"
    blk.close()
    del kc, vc, kp, vp
    torch.cuda.empty_cache()


def test_paged_argument_errors():
    import torch
    import qwen3_gqa_attention_amd as q3
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=1, T=8)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    pool = torch.zeros((4, w.n_kv, 64, 128), dtype=x.dtype, device="cuda")
    table = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    ws = torch.empty(blk.workspace_size(False, 1, 8), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    P = lambda t: t.data_ptr()
    f = q3.qwen3_attn_forward_prefill_paged
    for bs in (32, 96, 0):   # not a power of two >= 64
        assert f(blk.handle, P(x), P(pos), None, P(table), 4, P(pool), P(pool), bs, P(out), 1, 8,
                 P(ws), ws.numel(), None) == 1
    assert f(blk.handle, P(x), P(pos), None, None, 4, P(pool), P(pool), 64, P(out), 1, 8,
             P(ws), ws.numel(), None) == 1                    # no block table
    assert f(blk.handle, P(x), P(pos), None, P(table), 0, P(pool), P(pool), 64, P(out), 1, 8,
             P(ws), ws.numel(), None) == 1                    # max_blocks 0
    blk.close()


def test_decode_equals_last_prefill_row_on_gpu():
    import torch
    w = WORKLOADS[2]
    T = 301
    inp = prefill_inputs(w, B=2, T=T)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    cap = 384
    kc = torch.zeros((2, w.n_kv, cap, 128), dtype=x.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    y = blk.prefill(x, torch.from_numpy(inp["positions"]).to("cuda"), kc, vc)
    kc2 = kc.clone()
    vc2 = vc.clone()
    kc2[:, :, T - 1:] = 0
    vc2[:, :, T - 1:] = 0
    yd = blk.decode(x[:, T - 1].contiguous(), torch.full((2,), T - 1, dtype=torch.int32, device="cuda"), kc2, vc2)
    torch.cuda.synchronize()
    assert_close(host(yd), host(y[:, T - 1]), w.dtype, "decode vs last prefill row")
    # the same key computed by the decode and the prefill projections
    # (different accumulation orders, so equal up to bf16 rounding)
    assert_close(host(kc2[:, :, T - 1]), host(kc[:, :, T - 1]), w.dtype, "new k: decode vs prefill")
    blk.close()


# ---------------------------------------------------------------- host-side errors
def test_forward_argument_errors():
    import torch
    import qwen3_gqa_attention_amd as q3
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=1, T=8)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.zeros((1, w.n_kv, 16, 128), dtype=x.dtype, device="cuda")
    out = torch.empty_like(x)
    need = blk.workspace_size(False, 1, 8)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    f = q3.qwen3_attn_forward_prefill
    assert f(blk.handle, P(x), P(pos), P(kc), P(kc), 16, P(out), 1, 8, P(ws), need - 1, s) == 4
    assert f(blk.handle, P(x), P(pos), P(kc), P(kc), 16, P(out), 1, 8, None, need, s) == 4
    assert f(blk.handle, P(x), P(pos), P(kc), P(kc), 7, P(out), 1, 8, P(ws), need, s) == 1   # T > cap
    assert f(blk.handle, P(x), P(pos), P(kc), P(kc), 16, P(out), 0, 8, P(ws), need, s) == 1
    assert f(blk.handle, None, P(pos), P(kc), P(kc), 16, P(out), 1, 8, P(ws), need, s) == 1
    assert f(blk.handle, P(x), P(pos), P(kc), P(kc), 16, P(out), 1, 8, P(ws), need, s) == 0
    torch.cuda.synchronize()
    # the binding checks hidden's width against the handle's d_model (the C ABI cannot)
    x_narrow = x[..., : w.d // 2].contiguous()
    with pytest.raises(ValueError):
        blk.prefill(x_narrow, pos, kc, kc.clone())
    with pytest.raises(ValueError):
        blk.decode(x_narrow[0], torch.zeros(8, dtype=torch.int32, device="cuda"),
                   torch.zeros((8, w.n_kv, 16, 128), dtype=x.dtype, device="cuda"),
                   torch.zeros((8, w.n_kv, 16, 128), dtype=x.dtype, device="cuda"))
    blk.close()
    # decode with an n_rep the decode kernel does not instantiate
    w7 = dataclasses.replace(w, n_q=14, n_kv=2)
    inp7 = prefill_inputs(w7, B=1, T=1)
    b7 = block_from_inputs(inp7, 14, 2, "bf16")
    with pytest.raises(q3.Qwen3AttnError) as e:
        b7.decode(dev(inp7["X"][0], "bf16"), torch.zeros(1, dtype=torch.int32, device="cuda"),
                  torch.zeros((1, 2, 16, 128), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((1, 2, 16, 128), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 2
    b7.close()
