"""GPU parity of variable-length batches, through the C ABI, against the oracle.

The requests of a batch have different lengths and are packed one after
another into a single token list with row offsets cu_seqlens; each request
attends only to its own keys ("Assembling a large model from scratch",
section "Inference view": the tokens of many requests form one batch, with
attention computed per request).  The oracle runs each request on its own
(its chunked prefill over that request's cache).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import (assert_close, block_from_inputs, dev, from_paged, host, say,
                      storage_floor_rows, to_paged)
from workloads import (EPS, ROPE_THETA, WORKLOADS, bf16_bits_to_f32, decode_cache_host,
                       prefill_inputs, round_to_bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def varlen_case(idx, lens, past, *, seed=None, cap_extra=8):
    """Packed inputs of requests with lengths `lens` over caches holding
    `past` tokens; cache slots from past[b] on hold NaN (written or never read)."""
    w = WORKLOADS[idx]
    lens = np.asarray(lens, np.int32)
    past = np.asarray(past, np.int32)
    total = int(lens.sum())
    inp = prefill_inputs(w, B=1, T=total, seed=seed)
    inp["X"] = inp["X"][0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp["positions"] = np.concatenate(
        [p + np.arange(n, dtype=np.int32) for p, n in zip(past, lens)]).astype(np.int32)
    cap = int((past + lens).max()) + cap_extra
    kc, vc = decode_cache_host(w, past, cap, seed=w.seed + 1)
    for b, P in enumerate(past):
        kc[b, :, P:] = np.nan
        vc[b, :, P:] = np.nan
    return w, inp, lens, past, cu, kc, vc


def oracle_varlen(w, inp, lens, past, cu, kc, vc, *, window=None, g_in=None):
    """Each request through the oracle's chunked prefill on its own; with g_in
    the input RMSNorm and residual add around it."""
    Y, Kc, Vc = [], [], []
    for b, n in enumerate(lens):
        x = inp["X"][cu[b]:cu[b + 1]][None].astype(np.float64)
        xin = x if g_in is None else oracle.rms_norm(x, g_in, EPS)
        if n == 0:
            Y.append(np.zeros((0, w.d)))
            Kc.append(None)
            Vc.append(None)
            continue
        r = oracle.prefill_chunk(xin, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                                 inp["gk"], inp["positions"][cu[b]:cu[b + 1]][None], [past[b]],
                                 kc[b:b + 1], vc[b:b + 1], n_q=w.n_q, n_kv=w.n_kv, eps=EPS,
                                 theta=ROPE_THETA, window=window)
        Y.append(r["Y"][0] + (0 if g_in is None else x[0]))
        Kc.append(r["Kc"][0])
        Vc.append(r["Vc"][0])
    return np.concatenate(Y), Kc, Vc


def run_varlen_gpu(w, inp, lens, past, cu, kc, vc, *, with_past=True, **kw):
    import torch
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype, **kw)
    kcd, vcd = dev(kc, w.dtype), dev(vc, w.dtype)
    y = blk.prefill_varlen(dev(inp["X"], w.dtype), torch.from_numpy(inp["positions"]).to("cuda"),
                           torch.from_numpy(cu).to("cuda"), kcd, vcd, max_seqlen=int(lens.max()),
                           past_len=torch.from_numpy(past).to("cuda") if with_past else None)
    torch.cuda.synchronize()
    out = dict(Y=host(y), Kc=host(kcd), Vc=host(vcd))
    blk.close()
    return out


def check_caches(w, got, kc, lens, past, ref_k, ref_v):
    for b, (P, n) in enumerate(zip(past, lens)):
        np.testing.assert_array_equal(got["Kc"][b, :, :P], kc[b, :, :P])
        if n:
            assert_close(got["Kc"][b, :, P:P + n], ref_k[b], w.dtype, f"k cache (request {b})")
            assert_close(got["Vc"][b, :, P:P + n], ref_v[b], w.dtype, f"v cache (request {b})")
        assert np.all(np.isnan(got["Kc"][b, :, P + n:])), "slots past the request were written"


VARLEN_CASES = [
    (2, [1, 37, 300, 0, 129], [0, 5, 100, 7, 1000]),   # bf16, incl. an empty request
    (1, [17, 128, 3], [0, 40, 0]),                      # fp32
    (3, [64, 130], [129, 0]),                            # 4B shape (n_rep 4)
    (4, [65, 200], [0, 300]),                            # wide GQA (n_rep 16)
    (2, [513, 64, 1000, 2], [0, 0, 0, 0]),               # one long request among short ones
]


@pytest.mark.parametrize("idx,lens,past", VARLEN_CASES)
def test_varlen_prefill_parity(idx, lens, past):
    w, inp, lens, past, cu, kc, vc = varlen_case(idx, lens, past)
    say(f"varlen prefill parity: {w.name} lens={lens.tolist()} past={past.tolist()}")
    got = run_varlen_gpu(w, inp, lens, past, cu, kc, vc)
    Y, rk, rv = oracle_varlen(w, inp, lens, past, cu, kc, vc)
    check_caches(w, got, kc, lens, past, rk, rv)
    floor = None
    if w.dtype == "bf16":
        floor = np.concatenate([
            storage_floor_rows(inp["X"][cu[b]:cu[b + 1]], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                               inp["gq"], inp["gk"], inp["positions"][cu[b]:cu[b + 1]],
                               list(range(n)), n_q=w.n_q, n_kv=w.n_kv,
                               past_k=kc[b][:, :past[b]], past_v=vc[b][:, :past[b]])
            for b, n in enumerate(lens) if n > 0])
    assert_close(got["Y"], Y, w.dtype, "packed output Y", floor=floor)


def test_varlen_without_past_equals_empty_caches():
    # past_len = NULL (empty caches: the attention may use the handle's score
    # bound as a fixed softmax reference) against past_len = 0 everywhere (a
    # running max): the same cache writes bit for bit, outputs that agree with
    # the oracle and with each other up to the rounding of P.
    w, inp, lens, past, cu, kc, vc = varlen_case(2, [100, 7, 260], [0, 0, 0])
    a = run_varlen_gpu(w, inp, lens, past, cu, kc, vc, with_past=False)
    b = run_varlen_gpu(w, inp, lens, past, cu, kc, vc, with_past=True)
    np.testing.assert_array_equal(a["Kc"], b["Kc"])
    np.testing.assert_array_equal(a["Vc"], b["Vc"])
    Y, _, _ = oracle_varlen(w, inp, lens, past, cu, kc, vc)
    assert_close(a["Y"], Y, w.dtype, "Y (no past_len)")
    assert_close(b["Y"], Y, w.dtype, "Y (past_len = 0)")
    assert_close(a["Y"], b["Y"], w.dtype, "Y, the two references against each other")


def test_varlen_equal_lengths_match_the_fixed_length_call_bitwise():
    import torch
    w, inp, lens, past, cu, kc, vc = varlen_case(2, [300, 300], [37, 500])
    got = run_varlen_gpu(w, inp, lens, past, cu, kc, vc)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    kcd, vcd = dev(kc, w.dtype), dev(vc, w.dtype)
    y = blk.prefill_chunk(dev(inp["X"].reshape(2, 300, w.d), w.dtype),
                          torch.from_numpy(inp["positions"].reshape(2, 300)).to("cuda"),
                          torch.from_numpy(past).to("cuda"), kcd, vcd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["Y"], host(y).reshape(600, w.d))
    np.testing.assert_array_equal(got["Kc"], host(kcd))
    blk.close()


def test_varlen_paged_parity():
    import torch
    w, inp, lens, past, cu, kc, vc = varlen_case(2, [1, 37, 300, 129], [0, 5, 100, 1000])
    bs = 64
    say(f"varlen paged prefill parity: lens={lens.tolist()} past={past.tolist()} block_size={bs}")
    kp, vp, table = to_paged(kc, vc, past + lens, bs, seed=9)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    kpd, vpd = dev(kp, w.dtype), dev(vp, w.dtype)
    y = blk.prefill_varlen(dev(inp["X"], w.dtype), torch.from_numpy(inp["positions"]).to("cuda"),
                           torch.from_numpy(cu).to("cuda"), kpd, vpd, max_seqlen=int(lens.max()),
                           past_len=torch.from_numpy(past).to("cuda"),
                           block_table=torch.from_numpy(table).to("cuda"))
    torch.cuda.synchronize()
    Y, rk, rv = oracle_varlen(w, inp, lens, past, cu, kc, vc)
    assert_close(host(y), Y, w.dtype, "packed output Y (paged)")
    kp_got = host(kpd)
    for b, (P, n) in enumerate(zip(past, lens)):
        k_all = from_paged(kp_got, table, b, int(P + n))
        np.testing.assert_array_equal(k_all[:, :P], kc[b, :, :P])
        assert_close(k_all[:, P:], rk[b], w.dtype, f"k rows (request {b})")
    got_c = run_varlen_gpu(w, inp, lens, past, cu, kc, vc)
    np.testing.assert_array_equal(host(y), got_c["Y"])
    blk.close()


def test_varlen_with_window_and_input_norm():
    # The other options of the handle apply to a packed batch as well.
    w, inp, lens, past, cu, kc, vc = varlen_case(2, [100, 300, 1], [50, 0, 900])
    g = (1 + 0.1 * np.random.default_rng(5).standard_normal(w.d)).astype(np.float32)
    g = bf16_bits_to_f32(round_to_bf16_bits(g))
    say("varlen prefill parity with sliding window 128 and the input RMSNorm + residual")
    got = run_varlen_gpu(w, inp, lens, past, cu, kc, vc, sliding_window=128,
                         input_norm=dev(g, w.dtype))
    Y, rk, _ = oracle_varlen(w, inp, lens, past, cu, kc, vc, window=128, g_in=g)
    assert_close(got["Y"], Y, w.dtype, "layer output Y")
    assert_close(got["Kc"][1, :, :300], rk[1], w.dtype, "k cache (request 1)")


def test_varlen_argument_errors():
    import torch
    import qwen3_gqa_attention_amd as q3
    w, inp, lens, past, cu, kc, vc = varlen_case(2, [10, 20], [0, 0])
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    cud = torch.from_numpy(cu).to("cuda")
    kcd, vcd = dev(kc, w.dtype), dev(vc, w.dtype)
    for max_seqlen in (0, 14, 31):      # < 1, B * max < total, > total
        with pytest.raises(q3.Qwen3AttnError):
            blk.prefill_varlen(x, pos, cud, kcd, vcd, max_seqlen=max_seqlen)
    with pytest.raises(q3.Qwen3AttnError):   # longest request beyond the cache
        blk.prefill_varlen(x, pos, cud, kcd[:, :, :16].contiguous(), vcd[:, :, :16].contiguous(),
                           max_seqlen=20)
    torch.cuda.synchronize()
    blk.close()
