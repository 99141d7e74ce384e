"""GPU test of qwen3_attn_forward_decode_noalloc, through the C ABI.

The allocation-free decode must give what qwen3_attn_forward_decode gives
with a caller workspace: the same output and the same cache writes, bit for
bit, on two calls in a row (the second smaller, so it runs over what the first
left in the shared scratch array), and it must reject a call whose scratch
need exceeds the array before launching anything."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import qwen3_gqa_attention_amd as q3
from gpu_util import assert_close, block_from_inputs, dev, host, say
from workloads import EPS, ROPE_THETA, WORKLOADS, decode_cache_host, decode_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def decode_both(blk, w, N, cap, seed):
    """One decode step through both entry points on identical cache copies
    (hidden states and caches drawn for this call; the handle's weights fixed)."""
    import torch
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, cap, size=N).astype(np.int32)
    xs = decode_inputs(w, N=N, seed=seed)["X"]
    kc, vc = decode_cache_host(w, lens, cap, seed=seed)
    x = dev(xs, w.dtype)
    pos = torch.from_numpy(lens).to("cuda")
    k_a, v_a = dev(kc, w.dtype), dev(vc, w.dtype)
    k_b, v_b = k_a.clone(), v_a.clone()
    out_a = torch.full_like(x, float("nan"))
    out_b = torch.full_like(x, float("nan"))
    nbytes = blk.workspace_size(True, N, 1, cap)
    assert nbytes <= q3.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = q3.qwen3_attn_forward_decode(blk.handle, x.data_ptr(), pos.data_ptr(), k_a.data_ptr(),
                                      v_a.data_ptr(), cap, out_a.data_ptr(), N, ws.data_ptr(),
                                      nbytes, stream)
    assert st == 0, q3.qwen3_attn_status_string(st)
    st = q3.qwen3_attn_forward_decode_noalloc(blk.handle, x.data_ptr(), pos.data_ptr(),
                                              k_b.data_ptr(), v_b.data_ptr(), cap,
                                              out_b.data_ptr(), N, stream)
    assert st == 0, q3.qwen3_attn_status_string(st)
    torch.cuda.synchronize()
    return xs, lens, kc, vc, dict(out=host(out_a), k=host(k_a), v=host(v_a)), \
        dict(out=host(out_b), k=host(k_b), v=host(v_b))


def test_noalloc_decode_equals_the_workspace_call_twice_then_smaller():
    w = WORKLOADS[5]
    inp = decode_inputs(w)     # the handle's weights
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    for N, cap, seed in ((64, 4160, 5), (7, 600, 6)):
        say(f"no-alloc decode vs workspace decode: N={N} cap={cap}")
        xs, lens, kc, vc, a, b = decode_both(blk, w, N, cap, seed)
        for key in ("out", "k", "v"):
            assert np.array_equal(a[key], b[key], equal_nan=True), key
        assert np.all(np.isfinite(b["out"]))
        # and both against the oracle on two sequences (the shortest and longest)
        for s in (int(np.argmin(lens)), int(np.argmax(lens))):
            ref = oracle.decode(xs[s:s + 1], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                                inp["gq"], inp["gk"], lens[s:s + 1], kc[s:s + 1], vc[s:s + 1],
                                n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA)
            assert_close(b["out"][s:s + 1], ref["Y"], w.dtype, f"no-alloc decode Y (seq {s})")
    blk.close()


def test_noalloc_decode_rejects_a_call_larger_than_its_scratch():
    import torch
    w = WORKLOADS[5]
    inp = decode_inputs(w, N=2)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    N, cap = 64, 1000000      # per-chunk partials alone need about 260 MB
    assert blk.workspace_size(True, N, 1, cap) > q3.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((N, w.d), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(N, dtype=torch.int32, device="cuda")
    kc = torch.zeros((1,), dtype=torch.bfloat16, device="cuda")   # never touched: rejected first
    out = torch.full_like(x, float("nan"))
    st = q3.qwen3_attn_forward_decode_noalloc(blk.handle, x.data_ptr(), pos.data_ptr(),
                                              kc.data_ptr(), kc.data_ptr(), cap, out.data_ptr(),
                                              N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert q3.STATUS[st] == "EWORKSPACE"
    assert torch.isnan(out.float()).all()          # nothing was launched
    assert q3.qwen3_attn_forward_decode_noalloc(None, x.data_ptr(), pos.data_ptr(), kc.data_ptr(),
                                                kc.data_ptr(), 64, out.data_ptr(), 1, None) == 1
    blk.close()
