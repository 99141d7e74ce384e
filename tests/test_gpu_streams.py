"""The forward calls allocate nothing, never synchronise the host and launch
only on the caller's stream.  So they can be captured in a HIP graph and
replayed, and two handles can run on two streams at once.  Each case is
checked bit for bit against the same call run eagerly on the default
stream."""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import block_from_inputs, dev, host, say
from workloads import WORKLOADS, decode_cache_host, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def prefill_case(T=300, seed=None):
    import torch
    w = WORKLOADS[2]
    inp = prefill_inputs(w, B=2, T=T, seed=seed)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(inp["positions"]).to("cuda")
    kc = torch.zeros((2, w.n_kv, T + 8, 128), dtype=x.dtype, device="cuda")
    return w, blk, x, pos, kc


def test_prefill_replays_from_a_hip_graph():
    import torch
    w, blk, x, pos, kc = prefill_case()
    say("prefill captured in a HIP graph, replayed three times")
    ws = torch.empty(blk.workspace_size(False, 2, 300), dtype=torch.uint8, device="cuda")
    ref_k, ref_v, ref_y = torch.zeros_like(kc), torch.zeros_like(kc), torch.empty_like(x)
    blk.prefill(x, pos, ref_k, ref_v, out=ref_y, workspace=ws)
    torch.cuda.synchronize()
    k, v, y = torch.zeros_like(kc), torch.zeros_like(kc), torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream before capture
        blk.prefill(x, pos, k, v, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.prefill(x, pos, k, v, out=y, workspace=ws)
    for r in range(3):
        for t in (k, v, y):   # eager work between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(ref_y), err_msg=f"replay {r}: Y")
        np.testing.assert_array_equal(host(k)[:, :, :300], host(ref_k)[:, :, :300],
                                      err_msg=f"replay {r}: k cache")
        np.testing.assert_array_equal(host(v)[:, :, :300], host(ref_v)[:, :, :300],
                                      err_msg=f"replay {r}: v cache")
    del g
    blk.close()


def test_decode_replays_from_a_hip_graph():
    import torch
    w = WORKLOADS[5]
    lens = np.array([0, 1, 513, 1030, 2047, 77, 600, 1999], np.int32)
    inp = decode_inputs(w, N=len(lens))
    inp["positions"] = lens
    kc_h, vc_h = decode_cache_host(w, lens, 2112)
    blk = block_from_inputs(inp, w.n_q, w.n_kv, w.dtype)
    say("decode (split-K projections) captured in a HIP graph, replayed three times")
    x = dev(inp["X"], w.dtype)
    pos = torch.from_numpy(lens).to("cuda")
    ws = torch.empty(blk.workspace_size(True, len(lens), 1, 2112), dtype=torch.uint8, device="cuda")
    ref_k, ref_v, ref_y = dev(kc_h, w.dtype), dev(vc_h, w.dtype), torch.empty_like(x)
    blk.decode(x, pos, ref_k, ref_v, out=ref_y, workspace=ws)
    torch.cuda.synchronize()
    k, v, y = dev(kc_h, w.dtype), dev(vc_h, w.dtype), torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blk.decode(x, pos, k, v, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.decode(x, pos, k, v, out=y, workspace=ws)
    for r in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(ref_y), err_msg=f"replay {r}: Y")
        np.testing.assert_array_equal(host(k), host(ref_k), err_msg=f"replay {r}: k cache")
    del g
    blk.close()


def test_two_handles_on_two_streams_match_sequential_runs():
    import torch
    say("two handles, two streams, concurrent prefill")
    cases = [prefill_case(T=300), prefill_case(T=300, seed=77)]
    outs = []
    for w, blk, x, pos, kc in cases:   # sequential reference on the default stream
        k, v = torch.zeros_like(kc), torch.zeros_like(kc)
        y = blk.prefill(x, pos, k, v, workspace=torch.empty(blk.workspace_size(False, 2, 300),
                                                            dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        outs.append((host(y), host(k)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    res = []
    for (w, blk, x, pos, kc), s in zip(cases, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            k, v = torch.zeros_like(kc), torch.zeros_like(kc)
            ws = torch.empty(blk.workspace_size(False, 2, 300), dtype=torch.uint8, device="cuda")
            for _ in range(3):
                y = blk.prefill(x, pos, k, v, workspace=ws)
            res.append((y, k))
    torch.cuda.synchronize()
    for (y, k), (ry, rk) in zip(res, outs):
        np.testing.assert_array_equal(host(y), ry)
        np.testing.assert_array_equal(host(k), rk)
    for c in cases:
        c[1].close()
