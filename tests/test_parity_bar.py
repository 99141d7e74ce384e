"""CPU checks of the GPU pass bar's storage-floor rule (tests/gpu_util.py).

The bf16 bar is |got_i - ref_i| <= 2e-2 * max(1, |ref_i| / 4).  Where exact
arithmetic that keeps the block's bf16 storage points (q~, k~, v in the bf16
caches, the bf16 attention probabilities, the bf16 o_proj input A, Y) already
misses it, a bf16 implementation
cannot meet it; these tests show on which workload that happens, with the
oracle alone (no GPU)."""
import numpy as np

import oracle
from gpu_util import FLOOR_ALLOWANCE, bf16, element_bars, storage_floor_rows
from workloads import EPS, ROPE_THETA, WORKLOADS, prefill_inputs


def floor_case(idx, T, **kw):
    w = WORKLOADS[idx]
    inp = prefill_inputs(w, B=1, T=T)
    ref = oracle.prefill(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"], inp["gk"],
                         inp["positions"], n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA, **kw)
    fl = storage_floor_rows(inp["X"][0], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"],
                            inp["gk"], inp["positions"][0], list(range(T)), n_q=w.n_q,
                            n_kv=w.n_kv, **kw)
    return ref["Y"][0], fl


def test_storage_floor_is_the_exact_result_up_to_bf16_storage():
    ref, fl = floor_case(2, 96)
    assert np.array_equal(fl, bf16(fl))                          # Y itself is bf16
    rel = np.linalg.norm(fl - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 5e-3                                      # a few bf16 roundings, no more


def test_storage_floor_meets_the_bar_on_the_0p6b_shape():
    ref, fl = floor_case(2, 300)
    assert np.max(np.abs(fl - ref) / element_bars(ref, "bf16")) < 1.0 / FLOOR_ALLOWANCE


def test_storage_floor_misses_the_bar_on_the_wide_gqa_shape():
    # 64 query heads over 4 KV heads, d = 4096: o_proj sums 8192 bf16-rounded
    # inputs, so rows with large attention outputs (the first tokens, where A is
    # one value row) carry an error above 2e-2 even at |Y| <= 4.
    ref, fl = floor_case(4, 260)
    err = np.abs(fl - ref)
    small = np.abs(ref) <= 4
    assert err[small].max() > 2e-2
    assert np.max(err / element_bars(ref, "bf16")) > 1.0
