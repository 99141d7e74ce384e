"""C-ABI checks that need no GPU: exported symbols, host-side validation,
workspace sizing and status strings.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import qwen3_gqa_attention_amd as q3

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qwen3_attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwen3_attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert header_functions() == sorted(q3.EXPORTED)


def test_library_exports_every_declared_symbol(built_lib):
    lib = ctypes.CDLL(built_lib)
    for name in header_functions():
        assert hasattr(lib, name), name


def desc(**kw):
    base = dict(d_model=1024, n_q=16, n_kv=8, d_head=128, eps=1e-6, rope_theta=1e6, dtype=q3.QWEN3_ATTN_BF16)
    base.update(kw)
    return q3.Qwen3AttnDesc(**base)


WEIGHTS = q3.Qwen3AttnWeights(*([0x1000] * 6))   # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(n_q=12, n_kv=8), 1),          # n_q % n_kv != 0
    (dict(n_q=0), 1),
    (dict(n_kv=-1), 1),
    (dict(d_model=0), 1),
    (dict(d_head=127), 1),              # odd head dim
    (dict(d_head=64), 2),               # valid but not implemented
    (dict(d_model=1000), 2),            # d_model % 128 != 0
    (dict(dtype=7), 1),
    (dict(eps=-1.0), 1),
    (dict(eps=float("nan")), 1),
    (dict(rope_theta=0.5), 1),
    (dict(rope_theta=float("inf")), 1),
    (dict(sliding_window=-1), 1),
])
def test_create_rejects_bad_descriptors_before_any_hip_call(built_lib, kw, status):
    st, h = q3.qwen3_attn_create(desc(**kw), WEIGHTS, 0)
    assert st == status and h == 0


def test_create_with_input_norm_rejects_null_gain(built_lib):
    h = ctypes.c_void_p(1)
    st = q3.lib().qwen3_attn_create_with_input_norm(ctypes.byref(desc()),
                                                    ctypes.byref(q3.Qwen3AttnWeights(*([0x1000] * 6))),
                                                    None, None, ctypes.byref(h))
    assert st == 1 and not h.value


def test_create_rejects_null_weights(built_lib):
    for i in range(6):
        ptrs = [0x1000] * 6
        ptrs[i] = 0
        st, h = q3.qwen3_attn_create(desc(), q3.Qwen3AttnWeights(*ptrs), 0)
        assert st == 1 and h == 0
    lib = q3.lib()
    assert lib.qwen3_attn_create(ctypes.byref(desc()), None, None, None) == 1


def align(x):
    return (x + 255) // 256 * 256


def test_workspace_size_prefill_and_decode(built_lib):
    d = desc()
    # prefill: rotated q and merged attention output (512 query tiles: no key split)
    assert q3.qwen3_attn_workspace_size(d, 0, 2, 2048, 0) == 2 * align(2 * 2048 * 2048 * 2)
    d32 = desc(dtype=q3.QWEN3_ATTN_F32)
    # B=1, T=128: 16 query-tile workgroups (< 256), so each key range is split
    # 8 ways and the fp32 partials (O, then m and l) are reserved as well
    part = 8 * 128 * 16 * (128 + 2) * 4
    assert (q3.qwen3_attn_workspace_size(d32, 0, 1, 128, 0)
            == 2 * align(128 * 2048 * 4) + align(part))
    # decode: q and merged output, then per-chunk partials.  The size covers a
    # contiguous cache (64 sequences x 8 KV heads over 32832 slots: 2048-key
    # chunks) and a paged one of as many slots (512-key chunks), so the paged
    # one's 65 chunks per sequence and head are reserved
    cap, N = 32832, 64
    nchunk = -(-cap // 512)
    slots = N * 8 * nchunk * 2
    # bf16 64-row projections: the unsplit fp32 q/k/v product (64 x 4096) that
    # the finishing kernel normalises (o_proj needs none)
    part = 64 * 4096 * 4
    want = 2 * align(N * 2048 * 2) + align(slots * 128 * 4) + align(slots * 2 * 4) + align(part)
    assert q3.qwen3_attn_workspace_size(d, 1, N, 1, cap) == want
    # fp32: split-K partials (the fewest K slices giving at least 64
    # workgroups of 128 columns): q/k/v 2 slices x 64 x 4096, o_proj 8 x 64 x
    # 1024; the larger is reserved
    d32 = desc(dtype=q3.QWEN3_ATTN_F32)
    part = max(2 * 64 * 4096, 8 * 64 * 1024) * 4
    want = 2 * align(N * 2048 * 4) + align(slots * 128 * 4) + align(slots * 2 * 4) + align(part)
    assert q3.qwen3_attn_workspace_size(d32, 1, N, 1, cap) == want
    # a sliding window of W keys: partial slots for the ceil(W / chunk) + 1
    # chunks it can overlap; a 4096-key window takes 2048-key chunks over a
    # contiguous cache (64 x 8 x 2 = 1024 workgroups: 3 slots), 512-key ones
    # over a paged one (9 slots: reserved)
    dw = desc(sliding_window=4096)
    slots_w = N * 8 * 9 * 2
    want = (2 * align(N * 2048 * 2) + align(slots_w * 128 * 4) + align(slots_w * 2 * 4)
            + align(64 * 4096 * 4))
    assert q3.qwen3_attn_workspace_size(dw, 1, N, 1, cap) == want


@pytest.mark.parametrize("args", [(0, 0, 128, 0), (0, 2, 0, 0), (1, 4, 2, 100), (1, 4, 1, 0),
                                  (1, 0, 1, 100)])
def test_workspace_size_zero_for_invalid(built_lib, args):
    assert q3.qwen3_attn_workspace_size(desc(), *args) == 0
    assert q3.qwen3_attn_workspace_size(desc(n_q=12), 0, 1, 8, 0) == 0
    assert q3.qwen3_attn_workspace_size(desc(sliding_window=-4), 0, 1, 8, 0) == 0


def test_varlen_workspace_size(built_lib):
    d = desc()
    # equal lengths: the fixed-length prefill's workspace
    for B, T in ((2, 2048), (1, 128), (3, 77)):
        assert (q3.qwen3_attn_workspace_size_varlen(d, B, B * T, T)
                == q3.qwen3_attn_workspace_size(d, 0, B, T, 0) > 0)
    # ragged: rows sized by the total, key splits by B and the longest request
    assert q3.qwen3_attn_workspace_size_varlen(d, 4, 1000, 700) > 0
    for args in ((0, 10, 5), (2, 0, 1), (2, 10, 0), (2, 10, 11), (2, 10, 4)):
        assert q3.qwen3_attn_workspace_size_varlen(d, *args) == 0, args


def test_sliding_window_workspace(built_lib):
    # prefill: unchanged by the window
    for args in ((0, 2, 2048, 0), (0, 1, 128, 0)):
        assert (q3.qwen3_attn_workspace_size(desc(sliding_window=4096), *args)
                == q3.qwen3_attn_workspace_size(desc(), *args) > 0)
    # decode: partial slots for the ceil(W / chunk) + 1 chunks a window can overlap,
    # never more than the whole cache needs
    full = q3.qwen3_attn_workspace_size(desc(), 1, 64, 1, 32832)
    win = q3.qwen3_attn_workspace_size(desc(sliding_window=4096), 1, 64, 1, 32832)
    assert 0 < win < full
    for W in (1, 512, 513, 32832, 100000):
        assert 0 < q3.qwen3_attn_workspace_size(desc(sliding_window=W), 1, 64, 1, 32832) <= full
    assert (q3.qwen3_attn_workspace_size(desc(sliding_window=100000), 1, 64, 1, 32832) == full)


def test_varlen_rejects_missing_offsets_and_inconsistent_sizes(built_lib):
    # cu_seqlens NULL, then B * max_seqlen < total: EINVAL before the handle is used
    assert q3.qwen3_attn_forward_prefill_varlen(1, 1, 1, None, None, None, 0, 1, 1, 64, 0, 1, 2,
                                                10, 5, 1, 1 << 20, None) == 1
    assert q3.qwen3_attn_forward_prefill_varlen(1, 1, 1, 1, None, None, 0, 1, 1, 64, 0, 1, 2,
                                                10, 4, 1, 1 << 20, None) == 1
    assert q3.qwen3_attn_forward_prefill_varlen(None, 1, 1, 1, None, None, 0, 1, 1, 64, 0, 1, 2,
                                                10, 5, 1, 1 << 20, None) == 1


def test_forward_with_null_handle_is_einval(built_lib):
    assert q3.qwen3_attn_forward_prefill(None, 1, 1, 1, 1, 16, 1, 1, 8, 1, 1 << 20, None) == 1
    # chunked prefill: a missing past_len array is rejected before the handle is used
    assert q3.qwen3_attn_forward_prefill_chunk(1, 1, 1, None, 1, 1, 16, 1, 1, 8, 1, 1 << 20,
                                               None) == 1
    assert q3.qwen3_attn_forward_prefill_chunk(None, 1, 1, 1, 1, 1, 16, 1, 1, 8, 1, 1 << 20,
                                               None) == 1
    assert q3.qwen3_attn_forward_prefill_paged(None, 1, 1, None, 1, 4, 1, 1, 64, 1, 1, 8, 1,
                                               1 << 20, None) == 1
    assert q3.qwen3_attn_forward_decode_paged(None, 1, 1, 1, 4, 1, 1, 64, 1, 1, 1, 1 << 20,
                                              None) == 1
    assert q3.qwen3_attn_forward_decode(None, 1, 1, 1, 1, 16, 1, 1, 1, 1 << 20, None) == 1
    q3.qwen3_attn_destroy(None)   # NULL is a no-op


def test_status_strings(built_lib):
    for code in range(6):
        assert q3.qwen3_attn_status_string(code)
    assert q3.qwen3_attn_status_string(99) == "unknown status"


def test_binding_keeps_one_workspace_per_stream(monkeypatch):
    # The wrapper's own workspace (used when the caller passes none) is cached
    # per stream: two streams never share scratch memory, a stream reuses its
    # buffer while it is large enough, and a caller's workspace is passed
    # through untouched.  A stand-in for torch supplies the current stream.
    import types

    import torch

    current = {"stream": 11}
    fake = types.SimpleNamespace(
        uint8=torch.uint8,
        cuda=types.SimpleNamespace(current_stream=lambda: types.SimpleNamespace(
            cuda_stream=current["stream"])),
        empty=lambda n, dtype=None, device=None: torch.empty(n, dtype=dtype))
    monkeypatch.setattr(q3, "_torch", lambda: fake)
    obj = q3.Qwen3Attention.__new__(q3.Qwen3Attention)
    obj.handle = 0
    obj._ws = {}
    a = obj._workspace(100, None)
    assert obj._workspace(80, None) is a           # same stream, fits: reused
    current["stream"] = 22
    b = obj._workspace(100, None)
    assert b is not a and b.data_ptr() != a.data_ptr()   # another stream: its own buffer
    current["stream"] = 11
    assert obj._workspace(100, None) is a
    c = obj._workspace(400, None)                  # grows on its own stream only
    assert c is not a and c.numel() >= 400 and obj._workspace(10, None) is c
    current["stream"] = 22
    assert obj._workspace(10, None) is b
    mine = torch.empty(5, dtype=torch.uint8)
    assert obj._workspace(10 ** 6, mine) is mine   # the caller's workspace is used as given
