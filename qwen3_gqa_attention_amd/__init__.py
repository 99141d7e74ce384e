"""Python binding of libqwen3attn.so, the gfx950 Qwen3 self-attention block.

Argument marshalling only: every step of the block runs in the HIP kernels
behind the C ABI (include/qwen3_attn.h).  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if the library is missing
(not built) or no GPU is present, calls raise.

Low-level functions carry the C names (``qwen3_attn_create`` ...).  The
``Qwen3Attention`` class wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqwen3attn.so")

QWEN3_ATTN_F32 = 0
QWEN3_ATTN_BF16 = 1
STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "ENOMEM", 4: "EWORKSPACE", 5: "EHIP"}
EXPORTED = ("qwen3_attn_create", "qwen3_attn_create_with_input_norm", "qwen3_attn_workspace_size",
            "qwen3_attn_forward_prefill",
            "qwen3_attn_forward_prefill_chunk", "qwen3_attn_forward_prefill_paged",
            "qwen3_attn_forward_prefill_varlen", "qwen3_attn_workspace_size_varlen",
            "qwen3_attn_forward_decode", "qwen3_attn_forward_decode_paged",
            "qwen3_attn_forward_decode_noalloc", "qwen3_attn_destroy", "qwen3_attn_enable_stage_timing",
            "qwen3_attn_stage_times", "qwen3_attn_status_string")
STAGES = ("qkv_norm_rope_gemm", "attention", "o_proj_gemm")


class Qwen3AttnDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_double), ("dtype", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32)]


class Qwen3AttnWeights(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p),
                ("wo", ctypes.c_void_p), ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p)]


class Qwen3AttnError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {STATUS.get(status, status)} "
                         f"({qwen3_attn_status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqwen3attn.so (built in-tree by qwen3_gqa_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m qwen3_gqa_attention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.qwen3_attn_create.argtypes = [ctypes.POINTER(Qwen3AttnDesc), ctypes.POINTER(Qwen3AttnWeights),
                                        vp, ctypes.POINTER(vp)]
        L.qwen3_attn_create.restype = ctypes.c_int
        L.qwen3_attn_create_with_input_norm.argtypes = [ctypes.POINTER(Qwen3AttnDesc),
                                                        ctypes.POINTER(Qwen3AttnWeights), vp, vp,
                                                        ctypes.POINTER(vp)]
        L.qwen3_attn_create_with_input_norm.restype = ctypes.c_int
        L.qwen3_attn_workspace_size.argtypes = [ctypes.POINTER(Qwen3AttnDesc), i32, i32, i32, i64]
        L.qwen3_attn_workspace_size.restype = sz
        L.qwen3_attn_forward_prefill.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, sz, vp]
        L.qwen3_attn_forward_prefill.restype = ctypes.c_int
        L.qwen3_attn_forward_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i32, i32,
                                                       vp, sz, vp]
        L.qwen3_attn_forward_prefill_chunk.restype = ctypes.c_int
        L.qwen3_attn_forward_prefill_paged.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, vp, i32,
                                                       i32, vp, sz, vp]
        L.qwen3_attn_forward_prefill_paged.restype = ctypes.c_int
        L.qwen3_attn_forward_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i64,
                                                        i32, vp, i32, i32, i32, vp, sz, vp]
        L.qwen3_attn_forward_prefill_varlen.restype = ctypes.c_int
        L.qwen3_attn_workspace_size_varlen.argtypes = [ctypes.POINTER(Qwen3AttnDesc), i32, i32, i32]
        L.qwen3_attn_workspace_size_varlen.restype = sz
        L.qwen3_attn_forward_decode_paged.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, vp, i32, vp,
                                                      sz, vp]
        L.qwen3_attn_forward_decode_paged.restype = ctypes.c_int
        L.qwen3_attn_forward_decode.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp, sz, vp]
        L.qwen3_attn_forward_decode.restype = ctypes.c_int
        L.qwen3_attn_forward_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp]
        L.qwen3_attn_forward_decode_noalloc.restype = ctypes.c_int
        L.qwen3_attn_destroy.argtypes = [vp]
        L.qwen3_attn_destroy.restype = None
        L.qwen3_attn_enable_stage_timing.argtypes = [vp, i32]
        L.qwen3_attn_enable_stage_timing.restype = ctypes.c_int
        L.qwen3_attn_stage_times.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.qwen3_attn_stage_times.restype = ctypes.c_int
        L.qwen3_attn_status_string.argtypes = [ctypes.c_int]
        L.qwen3_attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- C-named calls
def qwen3_attn_status_string(status: int) -> str:
    return lib().qwen3_attn_status_string(int(status)).decode()


def qwen3_attn_create(desc: Qwen3AttnDesc, weights: Qwen3AttnWeights, stream: int) -> tuple[int, int]:
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = lib().qwen3_attn_create(ctypes.byref(desc), ctypes.byref(weights), ctypes.c_void_p(stream),
                                 ctypes.byref(h))
    return st, (h.value or 0)


def qwen3_attn_create_with_input_norm(desc: Qwen3AttnDesc, weights: Qwen3AttnWeights, input_norm,
                                      stream: int) -> tuple[int, int]:
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = lib().qwen3_attn_create_with_input_norm(ctypes.byref(desc), ctypes.byref(weights), input_norm,
                                                 ctypes.c_void_p(stream), ctypes.byref(h))
    return st, (h.value or 0)


def qwen3_attn_workspace_size(desc: Qwen3AttnDesc, is_decode: int, B_or_N: int, T: int,
                              cache_cap: int) -> int:
    return lib().qwen3_attn_workspace_size(ctypes.byref(desc), is_decode, B_or_N, T, cache_cap)


def qwen3_attn_forward_prefill(handle, hidden, positions, k_cache, v_cache, cache_cap, out, B, T,
                               workspace, workspace_bytes, stream) -> int:
    return lib().qwen3_attn_forward_prefill(handle, hidden, positions, k_cache, v_cache, cache_cap,
                                            out, B, T, workspace, workspace_bytes, stream)


def qwen3_attn_forward_prefill_chunk(handle, hidden, positions, past_len, k_cache, v_cache,
                                     cache_cap, out, B, T, workspace, workspace_bytes,
                                     stream) -> int:
    return lib().qwen3_attn_forward_prefill_chunk(handle, hidden, positions, past_len, k_cache,
                                                  v_cache, cache_cap, out, B, T, workspace,
                                                  workspace_bytes, stream)


def qwen3_attn_forward_prefill_paged(handle, hidden, positions, past_len, block_table, max_blocks,
                                     k_pool, v_pool, block_size, out, B, T, workspace,
                                     workspace_bytes, stream) -> int:
    return lib().qwen3_attn_forward_prefill_paged(handle, hidden, positions, past_len, block_table,
                                                  max_blocks, k_pool, v_pool, block_size, out, B, T,
                                                  workspace, workspace_bytes, stream)


def qwen3_attn_forward_prefill_varlen(handle, hidden, positions, cu_seqlens, past_len, block_table,
                                      max_blocks, k_cache, v_cache, cache_cap, block_size, out, B,
                                      total_tokens, max_seqlen, workspace, workspace_bytes,
                                      stream) -> int:
    return lib().qwen3_attn_forward_prefill_varlen(handle, hidden, positions, cu_seqlens, past_len,
                                                   block_table, max_blocks, k_cache, v_cache,
                                                   cache_cap, block_size, out, B, total_tokens,
                                                   max_seqlen, workspace, workspace_bytes, stream)


def qwen3_attn_workspace_size_varlen(desc: Qwen3AttnDesc, B: int, total_tokens: int,
                                     max_seqlen: int) -> int:
    return lib().qwen3_attn_workspace_size_varlen(ctypes.byref(desc), B, total_tokens, max_seqlen)


def qwen3_attn_forward_decode_paged(handle, hidden, positions, block_table, max_blocks, k_pool,
                                    v_pool, block_size, out, N, workspace, workspace_bytes,
                                    stream) -> int:
    return lib().qwen3_attn_forward_decode_paged(handle, hidden, positions, block_table, max_blocks,
                                                 k_pool, v_pool, block_size, out, N, workspace,
                                                 workspace_bytes, stream)


def qwen3_attn_forward_decode(handle, hidden, positions, k_cache, v_cache, cache_cap, out, N,
                              workspace, workspace_bytes, stream) -> int:
    return lib().qwen3_attn_forward_decode(handle, hidden, positions, k_cache, v_cache, cache_cap,
                                           out, N, workspace, workspace_bytes, stream)


def qwen3_attn_forward_decode_noalloc(handle, hidden, positions, k_cache, v_cache, cache_cap, out,
                                      N, stream) -> int:
    return lib().qwen3_attn_forward_decode_noalloc(handle, hidden, positions, k_cache, v_cache,
                                                   cache_cap, out, N, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20   # QWEN3_ATTN_NOALLOC_SCRATCH_BYTES


def qwen3_attn_destroy(handle) -> None:
    lib().qwen3_attn_destroy(handle)


def qwen3_attn_enable_stage_timing(handle, capacity: int) -> int:
    return lib().qwen3_attn_enable_stage_timing(handle, capacity)


def qwen3_attn_stage_times(handle) -> tuple[int, list[float], int]:
    """Returns (status, summed ms per kernel [3], number of calls)."""
    ms = (ctypes.c_float * 3)()
    n = ctypes.c_int32()
    st = lib().qwen3_attn_stage_times(handle, ms, ctypes.byref(n))
    return st, list(ms), n.value


# ---------------------------------------------------------------- torch wrapper
def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return QWEN3_ATTN_F32
    if dtype == torch.bfloat16:
        return QWEN3_ATTN_BF16
    raise TypeError(f"unsupported dtype {dtype} (float32 or bfloat16)")


def _ptr(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


class Qwen3Attention:
    """One Qwen3 attention block on the current HIP device.

    Weights are torch tensors stored [out, in]; the handle copies them.
    """

    def __init__(self, wq, wk, wv, wo, q_norm, k_norm, *, n_q: int, n_kv: int, d_head: int = 128,
                 eps: float = 1e-6, rope_theta: float = 1e6, input_norm=None,
                 sliding_window: int = 0):
        """input_norm [d] (optional): the handle then computes
        hidden + block(RMSNorm(hidden) * input_norm) (pre-norm and residual fused).
        sliding_window W > 0: each token sees only its W most recent keys."""
        torch = _torch()
        self.dtype = wq.dtype
        self.d_model = wq.shape[1]
        self.n_q, self.n_kv, self.d_head = n_q, n_kv, d_head
        self.desc = Qwen3AttnDesc(self.d_model, n_q, n_kv, d_head, eps, rope_theta,
                                  _dtype_code(self.dtype), sliding_window)
        d, hq, hkv = self.d_model, n_q * d_head, n_kv * d_head
        self.weights = Qwen3AttnWeights(
            _ptr(wq, "wq", self.dtype, (hq, d)), _ptr(wk, "wk", self.dtype, (hkv, d)),
            _ptr(wv, "wv", self.dtype, (hkv, d)), _ptr(wo, "wo", self.dtype, (d, hq)),
            _ptr(q_norm, "q_norm", self.dtype, (d_head,)), _ptr(k_norm, "k_norm", self.dtype, (d_head,)))
        stream = torch.cuda.current_stream().cuda_stream
        if input_norm is None:
            st, self.handle = qwen3_attn_create(self.desc, self.weights, stream)
            name = "qwen3_attn_create"
        else:
            st, self.handle = qwen3_attn_create_with_input_norm(
                self.desc, self.weights, _ptr(input_norm, "input_norm", self.dtype, (d,)), stream)
            name = "qwen3_attn_create_with_input_norm"
        if st != 0:
            raise Qwen3AttnError(name, st)
        # Workspaces the calls allocate when the caller passes none, one per
        # stream (two calls in flight on different streams need two).
        self._ws = {}

    def close(self):
        if getattr(self, "handle", 0):
            qwen3_attn_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def enable_stage_timing(self, capacity: int):
        st = qwen3_attn_enable_stage_timing(self.handle, capacity)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_enable_stage_timing", st)

    def stage_times(self) -> tuple[list[float], int]:
        """Summed kernel milliseconds [qkv gemm, attention, o_proj] and the call count."""
        st, ms, n = qwen3_attn_stage_times(self.handle)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_stage_times", st)
        return ms, n

    def workspace_size(self, is_decode: bool, B_or_N: int, T: int = 1, cache_cap: int = 0) -> int:
        return qwen3_attn_workspace_size(self.desc, int(is_decode), B_or_N, T, cache_cap)

    def _workspace(self, nbytes: int, workspace):
        """The caller's workspace, or this object's own one for the current
        stream.  Each stream gets its own buffer, allocated while that stream
        is current, so torch's allocator orders its reuse after the stream's
        earlier calls; growing it on the same stream is therefore safe too."""
        torch = _torch()
        if workspace is not None:
            return workspace
        key = torch.cuda.current_stream().cuda_stream
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
            self._ws[key] = ws
        return ws

    def prefill(self, hidden, positions, k_cache, v_cache, out=None, workspace=None):
        """hidden [B,T,d]; positions [B,T] int32; caches [B,n_kv,cap,128] (written)."""
        torch = _torch()
        B, T, d = hidden.shape
        cap = k_cache.shape[2]
        if out is None:
            out = torch.empty_like(hidden)
        nbytes = self.workspace_size(False, B, T)
        ws = self._workspace(nbytes, workspace)
        st = qwen3_attn_forward_prefill(
            self.handle, _ptr(hidden, "hidden", self.dtype, (B, T, self.d_model)), _ptr(positions, "positions", torch.int32, (B, T)),
            _ptr(k_cache, "k_cache", self.dtype, (B, self.n_kv, cap, self.d_head)),
            _ptr(v_cache, "v_cache", self.dtype, (B, self.n_kv, cap, self.d_head)), cap,
            _ptr(out, "out", self.dtype, (B, T, d)), B, T, _ptr(ws, "workspace"), ws.numel() * ws.element_size(),
            torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_prefill", st)
        return out

    def prefill_chunk(self, hidden, positions, past_len, k_cache, v_cache, out=None,
                      workspace=None):
        """hidden [B,T,d]; positions [B,T] int32; past_len [B] int32 (device) = tokens
        already cached per sequence; caches [B,n_kv,cap,128] (slots past..past+T-1 written)."""
        torch = _torch()
        B, T, d = hidden.shape
        cap = k_cache.shape[2]
        if out is None:
            out = torch.empty_like(hidden)
        nbytes = self.workspace_size(False, B, T)
        ws = self._workspace(nbytes, workspace)
        st = qwen3_attn_forward_prefill_chunk(
            self.handle, _ptr(hidden, "hidden", self.dtype, (B, T, self.d_model)), _ptr(positions, "positions", torch.int32, (B, T)),
            _ptr(past_len, "past_len", torch.int32, (B,)),
            _ptr(k_cache, "k_cache", self.dtype, (B, self.n_kv, cap, self.d_head)),
            _ptr(v_cache, "v_cache", self.dtype, (B, self.n_kv, cap, self.d_head)), cap,
            _ptr(out, "out", self.dtype, (B, T, d)), B, T, _ptr(ws, "workspace"), ws.numel() * ws.element_size(),
            torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_prefill_chunk", st)
        return out

    def prefill_paged(self, hidden, positions, past_len, block_table, k_pool, v_pool, out=None,
                      workspace=None):
        """Chunked prefill over a paged cache: pools [num_blocks, n_kv, block_size, 128];
        block_table [B, max_blocks] int32 (device); past_len [B] int32 (device) or None."""
        torch = _torch()
        B, T, d = hidden.shape
        nb, _, bs, _ = k_pool.shape
        mb = block_table.shape[1]
        if out is None:
            out = torch.empty_like(hidden)
        ws = self._workspace(self.workspace_size(False, B, T), workspace)
        st = qwen3_attn_forward_prefill_paged(
            self.handle, _ptr(hidden, "hidden", self.dtype, (B, T, self.d_model)), _ptr(positions, "positions", torch.int32, (B, T)),
            None if past_len is None else _ptr(past_len, "past_len", torch.int32, (B,)),
            _ptr(block_table, "block_table", torch.int32, (B, mb)), mb,
            _ptr(k_pool, "k_pool", self.dtype, (nb, self.n_kv, bs, self.d_head)),
            _ptr(v_pool, "v_pool", self.dtype, (nb, self.n_kv, bs, self.d_head)), bs,
            _ptr(out, "out", self.dtype, (B, T, d)), B, T, _ptr(ws, "workspace"),
            ws.numel() * ws.element_size(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_prefill_paged", st)
        return out

    def prefill_varlen(self, hidden, positions, cu_seqlens, k_cache, v_cache, *, max_seqlen,
                       past_len=None, block_table=None, out=None, workspace=None):
        """A variable-length batch: hidden [total, d] holds the requests one after
        another, cu_seqlens [B+1] int32 (device) their row offsets.  block_table
        None: caches [B, n_kv, cap, 128]; else pools [num_blocks, n_kv, block_size,
        128] with block_table [B, max_blocks]."""
        torch = _torch()
        total, d = hidden.shape
        B = cu_seqlens.shape[0] - 1
        if out is None:
            out = torch.empty_like(hidden)
        ws = self._workspace(qwen3_attn_workspace_size_varlen(self.desc, B, total, max_seqlen),
                             workspace)
        n0, _, s2, _ = k_cache.shape
        kshape = (n0, self.n_kv, s2, self.d_head)
        mb = 0 if block_table is None else block_table.shape[1]
        st = qwen3_attn_forward_prefill_varlen(
            self.handle, _ptr(hidden, "hidden", self.dtype, (total, self.d_model)),
            _ptr(positions, "positions", torch.int32, (total,)),
            _ptr(cu_seqlens, "cu_seqlens", torch.int32, (B + 1,)),
            None if past_len is None else _ptr(past_len, "past_len", torch.int32, (B,)),
            None if block_table is None else _ptr(block_table, "block_table", torch.int32, (B, mb)),
            mb, _ptr(k_cache, "k_cache", self.dtype, kshape),
            _ptr(v_cache, "v_cache", self.dtype, kshape),
            s2 if block_table is None else 0, 0 if block_table is None else s2,
            _ptr(out, "out", self.dtype, (total, d)), B, total, max_seqlen, _ptr(ws, "workspace"),
            ws.numel() * ws.element_size(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_prefill_varlen", st)
        return out

    def decode_paged(self, hidden, positions, block_table, k_pool, v_pool, out=None,
                     workspace=None):
        """Decode over a paged cache; positions [N] int32 = cached lengths."""
        torch = _torch()
        N, d = hidden.shape
        nb, _, bs, _ = k_pool.shape
        mb = block_table.shape[1]
        if out is None:
            out = torch.empty_like(hidden)
        ws = self._workspace(self.workspace_size(True, N, 1, mb * bs), workspace)
        st = qwen3_attn_forward_decode_paged(
            self.handle, _ptr(hidden, "hidden", self.dtype, (N, self.d_model)), _ptr(positions, "positions", torch.int32, (N,)),
            _ptr(block_table, "block_table", torch.int32, (N, mb)), mb,
            _ptr(k_pool, "k_pool", self.dtype, (nb, self.n_kv, bs, self.d_head)),
            _ptr(v_pool, "v_pool", self.dtype, (nb, self.n_kv, bs, self.d_head)), bs,
            _ptr(out, "out", self.dtype, (N, d)), N, _ptr(ws, "workspace"),
            ws.numel() * ws.element_size(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_decode_paged", st)
        return out

    def decode(self, hidden, positions, k_cache, v_cache, out=None, workspace=None):
        """hidden [N,d]; positions [N] int32 = cached lengths; caches [N,n_kv,cap,128]."""
        torch = _torch()
        N, d = hidden.shape
        cap = k_cache.shape[2]
        if out is None:
            out = torch.empty_like(hidden)
        nbytes = self.workspace_size(True, N, 1, cap)
        ws = self._workspace(nbytes, workspace)
        st = qwen3_attn_forward_decode(
            self.handle, _ptr(hidden, "hidden", self.dtype, (N, self.d_model)), _ptr(positions, "positions", torch.int32, (N,)),
            _ptr(k_cache, "k_cache", self.dtype, (N, self.n_kv, cap, self.d_head)),
            _ptr(v_cache, "v_cache", self.dtype, (N, self.n_kv, cap, self.d_head)), cap,
            _ptr(out, "out", self.dtype, (N, d)), N, _ptr(ws, "workspace"), ws.numel() * ws.element_size(),
            torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise Qwen3AttnError("qwen3_attn_forward_decode", st)
        return out
