// Host side of the C ABI declared in include/qwen3_attn.h: argument
// validation, workspace sizing, the handle's weight copy, and the launch
// sequence of each forward call on the caller's stream.
#include "qwen3_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <new>

#include "kernels.hpp"

struct qwen3_attn {
  qwen3_attn_desc desc;
  int device;
  void* mem;         // one device allocation holding everything below
  void* w_qkv;       // [(n_q + 2 n_kv) * 128, d]  (q rows, then k rows, then v rows)
  void* w_o;         // [d, n_q * 128]
  void* g_q;         // [128]
  void* g_k;         // [128]
  float* rope_rev;   // [128]: omega_i / (2 pi) as hi [0..63] + lo [64..127] floats,
                     // omega_i = theta^(-2i/128)
  float rope_rev_host[128];
  // Bound on |q~ . k~| (the attention scores in the log2 units of the exponent)
  // for keys this handle's QK-Norm produced: q_norm / k_norm leave every head
  // vector with norm <= sqrt(d_head) * max|gain| ("Qwen 3 From Scratch",
  // section "The idea": RMS-normalised q and k, which bounds the logits), RoPE
  // keeps the norm, and q~ carries log2(e) / sqrt(d_head).
  float score_bound;
  int in_norm;       // 1: forward = hidden + block(RMSNorm(hidden) * input gain)
  // measurement aid: events before each kernel and after the last
  int timing_cap;
  int timing_count;
  hipEvent_t* events;  // [timing_cap][4]
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int32_t dtype) { return dtype == QWEN3_ATTN_F32 ? 4 : 2; }

qwen3_attn_status check_desc(const qwen3_attn_desc* d) {
  if (!d) return QWEN3_ATTN_EINVAL;
  if (d->dtype != QWEN3_ATTN_F32 && d->dtype != QWEN3_ATTN_BF16) return QWEN3_ATTN_EINVAL;
  if (d->d_model <= 0 || d->n_q <= 0 || d->n_kv <= 0 || d->d_head <= 0) return QWEN3_ATTN_EINVAL;
  if (d->d_head % 2 != 0) return QWEN3_ATTN_EINVAL;
  if (d->n_q % d->n_kv != 0) return QWEN3_ATTN_EINVAL;
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return QWEN3_ATTN_EINVAL;
  if (!(d->rope_theta > 1.0) || !std::isfinite(d->rope_theta)) return QWEN3_ATTN_EINVAL;
  if (d->sliding_window < 0) return QWEN3_ATTN_EINVAL;
  if (d->d_head != 128) return QWEN3_ATTN_EUNSUPPORTED;
  if (d->d_model % 128 != 0) return QWEN3_ATTN_EUNSUPPORTED;
  if ((int64_t)(d->n_q + 2 * d->n_kv) * 128 > INT_MAX / 2) return QWEN3_ATTN_EUNSUPPORTED;
  return QWEN3_ATTN_OK;
}

struct WsLayout {
  size_t q_off, a_off, acc_off, ml_off, part_off, total;
  int nchunk;
  int chunk;  // decode: keys per chunk
  bool part;  // decode (<= 64 rows): the projections' fp32 products go through the part region
};

// Prefill of B sequences with n_tok token rows in all, at most max_T each.
bool ws_layout_prefill(const qwen3_attn_desc* d, int32_t B, int32_t n_tok, int32_t max_T,
                       WsLayout* L) {
  if (check_desc(d) != QWEN3_ATTN_OK) return false;
  if (B <= 0 || n_tok <= 0 || max_T <= 0 || max_T > n_tok) return false;
  if (n_tok > INT_MAX / 2 || (int64_t)B * max_T > INT_MAX / 2) return false;
  const size_t es = elem_size(d->dtype);
  const size_t hq = (size_t)d->n_q * 128;
  const size_t qb = align_up((size_t)n_tok * hq * es);
  L->q_off = 0;
  L->a_off = qb;
  L->acc_off = L->ml_off = 0;
  L->nchunk = 0;
  L->chunk = 0;
  L->part = false;
  L->part_off = 2 * qb;
  L->total = L->part_off +
             align_up(q3::flash_partial_floats(B, max_T, d->n_q, d->n_kv, n_tok) * sizeof(float));
  return true;
}

// Decode: `paged` picks the chunk length of a paged cache (cap = its
// max_blocks * block_size slots per sequence).
bool ws_layout(const qwen3_attn_desc* d, int is_decode, int32_t n, int32_t T, int64_t cap,
               WsLayout* L, bool paged = false) {
  if (check_desc(d) != QWEN3_ATTN_OK) return false;
  if (n <= 0 || T <= 0) return false;
  const size_t es = elem_size(d->dtype);
  const size_t hq = (size_t)d->n_q * 128;
  if (!is_decode) {
    if ((int64_t)n * T > INT_MAX / 2) return false;
    return ws_layout_prefill(d, n, n * T, T, L);
  }
  if (T != 1 || cap <= 0 || cap > INT_MAX) return false;
  // keys per chunk, from the most keys one (sequence, KV head) can see
  const int64_t span = d->sliding_window > 0 ? std::min<int64_t>(cap, d->sliding_window) : cap;
  const int chunk = q3::decode_chunk_keys(n, d->n_kv, span, paged);
  // partial slots per (sequence, KV head): every chunk of the cache, or with a
  // sliding window only the chunks one window can overlap
  int64_t nchunk = (cap + chunk - 1) / chunk;
  if (d->sliding_window > 0)
    nchunk = std::min<int64_t>(nchunk, ((int64_t)d->sliding_window + chunk - 1) / chunk + 1);
  const size_t n_rep = d->n_q / d->n_kv;
  const size_t slots = (size_t)n * d->n_kv * nchunk * n_rep;
  const size_t qb = align_up((size_t)n * hq * es);
  L->q_off = 0;
  L->a_off = qb;
  L->acc_off = 2 * qb;
  L->ml_off = L->acc_off + align_up(slots * 128 * sizeof(float));
  L->part_off = L->ml_off + align_up(slots * 2 * sizeof(float));
  L->part = n <= 64;
  size_t part_floats = 0;
  if (L->part) {
    const int es_i = static_cast<int>(es);
    const int nqkv = (d->n_q + 2 * d->n_kv) * 128;
    const size_t a = q3::small_m_partial_floats(n, nqkv, d->d_model, es_i);
    const size_t b = q3::small_m_partial_floats(n, d->d_model, d->n_q * 128, es_i);
    part_floats = a > b ? a : b;
  }
  L->total = L->part_off + align_up(part_floats * sizeof(float));
  L->nchunk = (int)nchunk;
  L->chunk = chunk;
  return true;
}

constexpr int kStages = 3;

void mark(qwen3_attn_t* h, hipStream_t s, int i) {
  if (h->timing_cap > 0 && h->timing_count < h->timing_cap)
    (void)hipEventRecord(h->events[h->timing_count * (kStages + 1) + i], s);
}
void mark_done(qwen3_attn_t* h, hipStream_t s) {
  if (h->timing_cap > 0 && h->timing_count < h->timing_cap) {
    mark(h, s, kStages);
    ++h->timing_count;
  }
}

void free_events(qwen3_attn_t* h) {
  if (h->events) {
    for (int i = 0; i < h->timing_cap * (kStages + 1); ++i) (void)hipEventDestroy(h->events[i]);
    delete[] h->events;
  }
  h->events = nullptr;
  h->timing_cap = 0;
  h->timing_count = 0;
}

qwen3_attn_status hip_status(hipError_t e) {
  return e == hipSuccess ? QWEN3_ATTN_OK : QWEN3_ATTN_EHIP;
}

template <typename T>
qwen3_attn_status run_prefill(qwen3_attn_t* h, const void* hidden, const int32_t* positions,
                              const int32_t* past, const int32_t* cu_seqlens, void* k_cache,
                              void* v_cache, const q3::KvAddr& kv, void* out, int B, int T_len,
                              int n_tok, char* ws, const WsLayout& L, hipStream_t s) {
  const qwen3_attn_desc& d = h->desc;
  const int M = n_tok;
  const int nqkv = (d.n_q + 2 * d.n_kv) * 128;
  const int hq = d.n_q * 128;
  T* qbuf = reinterpret_cast<T*>(ws + L.q_off);
  T* abuf = reinterpret_cast<T*>(ws + L.a_off);
  q3::QkvEpilogue e{qbuf, k_cache, v_cache, positions, h->g_q, h->g_k, h->rope_rev,
                    d.n_q, d.n_kv, kv, T_len, 0, d.eps, past,
                    h->in_norm ? hidden : nullptr, q3::kScoreScaleLog2, cu_seqlens, B};
  // Over empty caches every key of the call comes from this call's QK-Norm, so
  // the handle's score bound holds and the attention can use it as a fixed
  // softmax reference; keys already in a cache were written by someone else.
  const float fixed_ref =
      (past == nullptr && h->score_bound > 0.f && h->score_bound <= q3::kMaxFixedRef)
          ? h->score_bound
          : 0.f;
  mark(h, s, 0);
  hipError_t r = q3::launch_qkv_gemm<T>(reinterpret_cast<const T*>(hidden),
                                        reinterpret_cast<const T*>(h->w_qkv), M, nqkv, d.d_model,
                                        e, s, nullptr);
  if (r != hipSuccess) return QWEN3_ATTN_EHIP;
  mark(h, s, 1);
  r = q3::launch_flash_prefill<T>(qbuf, reinterpret_cast<const T*>(k_cache),
                                  reinterpret_cast<const T*>(v_cache), abuf, B, T_len, cu_seqlens,
                                  n_tok, d.n_q, d.n_kv, kv, past, d.sliding_window,
                                  reinterpret_cast<float*>(ws + L.part_off), fixed_ref, s);
  if (r != hipSuccess) return QWEN3_ATTN_EHIP;
  mark(h, s, 2);
  r = q3::launch_proj_gemm<T>(abuf, reinterpret_cast<const T*>(h->w_o), reinterpret_cast<T*>(out),
                              M, d.d_model, hq, s, nullptr,
                              h->in_norm ? reinterpret_cast<const T*>(hidden) : nullptr);
  mark_done(h, s);
  return hip_status(r);
}

template <typename T>
qwen3_attn_status run_decode(qwen3_attn_t* h, const void* hidden, const int32_t* positions,
                             void* k_cache, void* v_cache, const q3::KvAddr& kv, void* out, int N,
                             char* ws, const WsLayout& L, hipStream_t s) {
  const qwen3_attn_desc& d = h->desc;
  const int nqkv = (d.n_q + 2 * d.n_kv) * 128;
  const int hq = d.n_q * 128;
  T* qbuf = reinterpret_cast<T*>(ws + L.q_off);
  T* abuf = reinterpret_cast<T*>(ws + L.a_off);
  q3::QkvEpilogue e{qbuf, k_cache, v_cache, positions, h->g_q, h->g_k, h->rope_rev,
                    d.n_q, d.n_kv, kv, 1, 1, d.eps, nullptr,
                    h->in_norm ? hidden : nullptr, q3::kScoreScaleLog2};
  mark(h, s, 0);
  float* part = L.part ? reinterpret_cast<float*>(ws + L.part_off) : nullptr;
  hipError_t r = q3::launch_qkv_gemm<T>(reinterpret_cast<const T*>(hidden),
                                        reinterpret_cast<const T*>(h->w_qkv), N, nqkv, d.d_model,
                                        e, s, part);
  if (r != hipSuccess) return QWEN3_ATTN_EHIP;
  q3::DecodeScratch sc{reinterpret_cast<float*>(ws + L.acc_off),
                       reinterpret_cast<float*>(ws + L.ml_off), L.nchunk, L.chunk};
  mark(h, s, 1);
  r = q3::launch_decode_attn<T>(qbuf, reinterpret_cast<const T*>(k_cache),
                                reinterpret_cast<const T*>(v_cache), positions, abuf, N, d.n_q,
                                d.n_kv, kv, d.sliding_window, sc, s);
  if (r != hipSuccess) return QWEN3_ATTN_EHIP;
  mark(h, s, 2);
  r = q3::launch_proj_gemm<T>(abuf, reinterpret_cast<const T*>(h->w_o), reinterpret_cast<T*>(out),
                              N, d.d_model, hq, s, part,
                              h->in_norm ? reinterpret_cast<const T*>(hidden) : nullptr);
  mark_done(h, s);
  return hip_status(r);
}

qwen3_attn_status check_handle_device(const qwen3_attn_t* h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QWEN3_ATTN_EHIP;
  return dev == h->device ? QWEN3_ATTN_OK : QWEN3_ATTN_EINVAL;
}

qwen3_attn_status create_impl(const qwen3_attn_desc* desc, const qwen3_attn_weights* w,
                              const void* input_norm, void* stream, qwen3_attn_t** out) {
  if (!out) return QWEN3_ATTN_EINVAL;
  *out = nullptr;
  qwen3_attn_status st = check_desc(desc);
  if (st != QWEN3_ATTN_OK) return st;
  if (!w || !w->wq || !w->wk || !w->wv || !w->wo || !w->q_norm || !w->k_norm)
    return QWEN3_ATTN_EINVAL;

  qwen3_attn_t* h = new (std::nothrow) qwen3_attn_t();
  if (!h) return QWEN3_ATTN_ENOMEM;
  h->desc = *desc;
  const size_t es = elem_size(desc->dtype);
  const size_t d = desc->d_model, hq = (size_t)desc->n_q * 128, hkv = (size_t)desc->n_kv * 128;
  const size_t b_wqkv = align_up((hq + 2 * hkv) * d * es);
  const size_t b_wo = align_up(d * hq * es);
  const size_t b_g = align_up(128 * es);
  const size_t b_f = align_up(128 * sizeof(float));
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return QWEN3_ATTN_EHIP;
  }
  if (hipMalloc(&h->mem, b_wqkv + b_wo + 2 * b_g + b_f) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return QWEN3_ATTN_ENOMEM;
  }
  char* p = static_cast<char*>(h->mem);
  h->w_qkv = p;
  h->w_o = p + b_wqkv;
  h->g_q = p + b_wqkv + b_wo;
  h->g_k = p + b_wqkv + b_wo + b_g;
  h->rope_rev = reinterpret_cast<float*>(p + b_wqkv + b_wo + 2 * b_g);
  for (int i = 0; i < 64; ++i) {
    const double rev = std::pow(desc->rope_theta, -2.0 * i / 128.0) / (2.0 * M_PI);
    const float hi = static_cast<float>(rev);
    h->rope_rev_host[i] = hi;
    h->rope_rev_host[64 + i] = static_cast<float>(rev - static_cast<double>(hi));
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wqkv = static_cast<char*>(h->w_qkv);
  hipError_t r = hipMemcpyAsync(wqkv, w->wq, hq * d * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess)
    r = hipMemcpyAsync(wqkv + hq * d * es, w->wk, hkv * d * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess)
    r = hipMemcpyAsync(wqkv + (hq + hkv) * d * es, w->wv, hkv * d * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess) r = hipMemcpyAsync(h->w_o, w->wo, d * hq * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess) r = hipMemcpyAsync(h->g_q, w->q_norm, 128 * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess) r = hipMemcpyAsync(h->g_k, w->k_norm, 128 * es, hipMemcpyDeviceToDevice, s);
  if (r == hipSuccess)
    r = hipMemcpyAsync(h->rope_rev, h->rope_rev_host, 128 * sizeof(float), hipMemcpyHostToDevice, s);
  // Input RMSNorm: (x / rms(x) * g) W^T = (x W'^T) / rms(x) with W' = W * g by
  // columns, so the gain is folded into the q/k/v weights once here.
  h->in_norm = input_norm != nullptr;
  if (r == hipSuccess && input_norm) {
    const int rows = (desc->n_q + 2 * desc->n_kv) * 128, cols = desc->d_model;
    r = desc->dtype == QWEN3_ATTN_F32
            ? q3::launch_scale_columns<float>(static_cast<float*>(h->w_qkv), rows, cols,
                                              static_cast<const float*>(input_norm), s)
            : q3::launch_scale_columns<q3::bf16_t>(static_cast<q3::bf16_t*>(h->w_qkv), rows, cols,
                                                   static_cast<const q3::bf16_t*>(input_norm), s);
  }
  if (r == hipSuccess) r = hipStreamSynchronize(s);  // the host copy of rope_rev must complete
  // The gains' largest magnitudes give the score bound (see struct qwen3_attn):
  // |q~ . k~| <= scale * (sqrt(128) max|g_q|) * (sqrt(128) max|g_k|), times a
  // margin for the bf16 rounding of q~ and k~ (each norm grows by at most
  // 2^-9) and fp32 rounding in the norm, RoPE and the dot product.
  float gq_max = 0.f, gk_max = 0.f;
  if (r == hipSuccess) {
    unsigned char gbuf[2][128 * 4];
    r = hipMemcpy(gbuf[0], h->g_q, 128 * es, hipMemcpyDeviceToHost);
    if (r == hipSuccess) r = hipMemcpy(gbuf[1], h->g_k, 128 * es, hipMemcpyDeviceToHost);
    for (int w = 0; w < 2 && r == hipSuccess; ++w) {
      float mx = 0.f;
      for (int i = 0; i < 128; ++i) {
        float v;
        if (es == 4) {
          std::memcpy(&v, gbuf[w] + 4 * i, 4);
        } else {
          uint16_t b;
          std::memcpy(&b, gbuf[w] + 2 * i, 2);
          const uint32_t u = static_cast<uint32_t>(b) << 16;
          std::memcpy(&v, &u, 4);
        }
        mx = std::isfinite(v) ? std::fmax(mx, std::fabs(v)) : INFINITY;
      }
      (w == 0 ? gq_max : gk_max) = mx;
    }
  }
  h->score_bound = q3::kScoreScaleLog2 * 128.f * gq_max * gk_max * (1.f + 1.f / 64.f);
  if (r != hipSuccess) {
    (void)hipFree(h->mem);
    delete h;
    return QWEN3_ATTN_EHIP;
  }
  *out = h;
  return QWEN3_ATTN_OK;
}
}  // namespace

extern "C" {

qwen3_attn_status qwen3_attn_create(const qwen3_attn_desc* desc, const qwen3_attn_weights* w,
                                    void* stream, qwen3_attn_t** out) {
  return create_impl(desc, w, nullptr, stream, out);
}

qwen3_attn_status qwen3_attn_create_with_input_norm(const qwen3_attn_desc* desc,
                                                    const qwen3_attn_weights* w,
                                                    const void* input_norm, void* stream,
                                                    qwen3_attn_t** out) {
  if (!input_norm) {
    if (out) *out = nullptr;
    return QWEN3_ATTN_EINVAL;
  }
  return create_impl(desc, w, input_norm, stream, out);
}

size_t qwen3_attn_workspace_size(const qwen3_attn_desc* desc, int32_t is_decode, int32_t B_or_N,
                                 int32_t T, int64_t cache_cap) {
  WsLayout L;
  if (!ws_layout(desc, is_decode ? 1 : 0, B_or_N, T, cache_cap, &L)) return 0;
  if (!is_decode) return L.total;
  // one size for either kind of cache (a paged one may take shorter chunks)
  WsLayout P;
  if (!ws_layout(desc, 1, B_or_N, T, cache_cap, &P, true)) return 0;
  return L.total > P.total ? L.total : P.total;
}

size_t qwen3_attn_workspace_size_varlen(const qwen3_attn_desc* desc, int32_t B,
                                        int32_t total_tokens, int32_t max_seqlen) {
  WsLayout L;
  if ((int64_t)B * max_seqlen < total_tokens) return 0;
  if (!ws_layout_prefill(desc, B, total_tokens, max_seqlen, &L)) return 0;
  return L.total;
}

namespace {
// Paged cache addressing from the caller's block size (0 if unsupported).
bool paged_addr(const qwen3_attn_desc& d, const int32_t* table, int32_t max_blocks,
                int32_t block_size, q3::KvAddr* kv) {
  if (!table || max_blocks <= 0 || block_size < 64 || block_size > (1 << 20) ||
      (block_size & (block_size - 1)) != 0)
    return false;
  if ((int64_t)max_blocks * block_size > INT_MAX) return false;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  *kv = q3::KvAddr{table, block_size, max_blocks, lg, d.n_kv};
  return true;
}

// T is the chunk length of every sequence, or with cu_seqlens the longest
// one of a variable-length batch of n_tok rows in all (else n_tok = B * T).
qwen3_attn_status prefill_entry(qwen3_attn_t* h, const void* hidden, const int32_t* positions,
                                const int32_t* past, const int32_t* cu_seqlens, void* k_cache,
                                void* v_cache, const q3::KvAddr* paged, int64_t cache_cap,
                                void* out, int32_t B, int32_t T, int32_t n_tok, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!h || !hidden || !positions || !k_cache || !v_cache || !out) return QWEN3_ATTN_EINVAL;
  if (B <= 0 || T <= 0 || n_tok <= 0 || cache_cap <= 0 || T > cache_cap) return QWEN3_ATTN_EINVAL;
  if (cu_seqlens ? T > n_tok : (int64_t)B * T != n_tok) return QWEN3_ATTN_EINVAL;
  if (B > 65535 || cache_cap > INT_MAX) return QWEN3_ATTN_EUNSUPPORTED;
  const q3::KvAddr kv = paged ? *paged : q3::KvAddr{nullptr, cache_cap, 0, 0, h->desc.n_kv};
  WsLayout L;
  if (!ws_layout_prefill(&h->desc, B, n_tok, T, &L)) return QWEN3_ATTN_EUNSUPPORTED;
  if (!workspace || workspace_bytes < L.total) return QWEN3_ATTN_EWORKSPACE;
  qwen3_attn_status st = check_handle_device(h);
  if (st != QWEN3_ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (h->desc.dtype == QWEN3_ATTN_F32)
    return run_prefill<float>(h, hidden, positions, past, cu_seqlens, k_cache, v_cache, kv, out,
                              B, T, n_tok, ws, L, s);
  return run_prefill<q3::bf16_t>(h, hidden, positions, past, cu_seqlens, k_cache, v_cache, kv,
                                 out, B, T, n_tok, ws, L, s);
}

qwen3_attn_status decode_entry(qwen3_attn_t* h, const void* hidden, const int32_t* positions,
                               void* k_cache, void* v_cache, const q3::KvAddr* paged,
                               int64_t cache_cap, void* out, int32_t N, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!h || !hidden || !positions || !k_cache || !v_cache || !out) return QWEN3_ATTN_EINVAL;
  if (N <= 0 || cache_cap <= 0) return QWEN3_ATTN_EINVAL;
  if (N > 65535 || cache_cap > INT_MAX) return QWEN3_ATTN_EUNSUPPORTED;
  if (!q3::decode_nrep_supported(h->desc.n_q / h->desc.n_kv)) return QWEN3_ATTN_EUNSUPPORTED;
  WsLayout L;
  if (!ws_layout(&h->desc, 1, N, 1, cache_cap, &L, paged != nullptr))
    return QWEN3_ATTN_EUNSUPPORTED;
  if (!workspace || workspace_bytes < L.total) return QWEN3_ATTN_EWORKSPACE;
  qwen3_attn_status st = check_handle_device(h);
  if (st != QWEN3_ATTN_OK) return st;
  const q3::KvAddr kv = paged ? *paged : q3::KvAddr{nullptr, cache_cap, 0, 0, h->desc.n_kv};
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (h->desc.dtype == QWEN3_ATTN_F32)
    return run_decode<float>(h, hidden, positions, k_cache, v_cache, kv, out, N, ws, L, s);
  return run_decode<q3::bf16_t>(h, hidden, positions, k_cache, v_cache, kv, out, N, ws, L, s);
}
}  // namespace

qwen3_attn_status qwen3_attn_forward_prefill(qwen3_attn_t* h, const void* hidden,
                                             const int32_t* positions, void* k_cache,
                                             void* v_cache, int64_t cache_cap, void* out,
                                             int32_t B, int32_t T, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return prefill_entry(h, hidden, positions, nullptr, nullptr, k_cache, v_cache, nullptr,
                       cache_cap, out, B, T, B * T, workspace, workspace_bytes, stream);
}

qwen3_attn_status qwen3_attn_forward_prefill_chunk(qwen3_attn_t* h, const void* hidden,
                                                   const int32_t* positions,
                                                   const int32_t* past_len, void* k_cache,
                                                   void* v_cache, int64_t cache_cap, void* out,
                                                   int32_t B, int32_t T, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  if (!past_len) return QWEN3_ATTN_EINVAL;
  return prefill_entry(h, hidden, positions, past_len, nullptr, k_cache, v_cache, nullptr,
                       cache_cap, out, B, T, B * T, workspace, workspace_bytes, stream);
}

qwen3_attn_status qwen3_attn_forward_prefill_paged(qwen3_attn_t* h, const void* hidden,
                                                   const int32_t* positions,
                                                   const int32_t* past_len,
                                                   const int32_t* block_table,
                                                   int32_t max_blocks, void* k_pool, void* v_pool,
                                                   int32_t block_size, void* out, int32_t B,
                                                   int32_t T, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  if (!h) return QWEN3_ATTN_EINVAL;
  q3::KvAddr kv;
  if (!paged_addr(h->desc, block_table, max_blocks, block_size, &kv)) return QWEN3_ATTN_EINVAL;
  return prefill_entry(h, hidden, positions, past_len, nullptr, k_pool, v_pool, &kv,
                       (int64_t)max_blocks * block_size, out, B, T, B * T, workspace,
                       workspace_bytes, stream);
}

qwen3_attn_status qwen3_attn_forward_prefill_varlen(
    qwen3_attn_t* h, const void* hidden, const int32_t* positions, const int32_t* cu_seqlens,
    const int32_t* past_len, const int32_t* block_table, int32_t max_blocks, void* k_cache,
    void* v_cache, int64_t cache_cap, int32_t block_size, void* out, int32_t B,
    int32_t total_tokens, int32_t max_seqlen, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (!h || !cu_seqlens) return QWEN3_ATTN_EINVAL;
  if ((int64_t)B * max_seqlen < total_tokens) return QWEN3_ATTN_EINVAL;
  if (!block_table)
    return prefill_entry(h, hidden, positions, past_len, cu_seqlens, k_cache, v_cache, nullptr,
                         cache_cap, out, B, max_seqlen, total_tokens, workspace, workspace_bytes,
                         stream);
  q3::KvAddr kv;
  if (!paged_addr(h->desc, block_table, max_blocks, block_size, &kv)) return QWEN3_ATTN_EINVAL;
  return prefill_entry(h, hidden, positions, past_len, cu_seqlens, k_cache, v_cache, &kv,
                       (int64_t)max_blocks * block_size, out, B, max_seqlen, total_tokens,
                       workspace, workspace_bytes, stream);
}

qwen3_attn_status qwen3_attn_forward_decode_paged(qwen3_attn_t* h, const void* hidden,
                                                  const int32_t* positions,
                                                  const int32_t* block_table, int32_t max_blocks,
                                                  void* k_pool, void* v_pool, int32_t block_size,
                                                  void* out, int32_t N, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  if (!h) return QWEN3_ATTN_EINVAL;
  q3::KvAddr kv;
  if (!paged_addr(h->desc, block_table, max_blocks, block_size, &kv)) return QWEN3_ATTN_EINVAL;
  return decode_entry(h, hidden, positions, k_pool, v_pool, &kv, (int64_t)max_blocks * block_size,
                      out, N, workspace, workspace_bytes, stream);
}

qwen3_attn_status qwen3_attn_forward_decode(qwen3_attn_t* h, const void* hidden,
                                            const int32_t* positions, void* k_cache,
                                            void* v_cache, int64_t cache_cap, void* out,
                                            int32_t N, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  return decode_entry(h, hidden, positions, k_cache, v_cache, nullptr, cache_cap, out, N,
                      workspace, workspace_bytes, stream);
}

void qwen3_attn_destroy(qwen3_attn_t* h) {
  if (!h) return;
  int prev = -1;
  const bool switched = hipGetDevice(&prev) == hipSuccess && prev != h->device &&
                        hipSetDevice(h->device) == hipSuccess;
  (void)hipDeviceSynchronize();
  free_events(h);
  (void)hipFree(h->mem);
  if (switched) (void)hipSetDevice(prev);
  delete h;
}

qwen3_attn_status qwen3_attn_enable_stage_timing(qwen3_attn_t* h, int32_t capacity) {
  if (!h || capacity < 0) return QWEN3_ATTN_EINVAL;
  if (h->events) (void)hipDeviceSynchronize();
  free_events(h);
  if (capacity == 0) return QWEN3_ATTN_OK;
  h->events = new (std::nothrow) hipEvent_t[(size_t)capacity * (kStages + 1)];
  if (!h->events) return QWEN3_ATTN_ENOMEM;
  for (int i = 0; i < capacity * (kStages + 1); ++i) {
    if (hipEventCreate(&h->events[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(h->events[j]);
      delete[] h->events;
      h->events = nullptr;
      return QWEN3_ATTN_EHIP;
    }
  }
  h->timing_cap = capacity;
  h->timing_count = 0;
  return QWEN3_ATTN_OK;
}

qwen3_attn_status qwen3_attn_stage_times(qwen3_attn_t* h, float* ms, int32_t* n_calls) {
  if (!h || !ms || !n_calls) return QWEN3_ATTN_EINVAL;
  for (int j = 0; j < kStages; ++j) ms[j] = 0.f;
  *n_calls = h->timing_count;
  if (h->timing_count == 0) return QWEN3_ATTN_OK;
  if (hipEventSynchronize(h->events[h->timing_count * (kStages + 1) - 1]) != hipSuccess)
    return QWEN3_ATTN_EHIP;
  for (int c = 0; c < h->timing_count; ++c)
    for (int j = 0; j < kStages; ++j) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, h->events[c * (kStages + 1) + j],
                              h->events[c * (kStages + 1) + j + 1]) != hipSuccess)
        return QWEN3_ATTN_EHIP;
      ms[j] += t;
    }
  h->timing_count = 0;
  return QWEN3_ATTN_OK;
}

const char* qwen3_attn_status_string(qwen3_attn_status s) {
  switch (s) {
    case QWEN3_ATTN_OK: return "ok";
    case QWEN3_ATTN_EINVAL: return "invalid argument";
    case QWEN3_ATTN_EUNSUPPORTED: return "unsupported configuration";
    case QWEN3_ATTN_ENOMEM: return "device allocation failed";
    case QWEN3_ATTN_EWORKSPACE: return "workspace missing or too small";
    case QWEN3_ATTN_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
