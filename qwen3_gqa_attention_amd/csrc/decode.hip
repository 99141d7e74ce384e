// Decode attention: one new query token per sequence over its KV cache.
//
// What it computes ("Assembling a large model from scratch", section "The
// complete code": with a cache of L tokens the new token sits at position L
// and sees keys 0..L; query head h reads KV head h / n_rep) -- split over key
// chunks and merged with log-sum-exp weights, which reaches the same softmax
// up to rounding order.
//
// The step is bound by HBM: every cached key/value row is read once, and the
// n_rep query heads of a KV head share that read.  Grid = (key chunk, KV head,
// sequence); chunks past a sequence's length exit at once.  Inside a
// workgroup each wave streams a contiguous quarter of the chunk; within a
// wave four 16-lane groups take interleaved keys and each lane owns 8 of the
// 128 dims, so every key row is two coalesced 256-byte reads (K and V, bf16).
// Scores are a dot product over the lane's 8 dims reduced across the 16
// lanes; softmax statistics and the weighted V sum stay in fp32 registers.
// The four groups, then the four waves, are merged in registers / LDS and one
// partial (max, sum, weighted values) per chunk is written.  A second kernel
// merges the chunks of each (sequence, query head).
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace q3 {

constexpr int kDecodeUnroll = 4;  // keys per 16-lane group per iteration

// Keys per workgroup for a contiguous cache: the largest of 2048, 1024, 512
// that still launches at least 1024 workgroups (4 per CU) for `span` keys
// per (sequence, KV head).
// Longer chunks mean fewer workgroup start-ups and fewer partials to merge;
// too few workgroups leave the last round's CUs with little in flight.
// Measured on the 64-sequence decode step (1024..32768 keys): full caches
// 0.760 / 0.752 / 0.736 ms at 512 / 1024 / 2048 keys (4096: 0.738); a
// 4096-key window, with the launch's residency capped at 2 workgroups per
// CU (below), 0.193 / 0.186 / 0.182 ms (4096: 0.209).
int decode_chunk_keys(int N, int n_kv, int64_t span, bool paged) {
  // A paged cache (64-key blocks scattered over the pool, one scalar
  // block-table lookup every 16 keys) measured best at 512 keys on the same
  // step: 0.773 against 0.841 / 0.862 ms at 1024 / 2048.
  if (paged) return 512;
  int c = 2048;
  while (c > 512 && (int64_t)N * n_kv * ((span + c - 1) / c) < 1024) c >>= 1;
  return c;
}

// Streaming 16-byte load: the cache is read once per step, so it is fetched
// with the non-temporal hint and does not displace reused lines in L2 / MALL
// (on MI355X this sustains about 7.0 TB/s against 6.2 TB/s for plain loads
// in a pure-read stream).
__device__ __forceinline__ u32x4_v ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
}

template <typename T> struct RowSlice;  // 8 elements of a row
template <> struct RowSlice<bf16_t> {
  u32x4_v v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = ld16(p); }
  __device__ __forceinline__ void load_stream(const bf16_t* p) { v = ld16_stream(p); }
  __device__ __forceinline__ void zero() { v = u32x4_v{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float at(int e) const {
    const uint32_t w = v[e >> 1];
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
  }
};
template <> struct RowSlice<float> {
  u32x4_v v0, v1;
  __device__ __forceinline__ void load(const float* p) { v0 = ld16(p); v1 = ld16(p + 4); }
  __device__ __forceinline__ void load_stream(const float* p) {
    v0 = ld16_stream(p);
    v1 = ld16_stream(p + 4);
  }
  __device__ __forceinline__ void zero() { v0 = v1 = u32x4_v{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float at(int e) const {
    return __uint_as_float(e < 4 ? v0[e] : v1[e - 4]);
  }
};

template <typename T, int NREP>
__global__ __launch_bounds__(256) void decode_attn_kernel(const T* __restrict__ Q,
                                                          const T* __restrict__ Kc,
                                                          const T* __restrict__ Vc,
                                                          const int32_t* __restrict__ positions,
                                                          float* __restrict__ part_acc,
                                                          float* __restrict__ part_ml, int n_q,
                                                          int n_kv, KvAddr kv, int nchunk,
                                                          int chunk, int window) {
  const int g = blockIdx.y, s = blockIdx.z;
  const int nkeys = positions[s] + 1;
  // Sliding window W (0: none): only the last W keys are visible, and the
  // grid spans only the chunks a window can overlap, counted from the one
  // holding the sequence's first visible key.
  const int klo = window > 0 ? max(0, nkeys - window) : 0;
  const int c = klo / chunk + blockIdx.x;
  const int k0 = c * chunk;
  if (k0 >= nkeys || k0 + chunk <= klo) return;
  const int k1 = min(k0 + chunk, nkeys);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (read from the first lane), so that the key range and the
  // cache-block lookups below stay in scalar registers: a block-table entry
  // then comes through the scalar cache instead of a vector load (whose
  // result, moved to a scalar register, would first wait for every row load
  // in flight)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, oct = lane & 15;
  const int SUB = chunk / 4;
  const int wk0 = k0 + wave * SUB;
  const int wk1 = min(wk0 + SUB, k1);

  float q[NREP][8];
  {
    const T* qp = Q + (size_t)s * n_q * kHeadDim + (size_t)g * NREP * kHeadDim + oct * 8;
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
      RowSlice<T> x;
      x.load(qp + r * kHeadDim);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[r][e] = x.at(e);  // already times log2(e)/sqrt(d)
    }
  }
  float m[NREP], l[NREP], acc[NREP][8];
#pragma unroll
  for (int r = 0; r < NREP; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  constexpr int U = kDecodeUnroll;
  // One iteration: 4U keys from kb (a multiple of 4U, so they lie in one
  // cache block: one block lookup).  Every lane loads a row; a key outside
  // [klo, wk1) reads the row of key min(key, wk1 - 1) -- a visible or
  // masked slot of the same block, never past the sequence's last key --
  // and is then masked: score -inf, value row zero (a slot that was never
  // written may hold NaN).
  struct Rows {
    RowSlice<T> k[U], v[U];
    bool val[U];
  };
  // Addresses: the iteration's first row as a wave-uniform base (scalar
  // registers) plus a 32-bit byte offset per lane.
  auto load = [&](Rows& b, int kb) {
    const int64_t r0 = kv.row(s, g, kb);
    const uint32_t r0lo = __builtin_amdgcn_readfirstlane((uint32_t)r0);
    const uint32_t r0hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)r0 >> 32));
    const uint64_t off0 = ((uint64_t)r0hi << 32 | r0lo) * (kHeadDim * sizeof(T));
    const char* kbp = reinterpret_cast<const char*>(Kc) + off0;
    const char* vbp = reinterpret_cast<const char*>(Vc) + off0;
    const int lim = wk1 - 1 - kb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = kb + grp + 4 * u;
      b.val[u] = key < wk1 && key >= klo;
      const uint32_t o = (uint32_t)(min(grp + 4 * u, lim) * kHeadDim + oct * 8) * sizeof(T);
      b.k[u].load_stream(reinterpret_cast<const T*>(kbp + o));
      b.v[u].load_stream(reinterpret_cast<const T*>(vbp + o));
    }
  };
  // One head at a time (16 heads: the scores of all heads would not fit in
  // registers).
  auto consume_per_head = [&](Rows& b) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (!b.val[u]) b.v[u].zero();
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
      float sc[U];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[r][e], b.k[u].at(e), d);
        d = row16_sum(d);
        sc[u] = b.val[u] ? d : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      if (mx == -INFINITY) continue;  // uniform within the 16-lane group
      const float m_new = fmaxf(m[r], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[r] - m_new);
      m[r] = m_new;
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(sc[u] - m_new);
        l[r] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, b.v[u].at(e), acc[r][e]);
      }
    }
  };
  // Keys outer, heads inner: each row is widened to fp32 once and used by
  // all n_rep heads at once (per head, the compiler keeps every widened row
  // live across the heads).
  auto consume = [&](Rows& b) {
    if constexpr (NREP > 8) {
      consume_per_head(b);
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (!b.val[u]) b.v[u].zero();
    float sc[NREP][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = b.k[u].at(e);
#pragma unroll
      for (int r = 0; r < NREP; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[r][e], kf[e], d);
        d = row16_sum(d);
        sc[r][u] = b.val[u] ? d : -INFINITY;
      }
    }
    float p[NREP][U];
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[r][u]);
      if (mx == -INFINITY) {  // uniform within the 16-lane group
#pragma unroll
        for (int u = 0; u < U; ++u) p[r][u] = 0.f;
        continue;
      }
      const float m_new = fmaxf(m[r], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[r] - m_new);
      m[r] = m_new;
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[r][u] = __builtin_amdgcn_exp2f(sc[r][u] - m_new);
        l[r] += p[r][u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = b.v[u].at(e);
#pragma unroll
      for (int r = 0; r < NREP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p[r][u], vf[e], acc[r][e]);
    }
  };
  // Iterations stay on the 4U-key grid; keys below klo in the first one are
  // masked.  One row buffer: the loop streams at 7.0-7.5 TB/s in steady
  // state already, and a second buffer (the next iteration's rows loaded
  // before the current ones are consumed) measured slower.
  for (int kb = max(wk0, klo & ~(4 * U - 1)); kb < wk1; kb += 4 * U) {
    Rows b;
    load(b, kb);
    consume(b);
  }

  // Merge the four 16-lane groups of the wave (lanes oct, oct+16, +32, +48).
#pragma unroll
  for (int r = 0; r < NREP; ++r) {
    const float M = xor32_max(xor16_max(m[r]));
    const float sc = (m[r] == -INFINITY) ? 0.f : exp2f(m[r] - M);
    l[r] = xor32_sum(xor16_sum(l[r] * sc));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = xor32_sum(xor16_sum(acc[r][e] * sc));
    m[r] = M;
  }

  // Merge the four waves through LDS.
  __shared__ float sm_ml[4][NREP][2];
  __shared__ float sm_acc[4][NREP][kHeadDim];
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < NREP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][r][oct * 8 + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
      sm_ml[wave][r][0] = m[r];
      sm_ml[wave][r][1] = l[r];
    }
  }
  __syncthreads();
  // partial slot: the chunk's index inside the launched span (with a window
  // the span starts at the chunk holding the first visible key)
  const size_t slot = ((size_t)(s * n_kv + g) * nchunk + blockIdx.x) * NREP;
  for (int idx = tid; idx < NREP * kHeadDim; idx += 256) {
    const int r = idx / kHeadDim, d = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][r][0]);
    float a = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_ml[w][r][0];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      a += sc * sm_acc[w][r][d];
      lt += sc * sm_ml[w][r][1];
    }
    part_acc[(slot + r) * kHeadDim + d] = a;
    if (d == 0) {
      part_ml[(slot + r) * 2 + 0] = M;
      part_ml[(slot + r) * 2 + 1] = lt;
    }
  }
}

// Merge the key chunks of each (sequence, query head): grid (n_q, N), 256
// threads.  Wave w takes chunks w, w+4, ... in one online pass (8 chunks'
// partials loaded together so their latencies overlap; each lane holds two
// of the 128 dims), then the four waves' results are merged through LDS.
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part_acc,
                                                             const float* __restrict__ part_ml,
                                                             const int32_t* __restrict__ positions,
                                                             T* __restrict__ Out, int n_q, int n_kv,
                                                             int nchunk, int chunk,
                                                             int window) {
  constexpr int U = 8, NW = 4;
  const int head = blockIdx.x, s = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_rep = n_q / n_kv;
  const int g = head / n_rep, r = head % n_rep;
  const size_t base = (size_t)(s * n_kv + g) * nchunk;
  // Slots are numbered from the first chunk written (j = c - c_lo), so the
  // first batch is loaded before the sequence length arrives (every slot
  // below nchunk is allocated; the unwritten ones are masked after).
  float M = -INFINITY, lt = 0.f, a0 = 0.f, a1 = 0.f;
  float mv[U], lv[U];
  f32x2_v av[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int jj = min(wave + NW * u, nchunk - 1);
    const size_t sl = (base + jj) * n_rep + r;
    mv[u] = part_ml[sl * 2];
    lv[u] = part_ml[sl * 2 + 1];
    av[u] = *reinterpret_cast<const f32x2_v*>(part_acc + sl * kHeadDim + 2 * lane);
  }
  const int nkeys = positions[s] + 1;
  const int nc = (nkeys + chunk - 1) / chunk;
  const int c_lo = window > 0 ? max(0, nkeys - window) / chunk : 0;  // first chunk written
  const int nw = nc - c_lo;                                          // slots written
  for (int j0 = wave; j0 < nw; j0 += NW * U) {
    if (j0 > wave) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = min(j0 + NW * u, nchunk - 1);
        const size_t sl = (base + jj) * n_rep + r;
        mv[u] = part_ml[sl * 2];
        lv[u] = part_ml[sl * 2 + 1];
        av[u] = *reinterpret_cast<const f32x2_v*>(part_acc + sl * kHeadDim + 2 * lane);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + NW * u >= nw) {
        mv[u] = -INFINITY;
        lv[u] = 0.f;
        av[u] = f32x2_v{0.f, 0.f};
      }
    }
    float mx = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, mv[u]);  // finite: slot j0 < nw is written
    const float sc = exp2f(M - mx);   // 0 on the first pass (M = -inf)
    a0 *= sc;
    a1 *= sc;
    lt *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = exp2f(mv[u] - mx);
      a0 = fmaf(w, av[u][0], a0);
      a1 = fmaf(w, av[u][1], a1);
      lt = fmaf(w, lv[u], lt);
    }
    M = mx;
  }
  // Waves without a chunk keep M = -inf and contribute nothing; wave 0
  // always has slot 0.
  __shared__ float sm_ml[NW][2];
  __shared__ float sm_a[NW][kHeadDim];
  if (lane == 0) {
    sm_ml[wave][0] = M;
    sm_ml[wave][1] = lt;
  }
  sm_a[wave][2 * lane] = a0;
  sm_a[wave][2 * lane + 1] = a1;
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int d = threadIdx.x;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, sm_ml[w][0]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_ml[w][0];
      const float sc = mw == -INFINITY ? 0.f : exp2f(mw - Mx);
      a = fmaf(sc, sm_a[w][d], a);
      l = fmaf(sc, sm_ml[w][1], l);
    }
    Out[(size_t)s * n_q * kHeadDim + head * kHeadDim + d] = from_f32<T>(a / l);
  }
}

template <typename T, int NREP>
static void launch_decode_nrep(const T* Q, const T* Kc, const T* Vc, const int32_t* positions,
                               int N, int n_q, int n_kv, const KvAddr& kv, int window,
                               const DecodeScratch& ws, hipStream_t s) {
  // a window of W keys overlaps at most ceil(W / chunk) + 1 chunks
  // ws.nchunk chunks per (sequence, KV head): all of the cache, or with a
  // window of W keys the ceil(W / chunk) + 1 chunks it can overlap
  const int gx = ws.nchunk;
  // Residency: a short launch (at most 16 workgroups per CU in all) streams
  // faster with 2 resident per CU than with the 5 its registers allow (64
  // sequences, a 4096-key window in 1024-key chunks: 0.188 against 0.194
  // ms; 3 per CU 0.189; 1 per CU 0.239);
  // for long ones (full caches, paged pools) a cap measured within noise
  // either way (0.731-0.740 against 0.732-0.737 ms), so they are left alone.
  // The cap is dynamic LDS the kernel does not use, on top of its own merge
  // buffers (160 KB per CU).
  constexpr int kStaticLds = (4 * NREP * 2 + 4 * NREP * kHeadDim) * (int)sizeof(float);
  const int64_t per_cu = (int64_t)gx * n_kv * N / 256;
  const int pad = per_cu <= 16 ? 160 * 1024 / 2 - kStaticLds - 256 : 0;
  hipLaunchKernelGGL((decode_attn_kernel<T, NREP>), dim3(gx, n_kv, N), dim3(256), pad, s, Q,
                     Kc, Vc, positions, ws.part_acc, ws.part_ml, n_q, n_kv, kv, ws.nchunk,
                     ws.chunk, window);
}

template <typename T>
hipError_t launch_decode_attn(const T* Q, const T* Kc, const T* Vc, const int32_t* positions,
                              T* Out, int N, int n_q, int n_kv, const KvAddr& kv, int window,
                              const DecodeScratch& ws, hipStream_t s) {
  if (window < 0) return hipErrorInvalidValue;
  switch (n_q / n_kv) {
    case 1: launch_decode_nrep<T, 1>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 2: launch_decode_nrep<T, 2>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 3: launch_decode_nrep<T, 3>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 4: launch_decode_nrep<T, 4>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 5: launch_decode_nrep<T, 5>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 6: launch_decode_nrep<T, 6>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 8: launch_decode_nrep<T, 8>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    case 16: launch_decode_nrep<T, 16>(Q, Kc, Vc, positions, N, n_q, n_kv, kv, window, ws, s); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(n_q, N), dim3(256), 0, s, ws.part_acc,
                     ws.part_ml, positions, Out, n_q, n_kv, ws.nchunk, ws.chunk, window);
  return hipGetLastError();
}

bool decode_nrep_supported(int n_rep) {
  return n_rep == 1 || n_rep == 2 || n_rep == 3 || n_rep == 4 || n_rep == 5 || n_rep == 6 ||
         n_rep == 8 || n_rep == 16;
}

template hipError_t launch_decode_attn<float>(const float*, const float*, const float*,
                                              const int32_t*, float*, int, int, int, const KvAddr&,
                                              int, const DecodeScratch&, hipStream_t);
template hipError_t launch_decode_attn<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                               const int32_t*, bf16_t*, int, int, int, const KvAddr&,
                                               int, const DecodeScratch&, hipStream_t);

}  // namespace q3
