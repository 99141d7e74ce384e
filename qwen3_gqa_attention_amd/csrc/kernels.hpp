// Host-side launchers of the gfx950 kernels (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

typedef uint16_t bf16_t;

// Epilogue of the fused q/k/v projection: per-head RMSNorm of q and k with
// their gains, RoPE on q and k, then q to `q_out` and k/v into the caches.
// log2(e) / sqrt(d_head): softmax(q.k / sqrt(d)) = 2^(q'.k - max) / sum with
// q' = q * kScoreScaleLog2, so the attention kernels use the hardware exp2.
constexpr float kScoreScaleLog2 = 0.1275174308f;

// Where the cached key/value row of (sequence, KV head, key position) lives.
//   contiguous (table == nullptr): caches [seqs, n_kv, cap, 128];
//   paged: pools [num_blocks, n_kv, block_size, 128] and an int32 block table
//   [seqs, max_blocks]: logical block key / block_size of sequence seq is
//   physical block table[seq * max_blocks + key / block_size].
// block_size is a power of two >= 64, so a 64-key tile never straddles a
// block.  row() is the row index in units of 128 elements.
struct KvAddr {
  const int32_t* table;
  int64_t cap;     // contiguous: slots per (sequence, head); paged: block_size
  int max_blocks;  // paged: block-table row length
  int log2_bs;     // paged: log2(block_size)
  int n_kv;
  __host__ __device__ __forceinline__ int64_t row(int seq, int g, int key) const {
    if (!table) return ((int64_t)seq * n_kv + g) * cap + key;
    const int64_t blk = table[(int64_t)seq * max_blocks + (key >> log2_bs)];
    return ((blk * n_kv + g) << log2_bs) + (key & ((1 << log2_bs) - 1));
  }
};

struct QkvEpilogue {
  void* q_out;               // [rows, n_q*128]
  void* k_cache;             // [seqs, n_kv, cap, 128]
  void* v_cache;             // [seqs, n_kv, cap, 128]
  const int32_t* positions;  // [rows] position of each row (decode: its cache slot)
  const void* gq;            // [128] q_norm gain (dtype of the block)
  const void* gk;            // [128] k_norm gain
  const float* rope_rev;     // [128] omega_i / (2 pi) as hi [0..63] + lo [64..127] floats
  int n_q, n_kv;
  KvAddr kv;                 // cache addressing (contiguous or paged)
  int rows_per_seq;          // prefill: T (slot = past + row % T); decode: 1
  int decode;                // 1: cache slot = positions[row]
  float eps;
  const int32_t* past;       // prefill: [seqs] cached tokens before this chunk (slot =
                             // past[seq] + row % T), or null for empty caches
  const void* in_norm_x;     // non-null: the block's input is RMSNorm(x) (gain folded into
                             // the weights); x [rows, d] is read to form 1/rms per row
  float q_scale;             // q~ is stored times this (log2(e) / sqrt(d_head): the
                             // attention kernels then take exp2 of raw dot products)
  const int32_t* cu_seqlens; // prefill of a variable-length batch: [nseq + 1] row offsets,
                             // sequence s owns rows cu[s] .. cu[s+1]-1 (slot = past[s] +
                             // row - cu[s]); null: rows_per_seq rows each
  int nseq;
  int head0;                 // head of the launch's first column (a launch may cover a
                             // column range of the merged q/k/v projection)

  // Sequence and cache slot of projection row `row` (prefill and decode).
  __device__ __forceinline__ void seq_slot(int row, int* seq, int* slot) const {
    if (decode) {
      *seq = row;
      *slot = positions[row];
      return;
    }
    int s, t;
    if (cu_seqlens) {
      // the last sequence whose first row is <= row (empty sequences skipped)
      int lo = 0, hi = nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_seqlens[mid] <= row) lo = mid;
        else hi = mid - 1;
      }
      s = lo;
      t = row - cu_seqlens[lo];
    } else {
      s = row / rows_per_seq;
      t = row % rows_per_seq;
    }
    *seq = s;
    *slot = t + (past ? past[s] : 0);
  }
};

// q/k/v projection X[M,K] * Wqkv[N,K]^T with the fused epilogue; N = (n_q + 2 n_kv) * 128.
// `part` (may be null): fp32 scratch of small_m_partial_floats(M, N, K) floats;
// with it, M <= 64 runs as a split-K GEMM plus a finishing kernel that
// applies the epilogue.
template <typename T>
hipError_t launch_qkv_gemm(const T* X, const T* Wqkv, int M, int N, int K,
                           const QkvEpilogue& e, hipStream_t s, float* part);

// Plain projection C[M,N] = A[M,K] * W[N,K]^T (o_proj); `part` as above;
// `residual` (may be null, layout of C) is added in fp32 before rounding.
template <typename T>
hipError_t launch_proj_gemm(const T* A, const T* W, T* C, int M, int N, int K, hipStream_t s,
                            float* part, const T* residual);

// W[r][c] *= g[c] for a [rows, cols] matrix (folds an input RMSNorm gain
// into the projection weights).
template <typename T>
hipError_t launch_scale_columns(T* W, int rows, int cols, const T* g, hipStream_t s);

// fp32 scratch (floats) the split-K path of an M <= 64 projection needs.
int small_m_partial_floats(int M, int N, int K, int elem_size);

// Causal GQA flash attention of a T_len-token chunk over the caches, which
// hold past[b] earlier tokens of sequence b followed by the chunk (past may
// be null: empty caches).  cu_seqlens (may be null): a variable-length
// batch, sequence b owning token rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of
// the n_tok rows, at most T_len of them; null: every sequence has T_len
// tokens (n_tok = B * T_len).  window > 0 limits each token to the `window`
// most recent keys, its own included (0: full causal attention).
// `part`: fp32 scratch of flash_partial_floats(...) floats (may be null when
// that is 0): with few query tiles the key ranges are split over more
// workgroups and merged by a second kernel.
// fixed_ref in (0, kMaxFixedRef]: every score of the call (q~ . k~ in the
// log2 units of the exponent) is known to lie in [-fixed_ref, fixed_ref];
// the softmax then uses that constant reference instead of a running max.
// 0: running max (no bound known, e.g. keys the call did not write).
constexpr float kMaxFixedRef = 50.f;
template <typename T>
hipError_t launch_flash_prefill(const T* Q, const T* Kc, const T* Vc, T* Out, int B, int T_len,
                                const int32_t* cu_seqlens, int n_tok, int n_q, int n_kv,
                                const KvAddr& kv, const int32_t* past, int window, float* part,
                                float fixed_ref, hipStream_t s);
int flash_splits(int B, int T_len, int n_q, int n_kv);
size_t flash_partial_floats(int B, int T_len, int n_q, int n_kv, int n_tok);

// Split-K decode attention: partial (max, sum, weighted values) per key chunk,
// then the log-sum-exp merge into Out [N, n_q*128].  window > 0: the new
// token sees only its `window` most recent keys (0: all of them).
struct DecodeScratch {
  float* part_acc;  // [N, n_kv, nchunk, n_rep, 128]
  float* part_ml;   // [N, n_kv, nchunk, n_rep, 2]
  int nchunk;       // chunks launched per (sequence, KV head): all of the cache, or with a
                    // window the ceil(W / chunk) + 1 it can overlap (slot = index in that span)
  int chunk;        // keys per chunk (decode_chunk_keys)
};
// keys per chunk for `span` keys per (sequence, KV head), contiguous or paged cache
int decode_chunk_keys(int N, int n_kv, int64_t span, bool paged);
bool decode_nrep_supported(int n_rep);
template <typename T>
hipError_t launch_decode_attn(const T* Q, const T* Kc, const T* Vc, const int32_t* positions,
                              T* Out, int N, int n_q, int n_kv, const KvAddr& kv, int window,
                              const DecodeScratch& ws, hipStream_t s);

}  // namespace q3
