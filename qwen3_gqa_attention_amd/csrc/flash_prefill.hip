// Causal grouped-query flash attention for prefill (gfx950, MFMA 32x32).
//
// What it computes ("Assembling a large model from scratch", section "The
// complete code": scores q k^T / sqrt(d_head), the tril causal mask, fp32
// softmax, probabilities times V; query head h reads KV head h / n_rep as in
// "Hand-Writing a Vision-Language Model, Part 1", section "Attention:
// Grouped-Query Attention") -- the softmax reached in one pass with a running
// max and sum (the online softmax that "Qwen3 Architecture Layer-by-Layer"
// names in its cross-entropy section).
//
// Work decomposition.  One workgroup (4 waves) owns 128 "packed rows" of one
// (sequence, KV head): row R stands for token R / n_rep and query head
// g*n_rep + R % n_rep, so the n_rep query heads that share a KV head share
// every K/V tile staged in LDS; the KV heads are never copied.  Each wave owns
// 32 rows.  Workgroups are issued heaviest (longest key range) first.
//
// Per wave and 64-key tile (bf16):
//   S^T[key, q] = K . Q^T    -- A = K rows from LDS, B = Q^T held in VGPRs;
//                               the transposed product puts one query per
//                               lane, so row max / sum are lane-local plus one
//                               exchange between the two half-waves.
//   online softmax in fp32 (exp2 with log2(e)/sqrt(d) folded into the scale)
//   O^T[d, q] += V^T . P^T   -- B = P^T straight from the S^T accumulators
//                               (bf16), A = V^T from an LDS copy of V that is
//                               transposed while staging, with keys permuted
//                               inside each 16-key group so each lane's eight
//                               keys are one 16-byte LDS read.
// fp32 storage uses the 32x32x2 f32 MFMA with the same structure; there V is
// staged untransposed, since each lane reads a single element.
#include "device_common.hpp"
#include "kernels.hpp"

namespace q3 {

template <typename T> struct FlashTile;
template <> struct FlashTile<bf16_t> { static constexpr int BN = 64; };
template <> struct FlashTile<float> { static constexpr int BN = 32; };

// Position, inside its 16-key group, of key k in the transposed V tile.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <typename T>
__global__ __launch_bounds__(256, 2) void flash_prefill_kernel(const T* __restrict__ Q,
                                                            const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc,
                                                            T* __restrict__ Out, int B, int T_len,
                                                            int n_q, int n_kv, int64_t cap,
                                                            float scale_log2) {
  using MF = Mfma32<T>;
  constexpr int BN = FlashTile<T>::BN;
  constexpr int NKB = BN / 32;                 // 32-key blocks per tile
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int LDK = kHeadDim + EPC;          // K tile row (elements)
  constexpr bool VT = sizeof(T) == 2;          // V staged transposed (bf16)
  constexpr int LDV = VT ? (BN + 8) : LDK;
  constexpr int VSZ = VT ? kHeadDim * LDV : BN * LDV;
  constexpr int KCH = BN * (kHeadDim / EPC) / 256;  // K chunks per thread per tile
  constexpr int DSTEPS = kHeadDim / MF::K;     // MFMA steps over d_head

  __shared__ __attribute__((aligned(16))) T Ks[2][BN * LDK];
  __shared__ __attribute__((aligned(16))) T Vs[2][VSZ];

  const int n_rep = n_q / n_kv;
  const int rows_total = T_len * n_rep;
  const int tiles_per_group = (rows_total + 127) / 128;
  const int groups = B * n_kv;
  const int bg = blockIdx.x % groups;
  // Causal balance: the first half of the grid walks query tiles from the
  // heaviest down, the second half from the lightest up, so the two
  // workgroups that share a CU (one from each half) carry about equal work.
  const int rank = blockIdx.x / groups;
  const int half = (tiles_per_group + 1) / 2;
  const int qt = rank < half ? tiles_per_group - 1 - rank : rank - half;
  const int b = bg / n_kv, g = bg % n_kv;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hk = lane >> 5;

  const int R0 = qt * 128;
  const int Rw = R0 + wave * 32;
  const int Rl = Rw + c32;
  const bool row_ok = Rl < rows_total;
  const int tok = row_ok ? Rl / n_rep : T_len - 1;
  const int head = g * n_rep + (row_ok ? Rl % n_rep : 0);
  const bool wave_active = Rw < rows_total;
  const int w_tok_lo = min(Rw, rows_total - 1) / n_rep;
  const int w_tok_hi = min(Rw + 31, rows_total - 1) / n_rep;
  const int kmax = min(R0 + 127, rows_total - 1) / n_rep;
  const int ntiles = kmax / BN + 1;

  // Q^T fragments for the whole d_head, kept in VGPRs.
  typename MF::frag qf[DSTEPS];
  {
    const T* qrow = Q + ((size_t)(b * T_len + tok) * n_q + head) * kHeadDim + hk * MF::KL;
#pragma unroll
    for (int ks = 0; ks < DSTEPS; ++ks) qf[ks] = row_ok ? MF::load(qrow + ks * MF::K) : MF::zero();
  }

  const T* Kg = Kc + (size_t)(b * n_kv + g) * cap * kHeadDim;
  const T* Vg = Vc + (size_t)(b * n_kv + g) * cap * kHeadDim;

  u32x4_v rk[KCH], rv[KCH];
  // Per-thread K/V row pointers for tile 0; each tile advances them by BN rows.
  // bf16: K rows (tid >> 4) + 16 i, chunk tid & 15; V keys 4 (tid & 15) + d,
  // dims 8 (tid >> 4) .. + 7 (the thread owns 4 consecutive keys x 8 dims).
  const int k_row0 = VT ? (tid >> 4) : 0;
  const int v_key0 = VT ? (tid & 15) * 4 : 0;
  const T* kp = Kg + (size_t)k_row0 * kHeadDim + (VT ? (tid & 15) * EPC : 0);
  const T* vp0 = Vg + (size_t)v_key0 * kHeadDim + (VT ? (tid >> 4) * 8 : 0);
  auto gload = [&](int kt) {
    const int kbase = kt * BN;
    if constexpr (VT) {
      const T* kpt = kp + (size_t)kbase * kHeadDim;
      const T* vpt = vp0 + (size_t)kbase * kHeadDim;
      if (kbase + BN <= T_len) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) rk[i] = ld16(kpt + (size_t)i * 16 * kHeadDim);
#pragma unroll
        for (int d = 0; d < 4; ++d) rv[d] = ld16(vpt + (size_t)d * kHeadDim);
      } else {
#pragma unroll
        for (int i = 0; i < KCH; ++i)
          rk[i] = (kbase + k_row0 + 16 * i < T_len) ? ld16(kpt + (size_t)i * 16 * kHeadDim)
                                                    : u32x4_v{0u, 0u, 0u, 0u};
#pragma unroll
        for (int d = 0; d < 4; ++d)
          rv[d] = (kbase + v_key0 + d < T_len) ? ld16(vpt + (size_t)d * kHeadDim) : u32x4_v{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * 256, key = c >> 5, cc = c & 31;
        const size_t off = (size_t)(kbase + key) * kHeadDim + cc * EPC;
        const bool ok = kbase + key < T_len;
        rk[i] = ok ? ld16(Kg + off) : u32x4_v{0u, 0u, 0u, 0u};
        rv[i] = ok ? ld16(Vg + off) : u32x4_v{0u, 0u, 0u, 0u};
      }
    }
  };
  auto sstore = [&](int buf) {
    if constexpr (VT) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * 256, key = c >> 4, cc = c & 15;
        st16(&Ks[buf][key * LDK + cc * EPC], rk[i]);
      }
      const int quad = tid & 15, oct = tid >> 4;
      const int p0 = vt_pos(quad * 4);  // 4 consecutive positions
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims oct*8 + 2w (low halves) and oct*8 + 2w + 1 (high halves)
        const uint32_t x0 = rv[0][w], x1 = rv[1][w], x2 = rv[2][w], x3 = rv[3][w];
        u32x2_v lo{(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
        u32x2_v hi{(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
        *reinterpret_cast<u32x2_v*>(&Vs[buf][(oct * 8 + 2 * w) * LDV + p0]) = lo;
        *reinterpret_cast<u32x2_v*>(&Vs[buf][(oct * 8 + 2 * w + 1) * LDV + p0]) = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * 256, key = c >> 5, cc = c & 31;
        st16(&Ks[buf][key * LDK + cc * EPC], rk[i]);
        st16(&Vs[buf][key * LDV + cc * EPC], rv[i]);
      }
    }
  };

  f32x16_v o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_v{};
  float m_run = -INFINITY, l_run = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    if (wave_active && kt * BN <= w_tok_hi) {
      // S^T = K Q^T (raw scores; the 1/sqrt(d) and log2(e) scale is applied
      // inside the exponent, and max() commutes with a positive scale)
      f32x16_v s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16_v{};
        const T* ks_ptr = &Ks[buf][(kb * 32 + c32) * LDK + hk * MF::KL];
#pragma unroll
        for (int ks = 0; ks < DSTEPS; ++ks) s[kb] = MF::run(MF::load(ks_ptr + ks * MF::K), qf[ks], s[kb]);
      }
      // causal mask (only tiles that cross this wave's diagonal), running max
      if (kt * BN + BN - 1 > w_tok_lo) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kt * BN + kb * 32 + mfma32_row(i, lane) > tok) s[kb][i] = -INFINITY;
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, s[kb][i]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave)) * scale_log2;
      // Rescale the running sum and O only if some lane's max rose.
      if (__ballot(mloc > m_run) != 0) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], scale_log2, -m_run));

      // O^T += V^T P^T.  The running sum adds the bf16-rounded P that the
      // MFMA consumes, two at a time (dot2 with ones).
      if constexpr (VT) {
        float lsum = 0.f;
#pragma unroll
        for (int ks2 = 0; ks2 < BN / 16; ++ks2) {
          const int kb = ks2 >> 1, i0 = (ks2 & 1) * 8;
          const uint32_t w0 = pack_bf16x2(s[kb][i0 + 0], s[kb][i0 + 1]);
          const uint32_t w1 = pack_bf16x2(s[kb][i0 + 2], s[kb][i0 + 3]);
          const uint32_t w2 = pack_bf16x2(s[kb][i0 + 4], s[kb][i0 + 5]);
          const uint32_t w3 = pack_bf16x2(s[kb][i0 + 6], s[kb][i0 + 7]);
          lsum = sum2_bf16(w0, lsum);
          lsum = sum2_bf16(w1, lsum);
          lsum = sum2_bf16(w2, lsum);
          lsum = sum2_bf16(w3, lsum);
          const bf16x8_v pf = __builtin_bit_cast(bf16x8_v, u32x4_v{w0, w1, w2, w3});
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const T* vp = &Vs[buf][(db * 32 + c32) * LDV + ks2 * 16 + hk * 8];
            o[db] = MF::run(MF::load(vp), pf, o[db]);
          }
        }
        l_run += lsum;
      } else {
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) lsum += s[kb][i];
        l_run += lsum;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int st = 0; st < 16; ++st) {
            const int key = kb * 32 + 8 * (st >> 2) + 4 * hk + (st & 3);
#pragma unroll
            for (int db = 0; db < 4; ++db)
              o[db] = MF::run(Vs[buf][key * LDV + db * 32 + c32], s[kb][st], o[db]);
          }
      }
    }
    if (kt + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  if (!row_ok) return;
  l_run += __shfl_xor(l_run, 32, kWave);
  const float inv = 1.f / l_run;
  T* orow = Out + ((size_t)(b * T_len + tok) * n_q + head) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = db * 32 + 8 * i4 + 4 * hk;
      if constexpr (VT) {
        u32x2_v w{pack_bf16x2(o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv),
                  pack_bf16x2(o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2_v*>(orow + d) = w;
      } else {
        f32x4_v w{o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv, o[db][i4 * 4 + 2] * inv,
                  o[db][i4 * 4 + 3] * inv};
        *reinterpret_cast<f32x4_v*>(orow + d) = w;
      }
    }
}

template <typename T>
hipError_t launch_flash_prefill(const T* Q, const T* Kc, const T* Vc, T* Out, int B, int T_len,
                                int n_q, int n_kv, int64_t cap, hipStream_t s) {
  const int n_rep = n_q / n_kv;
  const int tiles = (T_len * n_rep + 127) / 128;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(kHeadDim));
  hipLaunchKernelGGL(flash_prefill_kernel<T>, dim3(tiles * B * n_kv), dim3(256), 0, s, Q, Kc, Vc,
                     Out, B, T_len, n_q, n_kv, cap, scale_log2);
  return hipGetLastError();
}

template hipError_t launch_flash_prefill<float>(const float*, const float*, const float*, float*,
                                                int, int, int, int, int64_t, hipStream_t);
template hipError_t launch_flash_prefill<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                                 bf16_t*, int, int, int, int, int64_t, hipStream_t);

}  // namespace q3
