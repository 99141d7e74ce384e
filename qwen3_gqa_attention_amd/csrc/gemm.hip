// Projections of the attention block as MFMA GEMMs, C[M,N] = A[M,K] * B[N,K]^T.
//
// Both operands are K-contiguous, the layout the checkpoints store weights in
// ([out, in], "Learning 10", section "Part 2 - tensor by tensor") and the
// layout of the token-major activations, so every MFMA operand fragment is a
// contiguous 16-byte run along K.
//
// Tile: BM x 128 x BK, BK = 128 bytes of K per row.  The 128-wide N tile is
// exactly one head of d_head = 128, so the q/k epilogue sees a whole head:
// the per-head RMSNorm and the RoPE pairing of column c with c + 64 stay
// inside one wavefront.  Each wave owns 32*MI rows and all 128 columns
// (4 MFMA 32x32 blocks): with the 32x32 accumulator layout a lane holds
// columns c, c+32, c+64, c+96 of its rows, so RoPE is lane-local and the
// sum of squares is a 32-lane butterfly.
//
// Staging: global -> VGPR (16-byte loads) -> LDS (double buffer, rows padded
// by 16 bytes so ds_read_b128 of 16 consecutive rows hits distinct banks),
// with the next k-tile's global loads in flight during the current MFMAs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace q3 {

struct StoreEpilogue {
  void* c;
  int ldc;
};

template <typename T, int WM, int MI, bool QKV>
__global__ __launch_bounds__(WM * 64) void gemm_nt_kernel(const T* __restrict__ A,
                                                           const T* __restrict__ B, int M,
                                                           int N, int K, QkvEpilogue qe,
                                                           StoreEpilogue se) {
  using MF = Mfma32<T>;
  constexpr int NT = WM * 64;
  constexpr int BM = 32 * MI * WM;
  constexpr int BN = 128;
  constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;            // 128 bytes of K per row per k-tile
  constexpr int LDK = BK + EPC;          // padded LDS row (elements)
  constexpr int A_CH = BM * 8 / NT;      // 16-byte chunks per thread per k-tile
  constexpr int B_CH = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) T As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hk = lane >> 5;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;

  u32x4_v ra[A_CH], rb[B_CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT, r = c >> 3, cc = c & 7;
      if (m0 + r < M)
        ra[i] = ld16(A + (size_t)(m0 + r) * K + k0 + cc * EPC);
      else
        ra[i] = u32x4_v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT, r = c >> 3, cc = c & 7;
      rb[i] = ld16(B + (size_t)(n0 + r) * K + k0 + cc * EPC);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT, r = c >> 3, cc = c & 7;
      st16(&As[buf][r * LDK + cc * EPC], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT, r = c >> 3, cc = c & 7;
      st16(&Bs[buf][r * LDK + cc * EPC], rb[i]);
    }
  };

  f32x16_v acc[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16_v{};

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const T* as = &As[buf][(wave * 32 * MI + c32) * LDK + hk * MF::KL];
    const T* bs = &Bs[buf][c32 * LDK + hk * MF::KL];
#pragma unroll
    for (int ks = 0; ks < BK / MF::K; ++ks) {
      typename MF::frag af[MI], bfr[4];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = MF::load(as + mi * 32 * LDK + ks * MF::K);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bfr[ni] = MF::load(bs + ni * 32 * LDK + ks * MF::K);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = MF::run(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  if constexpr (!QKV) {
    T* C = reinterpret_cast<T*>(se.c);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + wave * 32 * MI + mi * 32 + mfma32_row(i, lane);
        if (row < M) {
          T* dst = C + (size_t)row * se.ldc + n0 + c32;
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) dst[ni * 32] = from_f32<T>(acc[mi][ni][i]);
        }
      }
  } else {
    // Head index of this N tile: [0, n_q) query heads, then n_kv key heads,
    // then n_kv value heads.
    const int head = blockIdx.x;
    const int kind = head < qe.n_q ? 0 : (head < qe.n_q + qe.n_kv ? 1 : 2);
    float gain[4] = {1.f, 1.f, 1.f, 1.f};
    float w0 = 0.f, w1 = 0.f;
    if (kind != 2) {
      const T* g = reinterpret_cast<const T*>(kind == 0 ? qe.gq : qe.gk);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) gain[ni] = to_f32<T>(g[ni * 32 + c32]);
      w0 = qe.inv_freq[c32];
      w1 = qe.inv_freq[32 + c32];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + wave * 32 * MI + mi * 32 + mfma32_row(i, lane);
        const bool ok = row < M;
        float v0 = acc[mi][0][i], v1 = acc[mi][1][i], v2 = acc[mi][2][i], v3 = acc[mi][3][i];
        const int pos = ok ? qe.positions[row] : 0;
        if (kind != 2) {
          // RMS over the head's 128 columns: 4 per lane, 32 lanes per half-wave.
          float ss = v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
          ss = wave_xor_sum(ss, 1, 16);
          const float rs = rsqrtf(ss * (1.f / 128.f) + qe.eps);
          v0 *= rs * gain[0];
          v1 *= rs * gain[1];
          v2 *= rs * gain[2];
          v3 *= rs * gain[3];
          // RoPE: column c pairs with c + 64 (lane-local: blocks 0/2 and 1/3).
          float s0, c0, s1, c1;
          sincosf(static_cast<float>(pos) * w0, &s0, &c0);
          sincosf(static_cast<float>(pos) * w1, &s1, &c1);
          const float r0 = v0 * c0 - v2 * s0, r2 = v2 * c0 + v0 * s0;
          const float r1 = v1 * c1 - v3 * s1, r3 = v3 * c1 + v1 * s1;
          v0 = r0; v1 = r1; v2 = r2; v3 = r3;
        }
        if (!ok) continue;
        T* dst;
        if (kind == 0) {
          dst = reinterpret_cast<T*>(qe.q_out) + (size_t)row * (qe.n_q * kHeadDim) +
                head * kHeadDim;
        } else {
          const int g = head - qe.n_q - (kind == 2 ? qe.n_kv : 0);
          const int seq = qe.decode ? row : row / qe.rows_per_seq;
          const int slot = qe.decode ? pos : row % qe.rows_per_seq;
          T* cache = reinterpret_cast<T*>(kind == 1 ? qe.k_cache : qe.v_cache);
          dst = cache + ((size_t)(seq * qe.n_kv + g) * qe.cap + slot) * kHeadDim;
        }
        dst[c32] = from_f32<T>(v0);
        dst[32 + c32] = from_f32<T>(v1);
        dst[64 + c32] = from_f32<T>(v2);
        dst[96 + c32] = from_f32<T>(v3);
      }
  }
}

template <typename T, int WM, int MI, bool QKV>
static hipError_t launch_gemm(const T* A, const T* B, int M, int N, int K, const QkvEpilogue& qe,
                              const StoreEpilogue& se, hipStream_t s) {
  constexpr int BM = 32 * MI * WM;
  dim3 grid(N / 128, (M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_nt_kernel<T, WM, MI, QKV>), grid, dim3(WM * 64), 0, s, A, B, M, N, K,
                     qe, se);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qkv_gemm(const T* X, const T* Wqkv, int M, int N, int K, const QkvEpilogue& e,
                           hipStream_t s) {
  StoreEpilogue se{nullptr, 0};
  if (M <= 64) return launch_gemm<T, 2, 1, true>(X, Wqkv, M, N, K, e, se, s);
  return launch_gemm<T, 4, 1, true>(X, Wqkv, M, N, K, e, se, s);
}

template <typename T>
hipError_t launch_proj_gemm(const T* A, const T* W, T* C, int M, int N, int K, hipStream_t s) {
  QkvEpilogue qe{};
  StoreEpilogue se{C, N};
  if (M <= 64) return launch_gemm<T, 2, 1, false>(A, W, M, N, K, qe, se, s);
  return launch_gemm<T, 4, 1, false>(A, W, M, N, K, qe, se, s);
}

template hipError_t launch_qkv_gemm<float>(const float*, const float*, int, int, int,
                                           const QkvEpilogue&, hipStream_t);
template hipError_t launch_qkv_gemm<bf16_t>(const bf16_t*, const bf16_t*, int, int, int,
                                            const QkvEpilogue&, hipStream_t);
template hipError_t launch_proj_gemm<float>(const float*, const float*, float*, int, int, int,
                                            hipStream_t);
template hipError_t launch_proj_gemm<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, int, int, int,
                                             hipStream_t);

}  // namespace q3
