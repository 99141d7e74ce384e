// Projections of the attention block as MFMA GEMMs, C[M,N] = A[M,K] * B[N,K]^T.
//
// Both operands are K-contiguous, the layout the checkpoints store weights in
// ([out, in], "Learning 10", section "Part 2 - tensor by tensor") and the
// layout of the token-major activations, so every MFMA operand fragment is a
// contiguous 16-byte run along K.
//
// Workgroup tile BM x BN x BK (BK = 128 bytes of K per row), WM x WN waves,
// each wave owning (32*MI) x (32*NI) outputs as MI x NI accumulators of the
// 32x32 MFMA.  Large wave tiles keep LDS traffic per MFMA low: the 64x128
// wave tile of the q/k/v GEMM reads 6 fragments (6 KB) from LDS per 8 MFMAs.
// When a projection has only one tile per CU, KG = 2 (or 4, for 64x64
// tiles) gives the tile groups of waves that each run a part of K (see
// gemm_nt_kernel).
//
// For the q/k/v projection NI = 4: a wave's 128 columns are exactly one head
// of d_head = 128, so the epilogue sees whole heads.  With the 32x32
// accumulator layout a lane holds columns c, c+32, c+64, c+96 of its rows:
// the RoPE pair (c, c+64) is lane-local and the head's sum of squares is a
// 32-lane DPP/swizzle reduction.  cos/sin are evaluated in the epilogue from
// the row's position (rope_sincos: exact reduction to a fraction of a
// revolution, then the hardware sin/cos).
//
// Staging: direct global -> LDS loads, double buffered.  LDS rows are 128
// bytes, unpadded, with the 16-byte chunk c of row r stored at chunk
// c ^ ((r >> 1) & 7): the 16-byte writes of 8 lanes per row and the
// 16-byte fragment reads of 16 consecutive rows both hit distinct banks.  The
// next k-tile's loads are in flight during the current tile's MFMAs.
// Results leave through LDS as well, so every global store is 16 bytes of a
// row.  Workgroups are mapped so that each XCD (workgroups are dealt
// round-robin over the 8 XCDs) works on a compact block of tiles, which keeps
// the operands it shares in its own L2.
#include "device_common.hpp"
#include "kernels.hpp"

namespace q3 {

struct StoreEpilogue {
  void* c;
  int ldc;
  const void* residual;  // non-null: C = residual + A W^T (same layout as C), added in fp32
};

// Sum of squares of an operand fragment (for the per-row RMS of the input).
__device__ __forceinline__ float frag_sumsq(const bf16x8_v& a, float acc) {
  bf16x2_v p[4];
  __builtin_memcpy(p, &a, 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_fdot2_f32_bf16(p[e], p[e], acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sumsq(float a, float acc) { return fmaf(a, a, acc); }

constexpr int kXcds = 8;

// sin and cos of the RoPE angle p * omega for an integer position p, with
// omega / (2 pi) given as hi + lo floats.  The angle is reduced in
// revolutions exactly -- p * hi is split into its rounded value and its
// rounding error with one fma, and fract() of a float is exact -- so the
// hardware sin/cos (which take revolutions) see an argument in [0, 1)
// accurate to about 2^-24 revolutions for every position below 2^24 (the
// supported range: such positions convert to float exactly).
__device__ __forceinline__ void rope_sincos(int pos, float whi, float wlo, float* s, float* c) {
  const float p = static_cast<float>(pos);
  const float r = p * whi;
  const float e = fmaf(p, whi, -r) + p * wlo;
  const float f = __builtin_amdgcn_fractf(__builtin_amdgcn_fractf(r) + e);
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

// Linear workgroup id -> (m tile, n tile): XCD x gets the contiguous range
// [x*per, (x+1)*per) of a walk over GN-wide column groups (m slower, n
// faster inside a group).
__device__ __forceinline__ void tile_of_block(int bid, int mt, int nt, int* tm, int* tn) {
  const int total = mt * nt;
  int t = bid;
  if (total % kXcds == 0) {
    const int per = total / kXcds;
    t = (bid % kXcds) * per + bid / kXcds;
  }
  constexpr int GN = 4;
  const int group = t / (GN * mt);
  const int first_n = group * GN;
  const int gw = min(GN, nt - first_n);
  const int r = t - group * GN * mt;
  *tm = r / gw;
  *tn = first_n + r % gw;
}

// Element offset of (row, k) in a swizzled 128-byte-row LDS tile.
template <int EPC>
__device__ __forceinline__ int swz(int row, int k) {
  return row * (8 * EPC) + ((((k / EPC) ^ (row >> 1)) & 7) * EPC) + (k % EPC);
}

// NORM selects the decoder-layer variant.  q/k/v: the input rows are
// RMS-normalised on the fly -- the gain is folded into the weights, and the
// sum of squares of each A row is accumulated from the A fragments the MFMAs
// consume, so 1/rms(row) scales the accumulators in the epilogue.  Plain
// projection: the residual (se.residual) is added to the fp32 accumulators
// before the single rounding.  A compile-time switch, so the plain kernels
// carry none of this (the residual loads would raise register pressure).
//
// KG = 2 or 4 splits the K range of each tile over KG groups of WM x WN
// waves, each with its own LDS stages.  After the main loop every group
// leaves its accumulators in LDS, and each group sums (in group order) and
// finishes 1/KG of the tile's rows.  Used when there is one tile per CU:
// more waves per SIMD, so one wave's MFMAs cover the others' LDS and barrier
// waits, and more loads in flight per CU.
template <typename T, int WM, int WN, int MI, int NI, bool QKV, bool PARTIAL = false,
          int NSTAGE = 2, bool NORM = false, int KG = 1>
__global__ __launch_bounds__(WM * WN * 64 * KG) void gemm_nt_kernel(const T* __restrict__ A,
                                                                const T* __restrict__ B, int M,
                                                                int N, int K, QkvEpilogue qe,
                                                                StoreEpilogue se) {
  using MF = Mfma32<T>;
  constexpr int NT = WM * WN * 64;
  constexpr int BM = 32 * MI * WM;
  constexpr int BN = 32 * NI * WN;
  constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;            // 128 bytes of K per row
  constexpr int KS = BK / MF::K;         // MFMA k-steps per k-tile
  constexpr int STAGE = (BM + BN) * BK;  // elements per LDS stage
  // epilogue staging (bf16 only; fp32 results are stored from registers)
  constexpr int STAGED = sizeof(T) == 2 ? (NT / 64) * (32 * MI) * (32 * NI + 8) : 0;
  // KG > 1: every group's accumulators (and NORM sums of squares), fp32, as
  // [group][wave][lane][MROW] -- each lane's values contiguous, the row
  // length padded to 4 mod 32 floats so that the 16-byte accesses of
  // consecutive lanes fall on distinct banks.
  constexpr int MVALS = MI * NI * 16 + MI;
  constexpr int MROW = MVALS + ((4 - MVALS) % 32 + 32) % 32;
  static_assert(MROW >= MVALS && MROW % 32 == 4, "merge row");
  constexpr int MERGE1 = (NT / 64) * 64 * MROW;  // floats per group
  constexpr int MERGE = KG > 1 ? KG * MERGE1 * 4 / (int)sizeof(T) : 0;
  constexpr int SMEM1 = KG * NSTAGE * STAGE > STAGED ? KG * NSTAGE * STAGE : STAGED;
  constexpr int SMEM = SMEM1 > MERGE ? SMEM1 : MERGE;
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "2 to 4 LDS stages");
  static_assert(KG == 1 || ((KG == 2 || KG == 4) && !PARTIAL),
                "K groups: 1, or 2 or 4 without split-K partials");
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/threads mismatch");
  static_assert(!QKV || NI == 4, "q/k/v epilogue needs one whole head per wave");

  __shared__ __attribute__((aligned(16))) T smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kg = KG > 1 ? (tid >> 6) / (WM * WN) : 0;  // K group
  const int wave = (tid >> 6) % (WM * WN);             // wave inside its group
  const int wm = wave % WM, wn = wave / WM;
  const int c32 = lane & 31;
  const int hk = lane >> 5;
  int tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, N / BN, &tm, &tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  // Direct global -> LDS loads (global_load_lds_dwordx4): lane i of a wave
  // instruction writes the 16 bytes it fetched to LDS at base + 16 * i, so one
  // instruction fills 8 consecutive 128-byte rows.  The swizzle is applied on
  // the global side: the lane that lands on physical chunk p of row r fetches
  // logical chunk p ^ ((r >> 1) & 7).  No registers hold the data and no LDS
  // store instructions are issued; the copy runs while the MFMAs do.
  constexpr int NW = NT / 64;
  constexpr int A_INS = BM / 8 / NW;  // wave instructions per k-tile for A
  constexpr int B_INS = BN / 8 / NW;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows vs waves");
  typedef __attribute__((address_space(3))) void lds_void_t;
  typedef __attribute__((address_space(1))) void glb_void_t;
  T* const gsm = smem + kg * NSTAGE * STAGE;  // this group's stages
  auto gload_lds = [&](int buf, int k0) {
    char* as = reinterpret_cast<char*>(gsm + buf * STAGE);
    char* bs = as + BM * BK * sizeof(T);
    const int rsub = lane >> 3, p = lane & 7;
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int rb8 = (j * NW + wave) * 8;
      const int r = rb8 + rsub;
      const int row = min(m0 + r, M - 1);  // rows past M load a valid row; never stored
      const T* g = A + (size_t)row * K + k0 + (p ^ ((r >> 1) & 7)) * EPC;
      __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)(as + rb8 * 128), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int rb8 = (j * NW + wave) * 8;
      const int r = rb8 + rsub;
      const T* g = B + (size_t)(n0 + r) * K + k0 + (p ^ ((r >> 1) & 7)) * EPC;
      __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)(bs + rb8 * 128), 16, 0, 0);
    }
  };
  // Wait until at most `ahead` k-tiles of this wave's LDS-bound loads are
  // still in flight (loads complete in issue order; s_waitcnt vmcnt(n) with
  // the other counters left alone).
  constexpr int INS = A_INS + B_INS;
  static_assert((NSTAGE - 1) * INS < 64, "vmcnt range");
  auto wait_tiles = [](int ahead) {
    if (NSTAGE >= 4 && ahead >= 3) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((3 * INS) & 15) | (((3 * INS) >> 4) << 14));
    } else if (NSTAGE >= 3 && ahead >= 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * INS) & 15) | (((2 * INS) >> 4) << 14));
    } else if (ahead >= 1) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | (INS & 15) | ((INS >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  };

  f32x16_v acc[MI][NI];
  float ssq[MI];  // NORM: this lane's part of the sum of squares of its A rows
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) ssq[mi] = 0.f;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_v{};

  // Split-K (PARTIAL): blockIdx.y picks a K slice of K / gridDim.y; the fp32
  // partial tile goes to se.c as [gridDim.y][M][N].
  const int KT = K / BK / (PARTIAL ? gridDim.y : KG);
  if constexpr (PARTIAL || KG > 1) {
    const size_t koff = (size_t)(PARTIAL ? blockIdx.y : kg) * KT * BK;
    A += koff;
    B += koff;
  }
  const int arow = wm * 32 * MI + c32;   // this lane's first A row in the tile
  const int brow = wn * 32 * NI + c32;   // this lane's first B row in the tile
  // NSTAGE LDS buffers; k-tile kt lives in buffer kt % NSTAGE.  Every buffer
  // is free at the start, so the first NSTAGE tiles are issued at once (the
  // second tile's latency hides behind the first's); after that, tile
  // kt + NSTAGE - 1 is issued at iteration kt >= 1, into the buffer tile
  // kt - 1 has just released.
  // (0.6B q/k/v 45.2 -> 44.7 us, 4B o_proj 98.7 -> 96.9 us against issuing
  // NSTAGE - 1 tiles first; two alternating runs on one box)
#pragma unroll
  for (int st = 0; st < NSTAGE; ++st)
    if (st < KT) gload_lds(st, st * BK);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt % NSTAGE;
    // tile kt has landed (this wave's part): the tiles issued after it may
    // still be in flight
    wait_tiles(min(kt == 0 ? NSTAGE - 1 : NSTAGE - 2, KT - 1 - kt));
    lds_barrier();                             // ... and every wave's; tile kt-1 is consumed
    // The buffer refilled here held tile kt-1, which every wave finished
    // reading before the barrier above.
    if (kt > 0 && kt + NSTAGE - 1 < KT) gload_lds((kt + NSTAGE - 1) % NSTAGE, (kt + NSTAGE - 1) * BK);
    const T* as = gsm + buf * STAGE;
    const T* bs = as + BM * BK;
    // Fragments are double-buffered in registers: the LDS reads of k-step
    // ks+1 are in flight while the MI*NI MFMAs of step ks run.
    typename MF::frag af[2][MI], bfr[2][NI];
    auto lfrag = [&](int set, int ks) {
      const int k = ks * MF::K + hk * MF::KL;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[set][mi] = MF::load(as + swz<EPC>(arow + mi * 32, k));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[set][ni] = MF::load(bs + swz<EPC>(brow + ni * 32, k));
    };
    lfrag(0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);  // step 0's LDS reads first
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) lfrag((ks + 1) & 1, ks + 1);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = MF::run(af[ks & 1][mi], bfr[ks & 1][ni], acc[mi][ni]);
          if constexpr (NORM && QKV) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) ssq[mi] = frag_sumsq(af[ks & 1][mi], ssq[mi]);
      }
      // Pin the order the scheduler would otherwise undo: each MFMA of this
      // step is followed by one LDS read of the next step.
      constexpr int NR = MI + NI, NM = MI * NI;
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < (NR < NM ? NR : NM); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
        if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
    }
  }
  lds_barrier();  // the epilogue reuses the LDS of the last tiles
  // With K groups every group finishes a share of the tile: group kg sums
  // elements kg*IE .. kg*IE + IE-1 of each accumulator block over the groups
  // (in group order) and runs the epilogue on them -- rows rofs .. rofs +
  // 32/KG - 1 of every 32-row block -- so all the waves share the epilogue.
  constexpr int IE = KG > 1 ? 16 / KG : 16;  // accumulator elements finished per block
  const int rofs = KG > 1 ? (32 / KG) * kg : 0;
  if constexpr (KG > 1) {
    float* const mbase = reinterpret_cast<float*>(smem) + (size_t)(wave * 64 + lane) * MROW;
    {
      float* mw = mbase + (size_t)kg * MERGE1;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<f32x4_v*>(mw + (mi * NI + ni) * 16 + i4 * 4) =
                f32x4_v{acc[mi][ni][i4 * 4], acc[mi][ni][i4 * 4 + 1], acc[mi][ni][i4 * 4 + 2],
                        acc[mi][ni][i4 * 4 + 3]};
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) mw[MI * NI * 16 + mi] = ssq[mi];
    }
    lds_barrier();  // every group's sums are in LDS
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e4 = 0; e4 < IE / 4; ++e4) {
          f32x4_v t = *reinterpret_cast<const f32x4_v*>(mbase + (mi * NI + ni) * 16 + kg * IE + e4 * 4);
#pragma unroll
          for (int g = 1; g < KG; ++g)
            t += *reinterpret_cast<const f32x4_v*>(mbase + (size_t)g * MERGE1 + (mi * NI + ni) * 16 +
                                                   kg * IE + e4 * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mi][ni][e4 * 4 + e] = t[e];
        }
      float q = mbase[MI * NI * 16 + mi];
#pragma unroll
      for (int g = 1; g < KG; ++g) q += mbase[(size_t)g * MERGE1 + MI * NI * 16 + mi];
      ssq[mi] = q;
    }
    lds_barrier();  // merge reads done before the epilogue stages through the same LDS
  }

  // ------------------------------------------------------------------ epilogue
  const int row_base = m0 + wm * 32 * MI;
  if constexpr (PARTIAL) {
    float* P = reinterpret_cast<float*>(se.c) + (size_t)blockIdx.y * M * N;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = row_base + mi * 32 + mfma32_row(i, lane);
        if (row < M) {
          float* dst = P + (size_t)row * N + n0 + wn * 32 * NI + c32;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) dst[ni * 32] = acc[mi][ni][i];
        }
      }
    return;
  }
  if constexpr (NORM && QKV) {
    // Lane l holds half of row (l % 32)'s sum of squares; the accumulator
    // element i of lane l belongs to row mfma32_row(i, l).
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ssq[mi]),
                                                       __float_as_uint(ssq[mi]), false, false);
      const float full = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
#pragma unroll
      for (int i = 0; i < IE; ++i) {
        const float ss = __shfl(full, mfma32_row(i, lane) + rofs, kWave);
        const float rs = rsqrtf(ss / (float)K + qe.eps);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni][i] *= rs;
      }
    }
  }
  if constexpr (!QKV && NORM) {
    const T* res = reinterpret_cast<const T*>(se.residual);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int i = 0; i < IE; ++i) {
        const int row = min(row_base + mi * 32 + rofs + mfma32_row(i, lane), M - 1);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni][i] += to_f32<T>(res[(size_t)row * se.ldc + n0 + wn * 32 * NI + ni * 32 + c32]);
      }
      // one 32-row block's residual loads at a time: bounds the registers
      // they hold in flight
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  int head = 0, kind = 3;  // kind 3: plain projection output
  // 256x256 q/k/v tiles: the two waves of a row block share the RoPE angles
  constexpr bool kShareAngles = QKV && WN == 2 && KG == 1;
  const bool share = kShareAngles && qe.head0 + (n0 >> 7) < qe.n_q + qe.n_kv;
  static_assert(!kShareAngles || WM * MI * 16 * 64 * 16 <= SMEM * (int)sizeof(T), "angles do not fit");
  if constexpr (QKV) {
    // This wave's 128 columns are head head0 + n0/128 + wn: [0, n_q) query heads,
    // then n_kv key heads, then n_kv value heads.
    head = qe.head0 + (n0 >> 7) + wn;
    kind = head < qe.n_q ? 0 : (head < qe.n_q + qe.n_kv ? 1 : 2);
    if constexpr (kShareAngles) {
      // The tile's two waves of a row block need the same (row, frequency)
      // angles: wave wn evaluates frequency c32 + 32*wn for all its rows and
      // the pair swaps them through LDS, halving the sin/cos work.  Every
      // wave of the workgroup takes part when the tile's first head is a
      // query or key head (a value-head wave next to a key head included).
      if (share) {
        const int f = c32 + 32 * wn;
        const float wh = qe.rope_rev[f], wl = qe.rope_rev[64 + f];
        float* ang = reinterpret_cast<float*>(smem) + ((size_t)wm * MI * 16 * 64 + lane) * 4 + 2 * wn;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = min(row_base + mi * 32 + mfma32_row(i, lane), M - 1);
            float sn, cn;
            rope_sincos(qe.positions[row], wh, wl, &sn, &cn);
            *reinterpret_cast<float2*>(ang + (mi * 16 + i) * 64 * 4) = make_float2(cn, sn);
          }
        lds_barrier();  // both frequencies of every row are in LDS
      }
    }
    if (kind != 2) {
      float gain[4];
      const T* g = reinterpret_cast<const T*>(kind == 0 ? qe.gq : qe.gk);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        gain[ni] = to_f32<T>(g[ni * 32 + c32]) * (kind == 0 ? qe.q_scale : 1.f);
      // frequencies c32 and 32 + c32 of this lane, as revolutions (hi + lo)
      const float w0h = qe.rope_rev[c32], w0l = qe.rope_rev[64 + c32];
      const float w1h = qe.rope_rev[32 + c32], w1l = qe.rope_rev[96 + c32];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        float2 cs0[16], cs1[16];
        if constexpr (kShareAngles) {  // kind != 2 implies share here
          const float4* ang4 = reinterpret_cast<const float4*>(smem) + (wm * MI + mi) * 16 * 64 + lane;
#pragma unroll
          for (int i = 0; i < IE; ++i) {
            const float4 a = ang4[i * 64];
            cs0[i] = make_float2(a.x, a.y);
            cs1[i] = make_float2(a.z, a.w);
          }
        } else {
#pragma unroll
          for (int i = 0; i < IE; ++i) {
            const int row = min(row_base + mi * 32 + rofs + mfma32_row(i, lane), M - 1);
            const int pos = qe.positions[row];
            rope_sincos(pos, w0h, w0l, &cs0[i].y, &cs0[i].x);
            rope_sincos(pos, w1h, w1l, &cs1[i].y, &cs1[i].x);
          }
        }
#pragma unroll
        for (int i = 0; i < IE; ++i) {
          float v0 = acc[mi][0][i], v1 = acc[mi][1][i], v2 = acc[mi][2][i], v3 = acc[mi][3][i];
          // RMS over the head's 128 columns: 4 per lane, 32 lanes per half-wave.
          const float ss = half_wave_sum(v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3);
          const float rs = rsqrtf(ss * (1.f / 128.f) + qe.eps);
          v0 *= rs * gain[0];
          v1 *= rs * gain[1];
          v2 *= rs * gain[2];
          v3 *= rs * gain[3];
          // RoPE: column c pairs with c + 64 (lane-local: blocks 0/2 and 1/3).
          acc[mi][0][i] = v0 * cs0[i].x - v2 * cs0[i].y;
          acc[mi][2][i] = v2 * cs0[i].x + v0 * cs0[i].y;
          acc[mi][1][i] = v1 * cs1[i].x - v3 * cs1[i].y;
          acc[mi][3][i] = v3 * cs1[i].x + v1 * cs1[i].y;
        }
      }
    }
  }

  // Destination of row `row`, columns [col0, col0 + 32*NI) of this wave.
  auto dst_row = [&](int row) -> T* {
    if constexpr (!QKV) {
      return reinterpret_cast<T*>(se.c) + (size_t)row * se.ldc + n0 + wn * 32 * NI;
    } else {
      if (kind == 0)
        return reinterpret_cast<T*>(qe.q_out) + (size_t)row * (qe.n_q * kHeadDim) + head * kHeadDim;
      const int g = head - qe.n_q - (kind == 2 ? qe.n_kv : 0);
      int seq, slot;
      qe.seq_slot(row, &seq, &slot);
      T* cache = reinterpret_cast<T*>(kind == 1 ? qe.k_cache : qe.v_cache);
      return cache + qe.kv.row(seq, g, slot) * kHeadDim;
    }
  };

  if (kShareAngles && share) lds_barrier();  // angle reads done before the staging writes
  if constexpr (sizeof(T) == 2) {
    // Stage the wave's (32*MI) x (32*NI) bf16 block in LDS (rows padded by 16
    // bytes), then write whole 16-byte pieces of rows to global memory.
    constexpr int WCOLS = 32 * NI;
    constexpr int LDW = WCOLS + 8;
    constexpr int CPR = WCOLS / 8;        // 16-byte chunks per row
    static_assert(NT / 64 * (32 * MI) * LDW <= SMEM, "staging does not fit");
    constexpr int RB = 32 / (KG > 1 ? KG : 1);  // rows of each 32-row block this wave finishes
    T* st = smem + (kg * (NT / 64) + wave) * (RB * MI) * LDW;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < IE; ++i) {
        const int r = mi * RB + mfma32_row(i, lane);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) st[r * LDW + ni * 32 + c32] = from_f32<T>(acc[mi][ni][i]);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    constexpr int RPI = 64 / CPR;         // rows per wave instruction
#pragma unroll 4
    for (int r0 = 0; r0 < RB * MI; r0 += RPI) {
      const int r = r0 + lane / CPR, ch = lane % CPR;
      const int row = KG > 1 ? row_base + (r / RB) * 32 + rofs + r % RB : row_base + r;
      if ((RPI <= RB * MI || r < RB * MI) && row < M)
        st16(dst_row(row) + ch * 8, ld16(st + r * LDW + ch * 8));
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < IE; ++i) {
        const int row = row_base + mi * 32 + rofs + mfma32_row(i, lane);
        if (row < M) {
          T* dst = dst_row(row) + c32;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) dst[ni * 32] = acc[mi][ni][i];
        }
      }
  }
}

template <typename T, int WM, int WN, int MI, int NI, bool QKV, bool PARTIAL = false,
          int NSTAGE = 2, bool NORM = false, int KG = 1>
static hipError_t launch_gemm(const T* A, const T* B, int M, int N, int K, const QkvEpilogue& qe,
                              const StoreEpilogue& se, hipStream_t s, int ksplit = 1) {
  constexpr int BM = 32 * MI * WM;
  constexpr int BN = 32 * NI * WN;
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  hipLaunchKernelGGL((gemm_nt_kernel<T, WM, WN, MI, NI, QKV, PARTIAL, NSTAGE, NORM, KG>),
                     dim3(tiles, ksplit), dim3(WM * WN * 64 * KG), 0, s, A, B, M, N, K, qe, se);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-sized projections (M <= 64 rows), bound by reading the weights.
// bf16: the skinny kernel below (whole K per workgroup, split over its
// waves).  fp32: the K dimension is split over the grid (many workgroups
// streaming weights at once) into fp32 partials, which a second kernel sums.
// ---------------------------------------------------------------------------
constexpr int kSmallM = 64;

// Number of K slices for an fp32 decode projection: the fewest (a power of two,
// each slice a whole number of 128-byte k-tiles) that give at least 64
// workgroups.  More slices spread the weight stream over more CUs but write
// and re-read more fp32 partials: at 64 rows, 64 workgroups measured fastest
// (0.6B q/k/v 11.2 -> 10.5 us with 2 slices instead of 8; o_proj 10.3 ->
// 7.7 us with 8 instead of 32, partial GEMM plus its finishing kernel).
template <typename T>
static int small_m_ksplit(int N, int K) {
  constexpr int BK = 128 / sizeof(T);
  const int tiles = N / 128;
  int ks = 1;
  while (tiles * ks < 64 && (K / BK) % (ks * 2) == 0) ks *= 2;
  return ks;
}

int small_m_partial_floats(int M, int N, int K, int es) {
  // bf16: one unsplit fp32 product (the skinny kernel below); fp32: the slices
  const int ks = es == 2 ? 1 : small_m_ksplit<float>(N, K);
  return ks * M * N;
}

// ---------------------------------------------------------------------------
// Decode-sized bf16 projection without a K split over the grid: workgroup b
// owns a BM x BN block of C = A W^T over the whole of K, and its eight waves
// each take a contiguous eighth of K, then add their blocks through LDS.
// There is no LDS staging of the operands: each lane loads its 16x16x32 MFMA
// fragments (row or column l % 16, 8 consecutive k at 8 * (l / 16) of a
// 32-k step) straight from global memory, KW steps' worth at a time, so a
// CU has 128 KB of loads in flight at once -- the weights are read once,
// and the block's rows of A come from L2.  Blocks are numbered column block
// fastest; with a multiple of 8 column blocks every row block of a column
// block lands on the same XCD (workgroups go to XCDs round-robin), so its
// slab of W is fetched from HBM into one L2 once.
//   16x16x32 MFMA: lane l holds D row 4 * (l / 16) + i, column l % 16.
// Output: fp32 to Cf (row stride N), or, when Cf is null, T to Cb plus the
// optional residual (same layout), rounded once.
// ---------------------------------------------------------------------------
template <int BM, int BN, int KW>
__global__ __launch_bounds__(512) void skinny_gemm_kernel(const bf16_t* __restrict__ A,
                                                          const bf16_t* __restrict__ W, int M,
                                                          int N, int K, float* __restrict__ Cf,
                                                          bf16_t* __restrict__ Cb,
                                                          const bf16_t* __restrict__ residual) {
  constexpr int RB = BM / 16, CB = BN / 16;
  const int ncb = N / BN;
  const int cb0 = blockIdx.x % ncb, rb0 = blockIdx.x / ncb;
  const int m0 = rb0 * BM, n0 = cb0 * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  // this wave's 32-k steps: a contiguous range
  const int nsteps = K / 32;
  const int spw = (nsteps + 7) / 8;
  const int s_beg = min(wave * spw, nsteps), s_end = min(s_beg + spw, nsteps);
  const bf16_t* ap[RB];
  const bf16_t* wp[CB];
#pragma unroll
  for (int i = 0; i < RB; ++i) ap[i] = A + (size_t)min(m0 + 16 * i + r16, M - 1) * K + kq;
#pragma unroll
  for (int j = 0; j < CB; ++j) wp[j] = W + (size_t)(n0 + 16 * j + r16) * K + kq;
  f32x4_v acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_beg; s0 < s_end; s0 += KW) {
    bf16x8_v af[KW][RB], wf[KW][CB];
    // every load of the chunk first (steps past the range re-read the last
    // one and are zeroed, so the count stays fixed)
#pragma unroll
    for (int u = 0; u < KW; ++u) {
      const int k = min(s0 + u, s_end - 1) * 32;
#pragma unroll
      for (int i = 0; i < RB; ++i) af[u][i] = *reinterpret_cast<const bf16x8_v*>(ap[i] + k);
#pragma unroll
      for (int j = 0; j < CB; ++j) wf[u][j] = *reinterpret_cast<const bf16x8_v*>(wp[j] + k);
    }
    // keep the scheduler from sinking loads between the MFMAs (it would
    // reuse their registers and leave only a few in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KW; ++u) {
      if (s0 + u >= s_end) {
#pragma unroll
        for (int i = 0; i < RB; ++i) af[u][i] = bf16x8_v{};
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][i], wf[u][j], acc[i][j], 0, 0, 0);
    }
  }
  // sum of the eight waves' blocks
  __shared__ f32x4_v red[8][RB * CB][64];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) red[wave][i * CB + j][lane] = acc[i][j];
  __syncthreads();
  for (int q = threadIdx.x; q < RB * CB * 64; q += 512) {
    const int blk = q >> 6, l = q & 63;
    f32x4_v v = red[0][blk][l];
#pragma unroll
    for (int w = 1; w < 8; ++w) v += red[w][blk][l];
    const int col = n0 + (blk % CB) * 16 + (l & 15);
    const int rowb = m0 + (blk / CB) * 16 + 4 * (l >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = rowb + e;
      if (row >= M) break;
      const size_t o = (size_t)row * N + col;
      if (Cf) {
        Cf[o] = v[e];
      } else {
        const float r = residual ? bf16_to_f32(residual[o]) : 0.f;
        Cb[o] = f32_to_bf16(v[e] + r);
      }
    }
  }
}

// Launch of the skinny kernel: 32x32 blocks when they alone give a workgroup
// per CU, else 16x16 (e.g. o_proj of 64 rows, 1024 columns: 256 blocks).
// Each lane keeps 16 fragments (64 VGPRs) in flight per chunk.
static hipError_t launch_skinny(const bf16_t* A, const bf16_t* W, int M, int N, int K, float* Cf,
                                bf16_t* Cb, const bf16_t* residual, hipStream_t s) {
  const int t32 = ((M + 31) / 32) * (N / 32);
  if (N % 32 == 0 && t32 >= 256) {
    hipLaunchKernelGGL((skinny_gemm_kernel<32, 32, 4>), dim3(t32), dim3(512), 0, s, A, W, M, N, K,
                       Cf, Cb, residual);
  } else {
    const int t16 = ((M + 15) / 16) * (N / 16);
    hipLaunchKernelGGL((skinny_gemm_kernel<16, 16, 8>), dim3(t16), dim3(512), 0, s, A, W, M, N, K,
                       Cf, Cb, residual);
  }
  return hipGetLastError();
}

// Sum the K-slice partials of the q/k/v projection for one head (128
// columns) and 16 rows, then QK-Norm, RoPE and the stores, as the GEMM
// epilogue does.  256 threads: row = 16 * blockIdx.y + tid / 16 (one DPP row
// of 16 lanes per token), columns 8 * (tid % 16) .. + 7.  cos/sin are
// evaluated here from positions and omega / (2 pi) (hi + lo floats).  Every
// load that does not depend on another (the first K slice, the row's
// position, the gain, the RoPE constants) is issued before any is used, so
// the kernel waits for memory once.
template <typename T>
__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* __restrict__ part, int ks,
                                                         int M, int N, int K, QkvEpilogue qe) {
  const int head = blockIdx.x;
  const int tid = threadIdx.x, j = tid & 15;
  const int row = blockIdx.y * 16 + (tid >> 4);
  const int kind = head < qe.n_q ? 0 : (head < qe.n_q + qe.n_kv ? 1 : 2);
  const bool ok = row < M;
  const int r = ok ? row : 0;
  const float* p0 = part + (size_t)r * N + head * kHeadDim + j * 8;
  f32x4_v x0 = *reinterpret_cast<const f32x4_v*>(p0);
  f32x4_v x1 = *reinterpret_cast<const f32x4_v*>(p0 + 4);
  const int pos = qe.positions[r];
  const T* gp = reinterpret_cast<const T*>(kind == 0 ? qe.gq : qe.gk) + j * 8;
  T g8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) g8[e] = gp[e];
  const float* rp = qe.rope_rev + (j & 7) * 8;
  const f32x4_v rh0 = *reinterpret_cast<const f32x4_v*>(rp);
  const f32x4_v rh1 = *reinterpret_cast<const f32x4_v*>(rp + 4);
  const f32x4_v rl0 = *reinterpret_cast<const f32x4_v*>(rp + 64);
  const f32x4_v rl1 = *reinterpret_cast<const f32x4_v*>(rp + 68);
  for (int k0 = 1; k0 < ks; k0 += 4) {  // the other slices, four loads in flight at once
    f32x4_v x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* p = p0 + (size_t)(k0 + u) * M * N;
      const bool in = k0 + u < ks;
      x[u][0] = in ? *reinterpret_cast<const f32x4_v*>(p) : f32x4_v{0.f, 0.f, 0.f, 0.f};
      x[u][1] = in ? *reinterpret_cast<const f32x4_v*>(p + 4) : f32x4_v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x0 += x[u][0];
      x1 += x[u][1];
    }
  }
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = x0[e];
    v[4 + e] = x1[e];
  }
  if (qe.in_norm_x) {
    // Input RMSNorm (gain folded into the weights): 1/rms of the row of x,
    // K/16 elements per thread (K is a multiple of 128).
    const T* xr = reinterpret_cast<const T*>(qe.in_norm_x) + (size_t)r * K;
    float sx = 0.f;
    for (int c = j * 8; c < K; c += 128)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = to_f32<T>(xr[c + e]);
        sx = fmaf(xv, xv, sx);
      }
    sx = row16_sum(sx);
    const float rx = rsqrtf(sx / (float)K + qe.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= rx;
  }
  if (kind != 2) {
    // RMS over the head's 128 columns: 8 per thread, 16 threads per row.
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    ss = row16_sum(ss);
    const float rs = rsqrtf(ss * (1.f / 128.f) + qe.eps);
    const float gs = rs * (kind == 0 ? qe.q_scale : 1.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= gs * to_f32<T>(g8[e]);
    // RoPE: column c pairs with c + 64, i.e. thread j with j ^ 8 (DPP row_ror:8).
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cn;
      rope_sincos(pos, e < 4 ? rh0[e] : rh1[e - 4], e < 4 ? rl0[e] : rl1[e - 4], &sn, &cn);
      const float other = dpp_move<0x128>(v[e]);
      v[e] = (j < 8) ? v[e] * cn - other * sn : v[e] * cn + other * sn;
    }
  }
  if (!ok) return;
  T* dst;
  if (kind == 0) {
    dst = reinterpret_cast<T*>(qe.q_out) + (size_t)row * (qe.n_q * kHeadDim) + head * kHeadDim;
  } else {
    const int g = head - qe.n_q - (kind == 2 ? qe.n_kv : 0);
    int seq, slot;
    qe.seq_slot(row, &seq, &slot);
    T* cache = reinterpret_cast<T*>(kind == 1 ? qe.k_cache : qe.v_cache);
    dst = cache + qe.kv.row(seq, g, slot) * kHeadDim;
  }
  dst += j * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = from_f32<T>(v[e]);
}

// out[m][n] = sum over K slices of part[k][m][n], rounded to T.
template <typename T>
__global__ __launch_bounds__(64) void sum_partials_kernel(const float* __restrict__ part, int ks,
                                                          int MN, T* __restrict__ out,
                                                          const T* __restrict__ residual) {
  const int i = (blockIdx.x * 64 + threadIdx.x) * 4;
  if (i >= MN) return;
  // Eight slices' loads in flight at once (a plain loop leaves the latency
  // of each exposed); the sum keeps slice order.
  f32x4_v a = f32x4_v{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < ks; k0 += 8) {
    f32x4_v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = k0 + u < ks ? *reinterpret_cast<const f32x4_v*>(part + (size_t)(k0 + u) * MN + i)
                         : f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  if (residual) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] += to_f32<T>(residual[i + j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) out[i + j] = from_f32<T>(a[j]);
}

constexpr int kCus = 256;

// K groups need a number of 128-byte k-tiles divisible by the group count.
template <typename T>
static bool k_groups_fit(int K, int groups = 2) {
  return (K / (128 / (int)sizeof(T))) % groups == 0;
}

// Tile choice.  Large problems: 256x256 tiles of 8 waves (64x128 each, two
// waves per SIMD so one wave's MFMAs cover the other's LDS and barrier
// waits).  Mid-size: 128x128 tiles.  Decode-sized M <= 64: 64x128 tiles.
template <typename T>
hipError_t launch_qkv_gemm(const T* X, const T* Wqkv, int M, int N, int K, const QkvEpilogue& e,
                           hipStream_t s, float* part) {
  StoreEpilogue se{nullptr, 0, nullptr};
  if (M <= kSmallM && part) {
    int ks = 1;
    hipError_t r;
    if constexpr (sizeof(T) == 2) {
      r = launch_skinny(X, Wqkv, M, N, K, part, nullptr, nullptr, s);
    } else {
      ks = small_m_ksplit<T>(N, K);
      StoreEpilogue ps{part, N, nullptr};
      r = launch_gemm<T, 2, 1, 1, 4, false, true>(X, Wqkv, M, N, K, e, ps, s, ks);
    }
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(qkv_finish_kernel<T>, dim3(N / kHeadDim, (M + 15) / 16), dim3(256), 0, s,
                       part, ks, M, N, K, e);
    return hipGetLastError();
  }
  const bool norm = e.in_norm_x != nullptr;
  if (M <= 64)
    return norm ? launch_gemm<T, 2, 1, 1, 4, true, false, 2, true>(X, Wqkv, M, N, K, e, se, s)
                : launch_gemm<T, 2, 1, 1, 4, true>(X, Wqkv, M, N, K, e, se, s);
  const int t256 = ((M + 255) / 256) * (N / 256), t128 = ((M + 255) / 256) * (N / 128);
  if (N % 256 == 0 && t256 >= kCus) {
    // 256x256 tiles unless their last round leaves many CUs idle: one tile
    // per CU per round, each round costing a fixed ~15 us (prologue,
    // epilogue, stores) plus the main loop, which is half as long for a
    // 256x128 tile (measured on the 0.6B, 4B and wide-GQA shapes).  A third
    // choice covers whole rounds with 256x256 tiles and the remaining
    // columns with 256x128 tiles in a second launch (e.g. the 4B shape:
    // one round of each instead of 1.5 rounds of 256x256 or 3 of 256x128).
    const float k = (float)K;
    const float r256 = 15.f + 0.0245f * k, r128 = 15.f + 0.0125f * k;
    const int mt = (M + 255) / 256;
    const float c256 = (float)((t256 + kCus - 1) / kCus) * r256;
    const float c128 = (float)((t128 + kCus - 1) / kCus) * r128;
    const int n1 = (t256 / kCus) * kCus / mt;  // 256-column tiles in whole rounds
    const int t_rest = mt * ((N - n1 * 256) / 128);
    const float cmix = (n1 > 0 && n1 * 256 < N)
                           ? (float)((mt * n1 + kCus - 1) / kCus) * r256 +
                                 (float)((t_rest + kCus - 1) / kCus) * r128
                           : 1e30f;
    if (cmix < c256 && cmix < c128) {
      const int N1 = n1 * 256;
      QkvEpilogue e2 = e;
      e2.head0 = e.head0 + N1 / kHeadDim;
      hipError_t r = norm ? launch_gemm<T, 4, 2, 2, 4, true, false, 2, true>(X, Wqkv, M, N1, K, e, se, s)
                          : launch_gemm<T, 4, 2, 2, 4, true>(X, Wqkv, M, N1, K, e, se, s);
      if (r != hipSuccess) return r;
      const T* W2 = Wqkv + (size_t)N1 * K;
      return norm ? launch_gemm<T, 8, 1, 1, 4, true, false, 2, true>(X, W2, M, N - N1, K, e2, se, s)
                  : launch_gemm<T, 8, 1, 1, 4, true>(X, W2, M, N - N1, K, e2, se, s);
    }
    if (c256 <= c128)
      return norm ? launch_gemm<T, 4, 2, 2, 4, true, false, 2, true>(X, Wqkv, M, N, K, e, se, s)
                  : launch_gemm<T, 4, 2, 2, 4, true>(X, Wqkv, M, N, K, e, se, s);
  }
  if (t128 >= kCus)  // 256x128 tiles of eight 32x128 waves
    return norm ? launch_gemm<T, 8, 1, 1, 4, true, false, 2, true>(X, Wqkv, M, N, K, e, se, s)
                : launch_gemm<T, 8, 1, 1, 4, true>(X, Wqkv, M, N, K, e, se, s);
  // 128x128 tiles of four 32x128 waves.  At most one per CU (e.g. a
  // 1024-token chunk: 256 tiles): the K range is split over two wave groups,
  // so eight waves keep loads in flight instead of four.
  if (((M + 127) / 128) * (N / 128) <= kCus && k_groups_fit<T>(K))
    return norm ? launch_gemm<T, 4, 1, 1, 4, true, false, 2, true, 2>(X, Wqkv, M, N, K, e, se, s)
                : launch_gemm<T, 4, 1, 1, 4, true, false, 2, false, 2>(X, Wqkv, M, N, K, e, se, s);
  return norm ? launch_gemm<T, 4, 1, 1, 4, true, false, 2, true>(X, Wqkv, M, N, K, e, se, s)
              : launch_gemm<T, 4, 1, 1, 4, true>(X, Wqkv, M, N, K, e, se, s);
}

template <typename T>
hipError_t launch_proj_gemm(const T* A, const T* W, T* C, int M, int N, int K, hipStream_t s,
                            float* part, const T* residual) {
  QkvEpilogue qe{};
  StoreEpilogue se{C, N, residual};
  const bool res = residual != nullptr;
  if constexpr (sizeof(T) == 2) {
    if (M <= kSmallM) return launch_skinny(A, W, M, N, K, nullptr, C, residual, s);
  }
  if (M <= kSmallM && part) {
    const int ks = small_m_ksplit<T>(N, K);
    StoreEpilogue ps{part, N, nullptr};
    hipError_t r = launch_gemm<T, 2, 1, 1, 4, false, true>(A, W, M, N, K, qe, ps, s, ks);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(sum_partials_kernel<T>, dim3((M * N / 4 + 63) / 64), dim3(64), 0, s, part,
                       ks, M * N, C, residual);
    return hipGetLastError();
  }
  if (M <= 64)
    return res ? launch_gemm<T, 2, 1, 1, 4, false, false, 2, true>(A, W, M, N, K, qe, se, s)
               : launch_gemm<T, 2, 1, 1, 4, false>(A, W, M, N, K, qe, se, s);
  // 256x256 tiles once they occupy at least half the CUs: with the long K
  // of o_proj a 256x256 tile beats four 128x128 ones even at 160 tiles
  // (4B shape: 95 against 101 us).
  if (N % 256 == 0 && ((M + 255) / 256) * (N / 256) >= kCus / 2)
    return res ? launch_gemm<T, 4, 2, 2, 4, false, false, 2, true>(A, W, M, N, K, qe, se, s)
               : launch_gemm<T, 4, 2, 2, 4, false>(A, W, M, N, K, qe, se, s);
  // 128x128 tiles of four 64x64 waves.  With exactly one tile per CU (the
  // 0.6B shape) the K range is split over two wave groups; with more, two
  // 4-wave workgroups share each CU.
  const int t128 = ((M + 127) / 128) * (N / 128);
  if (N % 128 == 0 && t128 >= kCus) {
    if (t128 == kCus && k_groups_fit<T>(K))
      return res ? launch_gemm<T, 2, 2, 2, 2, false, false, 2, true, 2>(A, W, M, N, K, qe, se, s)
                 : launch_gemm<T, 2, 2, 2, 2, false, false, 2, false, 2>(A, W, M, N, K, qe, se, s);
    return res ? launch_gemm<T, 2, 2, 2, 2, false, false, 2, true>(A, W, M, N, K, qe, se, s)
               : launch_gemm<T, 2, 2, 2, 2, false>(A, W, M, N, K, qe, se, s);
  }
  // Too few 128x128 tiles to fill the chip (e.g. o_proj of a 1024-token
  // chunk): 64x64 tiles, four 32x32 waves (N is a multiple of 64).  While
  // there is at most one per CU the K range is split over four wave groups
  // (16 waves, 128 KB of LDS stages): the tile is bound by how fast its
  // loads arrive, and that rate grows with the independent load streams a
  // CU keeps in flight (1024-token chunk o_proj: 15.5 -> 13.6 us against
  // two groups).  Larger tiles have no room in LDS for four groups.
  if (((M + 63) / 64) * (N / 64) <= kCus && k_groups_fit<T>(K, 4))
    return res ? launch_gemm<T, 2, 2, 1, 1, false, false, 2, true, 4>(A, W, M, N, K, qe, se, s)
               : launch_gemm<T, 2, 2, 1, 1, false, false, 2, false, 4>(A, W, M, N, K, qe, se, s);
  if (((M + 63) / 64) * (N / 64) <= kCus && k_groups_fit<T>(K))
    return res ? launch_gemm<T, 2, 2, 1, 1, false, false, 2, true, 2>(A, W, M, N, K, qe, se, s)
               : launch_gemm<T, 2, 2, 1, 1, false, false, 2, false, 2>(A, W, M, N, K, qe, se, s);
  return res ? launch_gemm<T, 2, 2, 1, 1, false, false, 2, true>(A, W, M, N, K, qe, se, s)
             : launch_gemm<T, 2, 2, 1, 1, false>(A, W, M, N, K, qe, se, s);
}

template hipError_t launch_qkv_gemm<float>(const float*, const float*, int, int, int,
                                           const QkvEpilogue&, hipStream_t, float*);
template hipError_t launch_qkv_gemm<bf16_t>(const bf16_t*, const bf16_t*, int, int, int,
                                            const QkvEpilogue&, hipStream_t, float*);
template hipError_t launch_proj_gemm<float>(const float*, const float*, float*, int, int, int,
                                            hipStream_t, float*, const float*);
template hipError_t launch_proj_gemm<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, int, int, int,
                                             hipStream_t, float*, const bf16_t*);

template <typename T>
__global__ __launch_bounds__(256) void scale_columns_kernel(T* __restrict__ W, int rows, int cols,
                                                            const T* __restrict__ g) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * cols) return;
  W[i] = from_f32<T>(to_f32<T>(W[i]) * to_f32<T>(g[i % cols]));
}

template <typename T>
hipError_t launch_scale_columns(T* W, int rows, int cols, const T* g, hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  hipLaunchKernelGGL(scale_columns_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     W, rows, cols, g);
  return hipGetLastError();
}
template hipError_t launch_scale_columns<float>(float*, int, int, const float*, hipStream_t);
template hipError_t launch_scale_columns<bf16_t>(bf16_t*, int, int, const bf16_t*, hipStream_t);

}  // namespace q3
