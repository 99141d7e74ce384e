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
// Work decomposition.  One workgroup owns 128 "packed rows" of one
// (sequence, KV head): row R stands for token R / n_rep and query head
// g*n_rep + R % n_rep, so the n_rep query heads that share a KV head share
// every K/V tile staged in LDS; the KV heads are never copied.  The workgroup
// has 8 waves: 4 query blocks of 32 rows times 2 halves of the key range,
// merged at the end (the same log-sum-exp merge as split-K decode).  The two
// waves that share a SIMD thus work on the same query tile for its whole
// duration, which halves its critical path.  Workgroups are issued heaviest
// (longest key range) first.
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
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace q3 {

template <typename T> struct FlashTile;
template <> struct FlashTile<bf16_t> { static constexpr int BN = 64; };
template <> struct FlashTile<float> { static constexpr int BN = 32; };

typedef __bf16 v4bf16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4bf16_t lds_v4bf16_t;

// Transposing LDS read (ds_read_b64_tr_b16): inside each 16-lane group, lane
// i receives element i % 4 of the 8-byte rows addressed by lanes i / 4,
// i / 4 + 4, i / 4 + 8 and i / 4 + 12.
__device__ __forceinline__ v4bf16_t ds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4bf16_t*)(__attribute__((address_space(3))) bf16_t*)(p));
}

// FIXED: the softmax reference is the constant fixed_ref instead of a running
// max.  softmax(s) = 2^(s - m) / sum 2^(s - m) for any finite m, so any
// reference gives the same O / l; a running max is only needed to keep
// 2^(s - m) inside the floating-point range.  When every score is known to
// lie in [-fixed_ref, fixed_ref] with fixed_ref <= kMaxFixedRef, m = fixed_ref
// keeps every probability in [2^-2 kMaxFixedRef, 1] -- normal numbers in fp32
// and in bf16 (same exponent range), so P keeps its full relative precision --
// and the per-tile max, its cross-lane exchange, the rescale test and the
// rescale itself all drop out of the key loop.  The host passes such a bound
// when every key of the call comes from this call's QK-Norm (see
// qwen3_attn_create).
template <typename T, int KSPLIT, bool FIXED>
__global__ __launch_bounds__(KSPLIT * 256, 2) void flash_prefill_kernel(const T* __restrict__ Q,
                                                            const T* __restrict__ Kc,
                                                            const T* __restrict__ Vc,
                                                            T* __restrict__ Out, int B, int T_len,
                                                            const int32_t* __restrict__ cu_seqlens,
                                                            int n_tok,
                                                            int n_q, int n_kv, KvAddr kv,
                                                            const int32_t* __restrict__ past,
                                                            int window, int nsplit,
                                                            float* __restrict__ part,
                                                            float fixed_ref, int items) {
  using MF = Mfma32<T>;
  constexpr int BN = FlashTile<T>::BN;
  constexpr int NKB = BN / 32;                 // 32-key blocks per tile
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr bool VT = sizeof(T) == 2;          // bf16: DMA staging + transposing V reads
  // bf16 tiles are unpadded 256-byte rows filled by direct global->LDS loads
  // (16-byte chunks XOR-swizzled per row); fp32 tiles are padded rows
  // written from registers.
  constexpr int LDK = VT ? kHeadDim : kHeadDim + EPC;  // K tile row (elements)
  constexpr int LDV = LDK;
  constexpr int VSZ = BN * LDV;
  constexpr int KCH = BN * (kHeadDim / EPC) / 256;  // K chunks per thread per tile
  constexpr int DSTEPS = kHeadDim / MF::K;     // MFMA steps over d_head

  // Two key halves x two stages of K and V tiles; after the key loop the
  // same memory carries the second half's partial results to the first.
  constexpr int KSZ = BN * LDK;
  // merge area: 4 query blocks x 64 lanes x (64 O + m + l, padded to 68), fp32
  constexpr int COMB = 4 * 64 * 68 * 4 / sizeof(T);
  constexpr int SMEM = 2 * KSPLIT * (KSZ + VSZ) > COMB ? 2 * KSPLIT * (KSZ + VSZ) : COMB;
  __shared__ __attribute__((aligned(16))) T smem[SMEM];
  auto Ks = [&](int st) { return smem + st * KSZ; };
  auto Vs = [&](int st) { return smem + 2 * KSPLIT * KSZ + st * VSZ; };

  const int n_rep = n_q / n_kv;
  // T_len is the (longest) chunk length the grid was sized for.
  const int tiles_per_group = (T_len * n_rep + 127) / 128;
  const int groups = B * n_kv;
  // With nsplit > 1 the key range of each query tile is cut into nsplit
  // parts run by separate workgroups (few query tiles: fill the chip); each
  // part leaves unnormalised partial results for flash_combine_kernel.
  // The (sequence, KV head) group varies fastest: workgroups are dealt
  // round-robin over the 8 XCDs, so each XCD keeps serving the same groups
  // and their K/V stay in its L2.
  const int bg = blockIdx.x % groups;
  const int rest = blockIdx.x / groups;
  const int split = rest % nsplit;
  const int b = bg / n_kv, g = bg % n_kv;
  // Query tiles are issued heaviest (longest key range) first, so lighter
  // ones fill CUs as they free up.  A paired workgroup (items == 2) runs two
  // work items of the same (sequence, KV head): the heavy query tile
  // tiles_per_group - 1 - j, then the light tile j, so that every workgroup
  // carries the same number of key tiles, and the second item's Q fragments
  // and first K/V tiles are loaded while the first item is merged and
  // stored.
  auto qt_of = [&](int item) {
    const int j = rest / nsplit;
    return item == 0 ? tiles_per_group - 1 - j : j;
  };
  // Token rows of sequence b: q0 .. q0 + Tb - 1 (a variable-length batch
  // gives them in cu_seqlens; else every sequence has T_len).  Query tiles
  // past a shorter sequence's end have no work.
  const int q0 = cu_seqlens ? cu_seqlens[b] : b * T_len;
  const int Tb = cu_seqlens ? cu_seqlens[b + 1] - q0 : T_len;
  const int rows_total = Tb * n_rep;
  if (qt_of(0) * 128 >= rows_total) return;  // whole workgroup, before any barrier
  // Chunked prefill: the sequence already holds P cached tokens, chunk token
  // t is key P + t and sees keys 0 .. P + t (P = 0 for a first prefill).
  const int P = past ? past[b] : 0;
  const int S_len = __builtin_amdgcn_readfirstlane(P + Tb);

  // Wave w owns query block w & 3 (32 rows) over key half w >> 2 (with
  // KSPLIT = 2; with KSPLIT = 1 four waves cover the whole key range).
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qblk = wave & 3, kh = KSPLIT == 2 ? (wave >> 2) : 0;
  const int th = tid & 255;                    // thread index inside the key half
  const int c32 = lane & 31, hk = lane >> 5;

  // The rows and key range of the current work item (set_item).
  int qt, R0, Rw, qtok, tok, head, w_tok_lo, w_tok_hi, key_lo, w_key_lo, w_mask_lo, t_lo, ntiles;
  bool row_ok, wave_active;
  auto set_item = [&](int q) {
    qt = q;
    R0 = qt * 128;
    Rw = R0 + qblk * 32;
    const int Rl = Rw + c32;
    row_ok = Rl < rows_total;
    qtok = row_ok ? Rl / n_rep : Tb - 1;      // token inside the chunk
    tok = P + qtok;                           // its key position
    head = g * n_rep + (row_ok ? Rl % n_rep : 0);
    wave_active = Rw < rows_total;
    w_tok_lo = P + min(Rw, rows_total - 1) / n_rep;
    w_tok_hi = P + min(Rw + 31, rows_total - 1) / n_rep;
    // Sliding window W (0: none): key position j is visible to the token at
    // key position i iff i - W < j <= i.  key_lo is this lane's first visible
    // key; keys below w_mask_lo are masked for at least one row of the wave.
    key_lo = window > 0 ? tok - window + 1 : 0;
    w_key_lo = window > 0 ? w_tok_lo - window + 1 : 0;
    w_mask_lo = window > 0 ? w_tok_hi - window + 1 : 0;
    // Key tiles of the item: from the first key its first row sees to the
    // last key its last row sees.
    const int kmax = P + min(R0 + 127, rows_total - 1) / n_rep;
    const int kmin = window > 0 ? max(0, P + R0 / n_rep - window + 1) : 0;
    const int tl0 = kmin / BN;
    const int ntiles_all = kmax / BN + 1 - tl0;
    const int per_split = (ntiles_all + nsplit - 1) / nsplit;
    const int s_lo = min(split * per_split, ntiles_all);
    t_lo = tl0 + s_lo;
    ntiles = min(s_lo + per_split, ntiles_all) - s_lo;  // this workgroup's key tiles
  };
  set_item(qt_of(0));

  // Q^T fragments for the whole d_head, kept in VGPRs.
  typename MF::frag qf[DSTEPS];
  auto load_q = [&]() {
    const T* qrow = Q + ((size_t)(q0 + qtok) * n_q + head) * kHeadDim + hk * MF::KL;
#pragma unroll
    for (int ks = 0; ks < DSTEPS; ++ks) qf[ks] = row_ok ? MF::load(qrow + ks * MF::K) : MF::zero();
  };
  load_q();

  // Each key tile lies inside one cache block (paged block sizes are powers
  // of two >= 64), so one row lookup per tile addresses all its rows.
  auto tile_row = [&](int kbase) { return kv.row(b, g, kbase); };

  // ---- bf16 staging: direct global -> LDS loads -------------------------
  // One wave instruction (global_load_lds_dwordx4) fills 1 KB = 4 rows of
  // 256 bytes; lane i lands on row i / 16, physical chunk i % 16.  K rows use
  // physical chunk = logical ^ (row & 15): the 16 rows that one K-fragment
  // read touches per bank pass hit 16 different chunks.  V rows use
  // logical ^ 4 * (row & 3): a transposing V read covers 4 rows x 4 chunks.
  // Key rows past the sequence load its last row instead (always written, so
  // finite); the causal mask zeroes their weight.
  const int hw = wave & 3;  // wave index inside its key half
  constexpr int NDMA = VT ? BN / 16 : 1;  // DMA instructions per wave per tile (K and V each)
  constexpr uint32_t ROWB = kHeadDim * sizeof(T);  // bytes per cache row
  // Byte offset, from the tile's first row, of the 16 bytes this lane fetches
  // in DMA instruction j of a full tile (row dma_row(j), swizzled chunk).
  auto dma_row = [&](int j) { return (j * 4 + hw) * 4 + (lane >> 4); };
  uint32_t dk_off[NDMA], dv_off[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int r = dma_row(j);
    dk_off[j] = r * ROWB + ((lane & 15) ^ (r & 15)) * 16;
    dv_off[j] = r * ROWB + ((lane & 15) ^ (4 * (r & 3))) * 16;
  }
  const uint32_t smem_lds = lds_addr(smem);
  auto dma_tile = [&](int kt, int buf) {
    // Everything but the lane offsets is wave-uniform and kept scalar.
    const int kbase = __builtin_amdgcn_readfirstlane(kt * BN);
    const uint32_t lk = smem_lds + (uint32_t)((Ks(buf) - smem) * sizeof(T));
    const uint32_t lv = smem_lds + (uint32_t)((Vs(buf) - smem) * sizeof(T));
    // the tile's first row: one uniform base per tile, per-lane 32-bit offsets
    // (a paged row comes from a per-lane load of one table entry; made
    // scalar here, so the base pointers are formed in scalar registers)
    const int64_t rv = tile_row(kbase);
    const int64_t r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(rv >> 32)) << 32) |
                                 (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)rv));
    const T* kt_base = Kc + r0 * kHeadDim;
    const T* vt_base = Vc + r0 * kHeadDim;
    if (kbase + BN <= S_len) {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const uint32_t r4b = (uint32_t)((j * 4 + hw) * 4 * LDK * sizeof(T));  // instruction's first row
        dma16_to_lds_sv(kt_base, dk_off[j], lk + r4b);
        dma16_to_lds_sv(vt_base, dv_off[j], lv + r4b);
      }
    } else {  // last tile: rows past the sequence re-read its last row
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const uint32_t back = dma_row(j) - (min(kbase + dma_row(j), S_len - 1) - kbase);
        const uint32_t r4b = (uint32_t)((j * 4 + hw) * 4 * LDK * sizeof(T));
        dma16_to_lds_sv(kt_base, dk_off[j] - back * ROWB, lk + r4b);
        dma16_to_lds_sv(vt_base, dv_off[j] - back * ROWB, lv + r4b);
      }
    }
  };

  // ---- fp32 staging: registers -> LDS ----------------------------------
  constexpr int RCH = VT ? 1 : KCH;
  u32x4_v rkA[RCH], rvA[RCH];
  auto gload = [&](int kt) {
    const int kbase = kt * BN;
    const int64_t r0 = tile_row(kbase);
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = th + i * 256, key = c >> 5, cc = c & 31;
      const int64_t off = (r0 + key) * kHeadDim + cc * EPC;
      const bool ok = kbase + key < S_len;
      rkA[i] = ok ? ld16(Kc + off) : u32x4_v{0u, 0u, 0u, 0u};
      rvA[i] = ok ? ld16(Vc + off) : u32x4_v{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = th + i * 256, key = c >> 5, cc = c & 31;
      st16(Ks(buf) + key * LDK + cc * EPC, rkA[i]);
      st16(Vs(buf) + key * LDV + cc * EPC, rvA[i]);
    }
  };

  // m_run: the reference max of the (log2-scaled) scores, at most kMaxSlack
  // below their running max (see the rescale below), -inf until this lane has
  // seen a key.  The score accumulators start at -m_run (0 while m_run is
  // -inf), so they come out of the MFMAs already relative to it.  Reset for
  // every work item.
  f32x16_v o[4];
  float m_run, l_run;
  f32x16_v mbias;
  auto reset_acc = [&]() {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16_v{};
    m_run = FIXED ? fixed_ref : -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mbias[i] = FIXED ? -fixed_ref : 0.f;
    // A fixed reference is the same for every tile: in the 8-wave variant
    // keep it in the 16 VGPRs the first MFMAs read as their accumulator input,
    // instead of letting the compiler treat it as a scalar and rebuild the
    // vector on every tile (0.6B shape: attention 1.3 us faster; the 4-wave
    // variant ran 1% slower with it and keeps the scalar form).
    if constexpr (FIXED && KSPLIT == 2 && sizeof(T) == 2) asm volatile("" : "+v"(mbias));
  };

  // One key tile from stage P (0 or 1, a compile-time constant) of this
  // wave's key half.
  // Per-lane LDS element offsets of the fragment reads, fixed for the whole
  // key loop (the swizzles depend on the lane only): k_off[ks] for the K
  // fragment of MFMA step ks, v_off[db] for the first transposing V read of
  // dim block db (other key groups add whole rows).
  constexpr int NKOFF = VT ? DSTEPS : 1;
  int k_off[NKOFF], v_off[4];
#pragma unroll
  for (int ks = 0; ks < NKOFF; ++ks)
    k_off[ks] = c32 * LDK + (VT ? ((2 * ks + hk) ^ (c32 & 15)) * EPC : 0);
  {
    const int j = lane & 15;
    const int key0 = 4 * hk + (j >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int ch = (d >> 3) ^ (4 * (key0 & 3));  // same for key0 + 16 i and key0 + 8
      v_off[db] = key0 * LDV + ch * EPC + (d & 7);
    }
  }

  // Fragment addresses in stage 0 of this wave's key half, loop-invariant;
  // stage 1 and the other key blocks / rows are compile-time offsets, which
  // the LDS reads take as immediates (no address arithmetic per tile).
  const T* kfrag[NKOFF];
  const T* vfrag[4];
#pragma unroll
  for (int ks = 0; ks < NKOFF; ++ks) kfrag[ks] = Ks(kh * 2) + k_off[ks];
#pragma unroll
  for (int db = 0; db < 4; ++db) vfrag[db] = Vs(kh * 2) + v_off[db];

  auto tile = [&](int kt, auto stage) {
    constexpr int P = decltype(stage)::value;
    const int buf = kh * 2 + P;
    if (wave_active && kt * BN <= w_tok_hi && kt * BN + BN - 1 >= w_key_lo) {
      // S^T = K Q^T - m_run.  Q carries the log2(e)/sqrt(d) factor, so the
      // scores are already in the base-2 units of the exponent.
      // The NKB accumulation chains are interleaved, and each k-step's K
      // fragments are read from LDS one step ahead of their MFMAs.
      f32x16_v s[NKB];
      const T* ks_ptr = Ks(buf);
      // The first MFMA step of each chain adds to mbias instead of zero.
      // element offset of this lane's K fragment for MFMA step ks
      auto kfr = [&](int ks, int kb) -> const T* {
        if constexpr (VT) return kfrag[ks] + P * KSZ + kb * 32 * LDK;
        else return ks_ptr + c32 * LDK + ks * MF::K + hk * MF::KL + kb * 32 * LDK;
      };
      // K fragments are read KPF steps ahead of their MFMAs (a ring of KPF+1
      // register sets): one step's NKB MFMAs are shorter than an LDS read.
      constexpr int KPF = VT ? 3 : 1;
      typename MF::frag kf[KPF + 1][NKB];
#pragma unroll
      for (int p = 0; p < KPF; ++p)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kf[p][kb] = MF::load(kfr(p, kb));
      // The scheduler would sink the reads next to their MFMAs; pin the
      // order: the prologue reads first, then each MFMA followed by one read
      // KPF steps ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, KPF * NKB, 0);
#pragma unroll
      for (int ks = 0; ks < DSTEPS; ++ks) {
        if (ks + KPF < DSTEPS) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            kf[(ks + KPF) % (KPF + 1)][kb] = MF::load(kfr(ks + KPF, kb));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = MF::run(kf[ks % (KPF + 1)][kb], qf[ks], ks == 0 ? mbias : s[kb]);
        if (ks + KPF < DSTEPS) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, NKB, 0);
        }
      }
      // Causal mask (only tiles that cross this wave's diagonal) and the
      // window's lower edge (only tiles that cross it).  Element (kb, i) of
      // this lane is key kt*BN + 4*hk + c with the constant
      // c = kb*32 + 8*(i/4) + i%4, so each test is one compare of a
      // constant against a per-lane limit.
      const int key0 = kt * BN + 4 * hk;
      if (kt * BN + BN - 1 > w_tok_lo) {
        const int lim = tok - key0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
      }
      if (kt * BN < w_mask_lo) {
        const int lo = key_lo - key0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + 8 * (i >> 2) + (i & 3) < lo) s[kb][i] = -INFINITY;
      }
      if constexpr (!FIXED) {
      // Tile max relative to the running max; the two half-waves hold the
      // two halves of each query's keys.
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, s[kb][i]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc),
                                                         __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // m_run is a reference point, not necessarily the exact running max:
      // O and l are both sums of exp2(s - m_run), so any finite reference
      // gives the same O / l.  It must be set on a lane's first tile with an
      // unmasked key, and is raised only once a tile's max exceeds it by more
      // than kMaxSlack, which keeps every probability below 2^kMaxSlack
      // (far from fp32 and bf16 overflow).  With 32 queries per wave, the
      // wave-wide rescale would otherwise run on nearly every tile, because
      // some query's max moves; with the slack it runs only on the first
      // tiles.  When it runs, every lane whose max moved catches up.
      constexpr float kMaxSlack = 8.f;
      const bool first = m_run == -INFINITY;
      const bool moved = first ? (mloc > -INFINITY) : (mloc > 0.f);
      const bool must = first ? moved : (mloc > kMaxSlack);
      if (__ballot(must) != 0) {
        const float delta = moved ? mloc : 0.f;
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) o[db] *= alpha;
        }
        m_run = moved ? (first ? mloc : m_run + delta) : m_run;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] -= delta;
        const float nb = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int i = 0; i < 16; ++i) mbias[i] = nb;
      }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i]);

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
            // V^T fragment (dim db*32 + c32; the 8 keys whose P this lane
            // packed: ks2*16 + 4*hk + {0..3} and + 8 + {0..3}) from two
            // transposing reads of the row-major V tile.  In each read,
            // lane j of a 16-lane group addresses key K0 + j/4, dims
            // D0 + 4*(j%4) .. +3, and receives dim D0 + j of keys K0 .. K0+3.
            const T* vq = vfrag[db] + P * VSZ + ks2 * 16 * LDV;
            const v4bf16_t lo = ds_read_tr16(vq);
            const v4bf16_t hi = ds_read_tr16(vq + 8 * LDV);
            const bf16x8_v vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = MF::run(vf, pf, o[db]);
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
              o[db] = MF::run(Vs(buf)[key * LDV + db * 32 + c32], s[kb][st], o[db]);
          }
      }
    }
  };

  // Key halves: half 0 takes tiles [0, n0), half 1 tiles [n0, ntiles).  Each
  // half has two LDS stages (kh*2, kh*2+1).  Both halves run n0 iterations
  // so every wave meets every barrier.  (n0, base, cnt are uniform; read from
  // the first lane so the loop control stays scalar.)
  int n0, base, cnt;
  auto set_range = [&]() {
    n0 = __builtin_amdgcn_readfirstlane(KSPLIT == 2 ? (ntiles + 1) / 2 : ntiles);
    base = __builtin_amdgcn_readfirstlane(t_lo + (kh ? n0 : 0));
    cnt = __builtin_amdgcn_readfirstlane(kh ? ntiles - n0 : n0);
  };
  set_range();
  const int s0 = kh * 2, s1 = kh * 2 + 1;
  if constexpr (VT) {
    if (cnt > 0) dma_tile(base, s0);
  }

  for (int item = 0; item < items; ++item) {
  reset_acc();
  if constexpr (VT) {
    // Two LDS stages per key half: tile i+1's loads are issued before tile i
    // runs into the stage that tile i-1 used (free once every wave passed the
    // barrier that ended tile i-1).
    // Unrolled by two so that each copy reads a fixed stage: tile i sits in
    // stage i % 2 of the half.  Tile 0 was issued before the item began.
    auto step = [&](int i, auto stage) {
      constexpr int P = decltype(stage)::value;
      if (i + 1 < cnt) dma_tile(base + i + 1, P ? s0 : s1);
      if (i < cnt) tile(base + i, stage);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile i+1 has landed
      lds_barrier();
    };
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and tile 0
    lds_barrier();
    for (int i = 0; i < n0; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      if (i + 1 < n0) step(i + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int i = 0; i < n0; ++i) {
      if (i < cnt) {
        gload(base + i);
        sstore(s0);
      }
      lds_barrier();
      if (i < cnt) tile(base + i, std::integral_constant<int, 0>{});
      lds_barrier();
    }
  }

  // The current item's output rows (set_item moves on to the next item
  // before they are stored).
  const int o_qtok = qtok, o_head = head, o_Rw = __builtin_amdgcn_readfirstlane(Rw);
  const bool o_ok = row_ok;
  const bool more = item + 1 < items;

  // Merge the two key halves: half 1 hands (O, m, l) to half 0 through LDS,
  // each lane's 66 values contiguous (rows of 68 floats: the 16-byte accesses
  // of 16 consecutive lanes hit distinct banks), so both sides move them with
  // 16-byte LDS instructions.
  if constexpr (KSPLIT == 2) {
  float* comb = reinterpret_cast<float*>(smem) + (qblk * 64 + lane) * 68;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4_v*>(comb + db * 16 + i4 * 4) =
            f32x4_v{o[db][i4 * 4], o[db][i4 * 4 + 1], o[db][i4 * 4 + 2], o[db][i4 * 4 + 3]};
    *reinterpret_cast<f32x2_v*>(comb + 64) = f32x2_v{m_run, l_run};
  }
  if (more) {  // the next item's Q fragments (qf is free once the key loop is done)
    set_item(qt_of(item + 1));
    load_q();
  }
  lds_barrier();
  if (kh == 0) {
  if constexpr (FIXED) {
    // both halves are relative to the same reference: plain sums
    l_run += comb[65];
#pragma unroll
    for (int db = 0; db < 4; ++db)
    {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4_v c = *reinterpret_cast<const f32x4_v*>(comb + db * 16 + i4 * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][i4 * 4 + e] += c[e];
      }
      // one block's 16 values in flight at a time (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const float m1 = comb[64], l1 = comb[65];
    const float M = fmaxf(m_run, m1);
    const float a0 = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - M);
    l_run = a0 * l_run + a1 * l1;
    m_run = M;  // O and l are now relative to the merged max (the split path writes it)
#pragma unroll
    for (int db = 0; db < 4; ++db)
    {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4_v c = *reinterpret_cast<const f32x4_v*>(comb + db * 16 + i4 * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][i4 * 4 + e] = a0 * o[db][i4 * 4 + e] + a1 * c[e];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }
  if (more) {
    // comb has been read: the next item's first tiles may land in LDS while
    // this item's rows are normalised and stored.
    lds_barrier();
    set_range();
    if constexpr (VT) {
      if (cnt > 0) dma_tile(base, s0);
    }
  }
  } else if (more) {
    set_item(qt_of(item + 1));
    load_q();
    set_range();
    if constexpr (VT) {
      if (cnt > 0) dma_tile(base, s0);
    }
  }

  if (kh == 0) {
  // (the two lanes of a row have the same o_ok, so the exchange is within
  // valid or within invalid rows)
  l_run += __shfl_xor(l_run, 32, kWave);
  if (nsplit > 1) {
    if (o_ok) {
      // Partial results of this key range: O unnormalised, and (m, l).
      const size_t prow = ((size_t)split * n_tok + q0 + o_qtok) * n_q + o_head;
      float* po = part + prow * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = db * 32 + 8 * i4 + 4 * hk;
          *reinterpret_cast<f32x4_v*>(po + d) =
              f32x4_v{o[db][i4 * 4 + 0], o[db][i4 * 4 + 1], o[db][i4 * 4 + 2], o[db][i4 * 4 + 3]};
        }
      if (hk == 0) {
        float* pml = part + (size_t)nsplit * n_tok * n_q * kHeadDim + prow * 2;
        pml[0] = m_run;
        pml[1] = l_run;
      }
    }
  } else if constexpr (VT && KSPLIT == 2) {
    // The wave's 32 rows leave through LDS so that every store is a whole
    // 16-byte piece of a row (one instruction covers 4 rows; storing from
    // the accumulator layout takes 16 instructions of 32 scattered 16-byte
    // pieces each): 0.6B attention 46.7 -> 45.6 us.  (The 4-wave variant
    // keeps the direct stores: there the extra registers cost more, 4B
    // attention 133.2 -> 135.3 us.)  8 KB per wave, in stages that neither
    // the merge area nor the next item's first tiles use; the next item
    // loads into them only after the barrier that starts its key loop.  Row
    // r keeps its 16-byte chunk c at c ^ (r & 15) (conflict-free on both
    // sides).
    const float inv = 1.f / l_run;
    T* ost = Vs(qblk < 2 ? 1 : 3) + (qblk & 1) * 32 * kHeadDim;
    // this lane's row and swizzle, formed here (an opaque value, so the
    // compiler does not precompute the addresses and hold them through the
    // key loop)
    int wrow = c32;
    asm volatile("" : "+v"(wrow));
    T* wst = ost + wrow * kHeadDim + 4 * hk;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const u32x2_v w{pack_bf16x2(o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv),
                        pack_bf16x2(o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2_v*>(wst + (((db * 4 + i4) ^ (wrow & 15)) * 8)) = w;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_sched_barrier(0);
    int ch = lane & 15, lr = lane >> 4;
    asm volatile("" : "+v"(ch), "+v"(lr));
    // rows o_Rw + r, r = 4 it + lane / 16: token and head advance by whole
    // steps of 4 rows (n_rep divides n_q; no division per store)
    int R = o_Rw + lr;
    int tk = R / n_rep, rm = R - tk * n_rep;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + lr;
      const u32x4_v v = ld16(ost + r * kHeadDim + ((ch ^ (r & 15)) * 8));
      if (R < rows_total)
        st16(Out + ((size_t)(q0 + tk) * n_q + g * n_rep + rm) * kHeadDim + ch * 8, v);
      R += 4;
      rm += 4;
      while (rm >= n_rep) {
        rm -= n_rep;
        ++tk;
      }
      if (it == 3) __builtin_amdgcn_sched_barrier(0);  // four rows' loads in flight at a time
    }
  } else if (o_ok) {
    const float inv = 1.f / l_run;
    T* orow = Out + ((size_t)(q0 + o_qtok) * n_q + o_head) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * hk;
        if constexpr (VT) {
          const u32x2_v w{pack_bf16x2(o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv),
                          pack_bf16x2(o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv)};
          *reinterpret_cast<u32x2_v*>(orow + d) = w;
        } else {
          const f32x4_v w{o[db][i4 * 4 + 0] * inv, o[db][i4 * 4 + 1] * inv,
                          o[db][i4 * 4 + 2] * inv, o[db][i4 * 4 + 3] * inv};
          *reinterpret_cast<f32x4_v*>(orow + d) = w;
        }
      }
  }
  }
  }  // work items
}

// Merge the nsplit partial results of each (token, query head): one online
// log-sum-exp pass over the parts, then O / l rounded to T.  32 threads per
// (token, head), 4 dims each (16-byte loads); 8 pairs per workgroup.  The
// parts are all loaded before the pass (NS >= nsplit slots: 2, 4 or 8), so
// the kernel waits for memory once.
constexpr int kMaxSplits = 8;
template <typename T, int NS>
__global__ __launch_bounds__(256) void flash_combine_kernel(const float* __restrict__ part,
                                                            int nsplit, int pairs,
                                                            T* __restrict__ Out) {
  const int pair = blockIdx.x * 8 + (threadIdx.x >> 5), d = (threadIdx.x & 31) * 4;
  if (pair >= pairs) return;
  const float* pml = part + (size_t)nsplit * pairs * kHeadDim;
  f32x2_v ml[NS];
  f32x4_v ops[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const size_t row = (size_t)min(sp, nsplit - 1) * pairs + pair;
    ml[sp] = *reinterpret_cast<const f32x2_v*>(pml + row * 2);
    ops[sp] = *reinterpret_cast<const f32x4_v*>(part + row * kHeadDim + d);
  }
  // Branch-free, so that the loads above stay ahead of the pass: a part
  // past nsplit, or with no key visible to the row, enters with weights
  // (1, 0) and leaves M, l and O as they are.
  float M = -INFINITY, l = 0.f;
  f32x4_v o = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const bool use = sp < nsplit && ml[sp][0] != -INFINITY;
    const float m = ml[sp][0], lp = ml[sp][1];
    const f32x4_v op = ops[sp];
    const float mn = use ? fmaxf(M, m) : M;
    const float a = use ? __builtin_amdgcn_exp2f(M - mn) : 1.f;  // 0 while M is -inf
    const float w = use ? __builtin_amdgcn_exp2f(m - mn) : 0.f;
    l = l * a + lp * w;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = o[e] * a + op[e] * w;
    M = mn;
  }
  const float inv = 1.f / l;
  T* dst = Out + (size_t)pair * kHeadDim + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[e] * inv);
}

// Query-tile workgroups of one prefill call and the number of key splits:
// below 256 workgroups the key ranges are split so that about 256 run.
static int flash_query_wgs(int B, int T_len, int n_q, int n_kv) {
  return (T_len * (n_q / n_kv) + 127) / 128 * B * n_kv;
}
int flash_splits(int B, int T_len, int n_q, int n_kv) {
  const int wgs = flash_query_wgs(B, T_len, n_q, n_kv);
  if (wgs >= 256) return 1;
  const int sp = 256 / wgs;
  return sp < 2 ? 2 : (sp > kMaxSplits ? kMaxSplits : sp);
}
size_t flash_partial_floats(int B, int T_len, int n_q, int n_kv, int n_tok) {
  const int sp = flash_splits(B, T_len, n_q, n_kv);
  return sp > 1 ? (size_t)sp * n_tok * n_q * (kHeadDim + 2) : 0;
}

template <typename T, bool FIXED>
static void launch_flash_kernel(int wgs, const T* Q, const T* Kc, const T* Vc, T* Out, int B,
                                int T_len, const int32_t* cu_seqlens, int n_tok, int n_q, int n_kv,
                                const KvAddr& kv, const int32_t* past, int window, int nsplit,
                                float* part, float fixed_ref, hipStream_t s) {
  // Few workgroups: split each query tile's key range over two wave groups
  // so both waves of a SIMD serve the same tile.  Many: 4-wave workgroups,
  // two resident per CU.
  if (wgs < 4 * 256) {
    // bf16 with whole 128-row query tiles, an even number of them per group
    // and no key-range split: pair the heavy and light tiles, two work items
    // per workgroup (the second one's loads overlap the first one's merge).
    const int rows = T_len * (n_q / n_kv);
    const int items =
        (sizeof(T) == 2 && nsplit == 1 && !cu_seqlens && rows % 256 == 0) ? 2 : 1;
    hipLaunchKernelGGL((flash_prefill_kernel<T, 2, FIXED>), dim3(wgs / items), dim3(512), 0, s, Q,
                       Kc, Vc, Out, B, T_len, cu_seqlens, n_tok, n_q, n_kv, kv, past, window,
                       nsplit, part, fixed_ref, items);
  } else {
    hipLaunchKernelGGL((flash_prefill_kernel<T, 1, FIXED>), dim3(wgs), dim3(256), 0, s, Q, Kc, Vc,
                       Out, B, T_len, cu_seqlens, n_tok, n_q, n_kv, kv, past, window, nsplit, part,
                       fixed_ref, 1);
  }
}

template <typename T>
hipError_t launch_flash_prefill(const T* Q, const T* Kc, const T* Vc, T* Out, int B, int T_len,
                                const int32_t* cu_seqlens, int n_tok, int n_q, int n_kv,
                                const KvAddr& kv, const int32_t* past, int window, float* part,
                                float fixed_ref, hipStream_t s) {
  if (window < 0 || !(fixed_ref >= 0.f) || fixed_ref > kMaxFixedRef) return hipErrorInvalidValue;
  const int nsplit = flash_splits(B, T_len, n_q, n_kv);
  if (nsplit > 1 && !part) return hipErrorInvalidValue;
  const int wgs = flash_query_wgs(B, T_len, n_q, n_kv) * nsplit;
  if (fixed_ref > 0.f)
    launch_flash_kernel<T, true>(wgs, Q, Kc, Vc, Out, B, T_len, cu_seqlens, n_tok, n_q, n_kv, kv,
                                 past, window, nsplit, part, fixed_ref, s);
  else
    launch_flash_kernel<T, false>(wgs, Q, Kc, Vc, Out, B, T_len, cu_seqlens, n_tok, n_q, n_kv, kv,
                                  past, window, nsplit, part, 0.f, s);
  if (nsplit > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pairs = n_tok * n_q;
    const dim3 grid((pairs + 7) / 8);
    if (nsplit <= 2)
      hipLaunchKernelGGL((flash_combine_kernel<T, 2>), grid, dim3(256), 0, s, part, nsplit, pairs,
                         Out);
    else if (nsplit <= 4)
      hipLaunchKernelGGL((flash_combine_kernel<T, 4>), grid, dim3(256), 0, s, part, nsplit, pairs,
                         Out);
    else
      hipLaunchKernelGGL((flash_combine_kernel<T, kMaxSplits>), grid, dim3(256), 0, s, part,
                         nsplit, pairs, Out);
  }
  return hipGetLastError();
}

template hipError_t launch_flash_prefill<float>(const float*, const float*, const float*, float*,
                                                int, int, const int32_t*, int, int, int,
                                                const KvAddr&, const int32_t*, int, float*, float,
                                                hipStream_t);
template hipError_t launch_flash_prefill<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                                 bf16_t*, int, int, const int32_t*, int, int, int,
                                                 const KvAddr&, const int32_t*, int, float*, float,
                                                 hipStream_t);

}  // namespace q3
