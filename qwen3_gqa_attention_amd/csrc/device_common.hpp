// Device-side building blocks shared by the gfx950 kernels of the block:
// storage types, MFMA wrappers with their lane layouts, conversions and
// wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;


// ---------------------------------------------------------------------------
// Conversions.  bf16 -> f32 is exact (a shift); f32 -> bf16 rounds to nearest
// even (gfx950 v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}
// Two f32 -> packed bf16x2 (lo = a, hi = b), one v_cvt_pk_bf16_f32.
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cv __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_cv));
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + lo + hi of a packed bf16 pair (one v_dot2 with (1, 1)).
__device__ __forceinline__ float sum2_bf16(uint32_t packed, float acc) {
  const uint32_t ones = 0x3f803f80u;
  bf16x2_v a, b;
  __builtin_memcpy(&a, &packed, 4);
  __builtin_memcpy(&b, &ones, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// 32x32 MFMA, fp32 accumulate.  D[32x32] += A[32xK] * B[Kx32].
//   A fragment: lane l holds row (l % 32), k-slice (l / 32) * KL .. + KL-1
//   B fragment: lane l holds col (l % 32), the same k-slice
//   D:          lane l, element i holds row 8*(i/4) + 4*(l/32) + (i%4),
//               col (l % 32)
// bf16: K = 16 per instruction, KL = 8 values per lane (one 16-byte load).
// f32:  K = 2 per instruction,  KL = 1 value per lane.
// Any permutation of k applied identically to A and B is harmless.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma32;

template <> struct Mfma32<bf16_t> {
  static constexpr int K = 16;
  static constexpr int KL = 8;
  typedef bf16x8_v frag;
  __device__ __forceinline__ static f32x16_v run(const frag& a, const frag& b, f32x16_v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16_t* p) {  // 16-byte aligned
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ __forceinline__ static frag zero() { return frag{}; }
};

template <> struct Mfma32<float> {
  static constexpr int K = 2;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16_v run(frag a, frag b, f32x16_v c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static frag zero() { return 0.f; }
};

// Row of element i of a 32x32 MFMA accumulator held by lane l.
__device__ __forceinline__ int mfma32_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ---------------------------------------------------------------------------
// 16-byte vector type used for global <-> LDS staging.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4_v ld16(const void* p) { return *reinterpret_cast<const u32x4_v*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_v v) { *reinterpret_cast<u32x4_v*>(p) = v; }

// 16-byte direct global -> LDS load (global_load_lds_dwordx4): lane i of the
// wave writes the 16 bytes at sbase + voff (its own offset) to LDS byte
// address lds_base + 16 * i (lds_base must be wave-uniform).  Written as
// inline asm so that the compiler does not treat it as a pending write to all
// of LDS: it would otherwise make every later LDS read it cannot disambiguate
// (the transposing reads, for instance) wait for the load.  The instruction
// has no result register; completion is tracked by vmcnt, so the caller
// waits with s_waitcnt vmcnt before a barrier that publishes the data.
//
// The load is addressed as a wave-uniform base (kept in SGPRs) plus a
// per-lane 32-bit byte offset: no 64-bit address arithmetic per lane.
// `sbase` must be the same in every lane; it is read from the first active
// lane so that the compiler keeps it in scalar registers.
//
// The LDS address goes through M0, which the statement writes itself (M0 is
// declared clobbered).  The CDNA3/CDNA4 ISA requires one wait state between an
// SALU write of M0 and an LDS-DMA load that reads it ("manually inserted wait
// states": SALU writes M0, then a global or buffer load with LDS = 1), and
// the compiler cannot insert it inside an asm statement, so the statement
// carries its own s_nop 0.  Without it the load may still see the M0 value
// from before the write, i.e. land on the LDS rows of an earlier load.
__device__ __forceinline__ void dma16_to_lds_sv(const void* sbase, uint32_t voff,
                                                uint32_t lds_base) {
  // (readfirstlane returns a signed int: each half goes through uint32_t so
  // that widening zero-extends it)
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint64_t u = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               : : "v"(voff), "s"(u), "s"(lds_base) : "memory", "m0");
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load (a workgroup fence on all memory), which
// would drain loads prefetched for later tiles; this one leaves them in
// flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 32 lanes of each half-wave (lanes 0-31 and 32-63) with DPP
// row permutes and one 16-lane row swap; every lane of a half gets the
// half's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// v + the value of lane l ^ 16 (v_permlane16_swap: the odd 16-lane rows of one
// copy trade places with the even rows of the other, so the two results hold,
// in every lane, its own row's value and its partner row's) -- a VALU op, no
// LDS round trip.
__device__ __forceinline__ float xor16_sum(float v) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
// v + the value of lane l ^ 32 (v_permlane32_swap, the same with the two halves).
__device__ __forceinline__ float xor32_sum(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]: xor 1
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]: xor 2
  v += dpp_move<0x141>(v);  // row_half_mirror: the other quad of each 8
  v += dpp_move<0x140>(v);  // row_mirror: the other 8 of each 16
  return xor16_sum(v);      // the other 16 of each 32
}

// Sum over each 16-lane DPP row (lanes 16r .. 16r+15); every lane of the row
// gets the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  return v;
}


}  // namespace q3
