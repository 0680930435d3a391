// fp8_device.h -- device helpers shared by the quantise and GEMM kernels of
// libfp8sg (gfx950 only).
//
// Numerics (stated by the FP8 quantisation training guide, sections "format
// choice: E4M3 and E5M2" and "three scaling algorithms", read with the OCP
// 8-bit formats): the cast of an FP32 value saturates magnitudes above the
// format's largest finite value (and +-inf) to +-max, keeps NaN, and rounds to
// nearest even with the hardware converter v_cvt_pk_{fp8,bf8}_f32.  The scale
// rule is scale = fmax / amax (IEEE FP32 division), 1 for a zero or non-finite
// amax, FLT_MAX when the quotient overflows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8sg {

enum : int { kE4M3 = 0, kE5M2 = 1 };

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<kE4M3> {
  static constexpr uint32_t max_bits = 0x43E00000u;  // 448.0f
  static constexpr float fmax = 448.0f;
  static constexpr int max_exp = 8;                  // 448 = 1.75 * 2^8
};
template <> struct FmtTraits<kE5M2> {
  static constexpr uint32_t max_bits = 0x47600000u;  // 57344.0f
  static constexpr float fmax = 57344.0f;
  static constexpr int max_exp = 15;                 // 57344 = 1.75 * 2^15
};

constexpr float kFltMax = 3.40282346638528859812e+38f;

// Clamp |v| to fmax when fmax < |v| <= inf; NaN and in-range values pass.
// v_med3_f32(v, -fmax, fmax) clamps but turns NaN into a number, so NaN is
// selected back (3 instructions).  NANS = false is for callers that know v is
// not NaN: the clamp alone (1 instruction).
template <int FMT, bool NANS = true>
__device__ __forceinline__ float saturate(float v) {
  constexpr float m = FmtTraits<FMT>::fmax;
  const float r = __builtin_amdgcn_fmed3f(v, -m, m);
  if constexpr (!NANS) return r;
  return __builtin_isnan(v) ? v : r;
}

// Four FP32 values -> four FP8 bytes, element 0 in the lowest byte.
template <int FMT, bool NANS = true>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  a = saturate<FMT, NANS>(a);
  b = saturate<FMT, NANS>(b);
  c = saturate<FMT, NANS>(c);
  d = saturate<FMT, NANS>(d);
  // The first conversion writes the low half and the second the high half,
  // so the initial contents of the word do not matter: it starts as a's bits
  // (a register that dies here) rather than a zero that needs a move.
  int w = __float_as_int(a);
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, w, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// 16-byte streaming load (the input is read exactly once).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// BF16 pair in one 32-bit word: element 0 in the low half.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Magnitude bits of the larger of two packed BF16 values (NaN > inf > finite).
__device__ __forceinline__ uint32_t absmax2(uint32_t w) {
  uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  return lo > hi ? lo : hi;
}
__device__ __forceinline__ uint32_t absmax8(uint4 v) {
  uint32_t a = max(absmax2(v.x), absmax2(v.y));
  uint32_t b = max(absmax2(v.z), absmax2(v.w));
  return max(a, b);
}

// Eight BF16 values (one 16-byte load) times `s` -> eight FP8 bytes.
template <int FMT, bool NANS = true>
__device__ __forceinline__ uint2 cast8(uint4 v, float s) {
  uint2 r;
  r.x = cvt4<FMT, NANS>(bf_lo(v.x) * s, bf_hi(v.x) * s, bf_lo(v.y) * s, bf_hi(v.y) * s);
  r.y = cvt4<FMT, NANS>(bf_lo(v.z) * s, bf_hi(v.z) * s, bf_lo(v.w) * s, bf_hi(v.w) * s);
  return r;
}

template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
  float s = 1.0f;
  if (amax > 0.0f && amax <= kFltMax) {
    s = FmtTraits<FMT>::fmax / amax;
    if (s > kFltMax) s = kFltMax;
  }
  return s;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Max over groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Block-wide max of a uint32 (blockDim.x = NT, multiple of 64); all threads get it.
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wid = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = max(m, red[i]);
  __syncthreads();
  return m;
}

// FP32 -> BF16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  uint32_t lo = __builtin_bit_cast(unsigned short, (__bf16)a);
  uint32_t hi = __builtin_bit_cast(unsigned short, (__bf16)b);
  return lo | (hi << 16);
}

// Buffer descriptors and LDS DMA (buffer_load ... lds).
typedef int v4i __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ pointer (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

// Buffer descriptor over `records` bytes from `base` (raw buffer, no stride,
// range-checked: loads past `records` return zeros).
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t records) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) & 0xffff;
  r[2] = (int)__builtin_amdgcn_readfirstlane(records);
  r[3] = 0x00020000;
  return r;
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from rsrc + voffset into LDS
// at m0 + 16 * lane.  Issued through inline assembly so that the compiler
// neither models it as an LDS write (which would make it wait for the load
// before unrelated LDS reads of the other buffer) nor reorders it; completion
// is awaited explicitly with vmcnt before the workgroup barrier.  m0 is
// reserved by the compiler, so the sequence restores it.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, int voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc)
      : "memory");
}

// The same with 4 bytes per lane (LDS at m0 + 4 * lane).
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, int voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc)
      : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace fp8sg
