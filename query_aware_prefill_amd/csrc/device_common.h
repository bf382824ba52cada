// Device helpers shared by the gfx950 kernels: number formats, MFMA, lane ops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quail {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest, ties to even) packed in a word:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return pack_bf16x2(x, 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two OCP E4M3 codes (byte 0/1 of the selected 16-bit half of w) -> two
// floats, exact (gfx950 decodes OCP E4M3).
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Four E4M3 codes in a 32-bit word -> four bf16 packed in two words, exact
// (every E4M3 value is a bf16 value).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  f32x2_t a = fp8x2_to_f32<false>(w);
  f32x2_t b = fp8x2_to_f32<true>(w);
  lo = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xFFFF0000u);
  hi = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xFFFF0000u);
}

// Four E4M3 codes, decoded and multiplied by `scale`, rounded to bf16.
__device__ __forceinline__ void fp8x4_to_bf16x4_scaled(uint32_t w, float scale, uint32_t& lo,
                                                       uint32_t& hi) {
  f32x2_t a = fp8x2_to_f32<false>(w);
  f32x2_t b = fp8x2_to_f32<true>(w);
  lo = pack_bf16x2(a[0] * scale, a[1] * scale);
  hi = pack_bf16x2(b[0] * scale, b[1] * scale);
}

// float -> OCP E4M3 code: saturate to +-448, round to nearest, ties to even.
// Normal range (|x| >= 2^-6): round the binary32 mantissa to 3 bits in the
// integer domain (carries move into the exponent) and rebias 127 -> 7.
// Subnormal range: the code is the integer nearest to |x| * 2^9 (ties even);
// 8 there is the smallest normal, which is code 8 as well.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t b = __float_as_uint(x);
  uint32_t sign = (b >> 24) & 0x80u;
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return sign | 0x7Fu;     // NaN
  float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a >= 0.015625f) {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    code = (u >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  }
  return sign | code;
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T bitcast(const uint4& u) {
  static_assert(sizeof(T) == 16, "16-byte cast");
  return __builtin_bit_cast(T, u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds_base + 16*i (gfx950 global_load_lds_dwordx4; lds_base is wave-uniform).
// An LDS-DMA load that reads M0 right after an SALU write of M0 needs one
// wait state on this generation, hence the s_nop inside the asm (the
// compiler's hazard recognizer does not look into inline asm).
// Issued through inline asm so that the compiler does not treat every later
// LDS read as a possible alias of the copy and wait for all copies in flight;
// callers wait explicitly (s_waitcnt vmcnt) before the barrier that publishes
// the data. M0 is a register the compiler reserves and does not preserve
// across asm statements; the kernels that use these copies have no other M0
// user (no LDS-DMA builtin, no indexed register moves), so nothing of the
// compiler's lives in M0 across them.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, const void* lds_base) {
  // the low 32 bits of a generic pointer into LDS are its LDS offset (no null
  // check needed: lds_base always points into a __shared__ array)
  const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the saddr form: no 64-bit address arithmetic per lane).
// `lds_addr` is the wave-uniform LDS byte address of the 1-KB destination.
__device__ __forceinline__ void copy16_to_lds_off(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // both operands are wave-uniform; readfirstlane makes that explicit to the
  // compiler (a no-op for values already in SGPRs)
  // (readfirstlane returns a signed int: each half goes through uint32_t so
  // that widening never sign-extends into the other half)
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint32_t a_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t a_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t sa = ((uint64_t)a_hi << 32) | (uint64_t)a_lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const void*>(sa)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// The same copy with the non-temporal hint (data read once: streamed past
// the caches rather than kept in them).
__device__ __forceinline__ void copy16_to_lds_off_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint32_t a_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t a_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t sa = ((uint64_t)a_hi << 32) | (uint64_t)a_lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(reinterpret_cast<const void*>(sa)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// a wave-uniform value as such (v_readfirstlane; free for values in SGPRs)
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// LDS byte address of a __shared__ object (low 32 bits of its generic pointer)
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: exchanges the
// two 32-lane halves, no LDS round trip)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup id remapped so that each of the 8 XCDs (which receive workgroups
// round-robin) processes one contiguous range of logical ids. Returns -1 for
// the padding ids of a grid rounded up to a multiple of 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
  const int64_t per = (total + 7) / 8;
  const int64_t logical = (bid % 8) * per + bid / 8;
  return logical < total ? logical : -1;
}

}  // namespace quail
