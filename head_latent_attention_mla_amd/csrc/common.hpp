// common.hpp — shared device types and helpers of libmla (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Model dimensions (latent, rotary, content-per-head, value-per-head).
constexpr int D_C = 512;
constexpr int D_R = 64;
constexpr int D_N = 128;
constexpr int D_V = 128;
constexpr int D_QK = D_C + D_R;          // 576 features of a cached row
constexpr int ROWS_PER_HEAD = D_N + D_V;  // 256 rows of wkv_b per head

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest-even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two floats -> packed pair of bf16 (low half = a), round to nearest-even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector(floatx2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Raw buffer resource (base, no stride, 2^31-1 bytes, 32-bit format) in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32));
  r[2] = 0x7FFFFFFF;
  r[3] = 0x00020000;
  return r;
}

// One wave-wide 16-byte-per-lane load from global memory straight into LDS:
// lane i's 16 bytes at (rsrc base + soff + voff) land at LDS byte
// lds_dst + 16*i. Issued from inline assembly so the compiler does not
// serialise consecutive LDS-DMA loads; it has no register outputs (m0, which
// it overwrites, is declared clobbered), and the caller waits with an explicit s_waitcnt vmcnt before the barrier that
// publishes the data.
// The compiler keeps m0 reserved and sets it right before each of its own
// uses, so nothing needs to survive across this statement; the clobber only
// orders the statement against those uses (clang's note that a reserved
// register is not preserved across the statement is what is wanted here).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_dst, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// 16-byte read of a __shared__ object through a generic pointer into it.
__device__ __forceinline__ u32x4 ld_lds16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace mla
