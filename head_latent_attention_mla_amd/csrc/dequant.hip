// dequant.hip — one-time FP8 (OCP E4M3) 128x128-block dequantisation to bf16.
//
// Operation ("DeepSeek-V3.2-Exp · Key–value latent", linear excerpt: one fp32
// scale per 128x128 block of a 1-byte weight; "Absorb key weights", decode
// excerpt: wkv_b is dequantised once and then reused):
//   out[i,j] = bf16_rne( f32_rne( e4m3(w[i,j]) * scale[i/128, j/128] ) )
//
// HBM-bound streaming kernel: 1 byte in, 2 bytes out per element. Each lane
// handles groups of 8 consecutive codes of one row (an 8-byte load, one
// 16-byte store), so the 64 lanes of a wave read 512 contiguous bytes and
// write 1 KiB contiguous bytes per instruction; 8 | 128, so a group lies in
// a single scale block. Each thread keeps DQ_UNROLL groups in flight: all
// its loads, codes and block scales, are issued before the first conversion;
// the stores then go out at most two at a time per wave. The codes are read
// and the output written non-temporally (each byte is touched once).
// Measured on one box, graph-replayed calls of the [32768, 512] weight:
// all loads first, then the stores two at a time, 8.8-8.9 us; each group's
// scale load and store one after another (one store in flight, a scale round
// trip per group) 9.2-9.5 us; all loads first, then eight stores in a burst,
// 9.8-10.0 us; at most four stores in flight, 10.1-10.2 us.
// gfx950's v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly; the multiply is one
// fp32 RNE operation and v_cvt_pk_bf16_f32 rounds to nearest-even.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int DQ_THREADS = 256;

// Non-temporal stores: the 32 MiB output is written once and not re-read by
// this kernel (measured 9.3 against 12.2 us with ordinary stores).
__device__ __forceinline__ void dq_store(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
constexpr int DQ_UNROLL = 8;

__device__ __forceinline__ uint32_t dequant4(uint32_t codes, float s, uint32_t* hi) {
  const floatx2 lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), false);
  const floatx2 hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), true);
  *hi = pack_bf16x2(hi2[0] * s, hi2[1] * s);
  return pack_bf16x2(lo2[0] * s, lo2[1] * s);
}

// I: the index type, 32-bit whenever the weight has fewer than 2^31 groups
// (a 32-bit division per group instead of a 64-bit one).
template <typename I>
__global__ __launch_bounds__(DQ_THREADS) void dequant_fp8_block_kernel(
    const uint8_t* __restrict__ w, const float* __restrict__ scale, I n8, I g8_row, I scols,
    uint16_t* __restrict__ out) {
  const I stride = static_cast<I>(gridDim.x) * DQ_THREADS * DQ_UNROLL;
  for (I base = static_cast<I>(blockIdx.x) * DQ_THREADS * DQ_UNROLL + threadIdx.x; base < n8;
       base += stride) {
    // every load of the thread's groups (codes and their block scales) is
    // issued before the first conversion waits for any of them. Groups past
    // the end re-read and re-write the last group (the same bytes again), so
    // no group is behind a branch: with a branch per group the compiler sinks
    // that group's loads into it, after the previous group's store.
    I gi[DQ_UNROLL];
    u32x2 c[DQ_UNROLL];
    float s[DQ_UNROLL];
#pragma unroll
    for (int u = 0; u < DQ_UNROLL; u++) {
      gi[u] = min(base + static_cast<I>(u * DQ_THREADS), n8 - 1);
      c[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(w + static_cast<int64_t>(gi[u]) * 8));
      const I i = gi[u] / g8_row;       // row
      const I j8 = gi[u] - i * g8_row;  // group within the row: columns 8*j8 .. 8*j8+7
      s[u] = scale[static_cast<int64_t>(i >> 7) * scols + (j8 >> 4)];
    }
    // (the scheduler would otherwise start the first conversion, and wait for
    // its codes, before the last loads are out)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < DQ_UNROLL; u++) {
      u32x4 o;
      uint32_t hi;
      o[0] = dequant4(c[u][0], s[u], &hi);
      o[1] = hi;
      o[2] = dequant4(c[u][1], s[u], &hi);
      o[3] = hi;
      // at most two stores of the wave in flight (loads and stores retire
      // through one in-order counter, and every load has landed by the
      // second store): paced stores stream faster than a burst of eight
      if (u > 0) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      dq_store(out + static_cast<int64_t>(gi[u]) * 8, o);
    }
  }
}

hipError_t launch_dequant_fp8_block(const uint8_t* w, const float* scale, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t stream) {
  const int64_t n8 = rows * (cols / 8);
  const int64_t scols = (cols + 127) >> 7;
  // one pass over the weight by 2048 workgroups at most; the loop strides
  // the rest
  int64_t blocks = (n8 + DQ_THREADS * DQ_UNROLL - 1) / (DQ_THREADS * DQ_UNROLL);
  if (blocks > 2048) blocks = 2048;
  // 32-bit indices while the loop's last base plus its stride still fits
  if (n8 + static_cast<int64_t>(blocks) * DQ_THREADS * DQ_UNROLL < (int64_t{1} << 31)) {
    hipLaunchKernelGGL(dequant_fp8_block_kernel<uint32_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(DQ_THREADS), 0, stream, w, scale, static_cast<uint32_t>(n8),
                       static_cast<uint32_t>(cols / 8), static_cast<uint32_t>(scols), out);
  } else {
    hipLaunchKernelGGL(dequant_fp8_block_kernel<int64_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(DQ_THREADS), 0, stream, w, scale, n8, cols / 8, scols, out);
  }
  return hipGetLastError();
}

}  // namespace mla
