// dequant.hip — one-time FP8 (OCP E4M3) 128x128-block dequantisation to bf16.
//
// Operation ("DeepSeek-V3.2-Exp · Key–value latent", linear excerpt: one fp32
// scale per 128x128 block of a 1-byte weight; "Absorb key weights", decode
// excerpt: wkv_b is dequantised once and then reused):
//   out[i,j] = bf16_rne( f32_rne( e4m3(w[i,j]) * scale[i/128, j/128] ) )
//
// HBM-bound streaming kernel: 1 byte in, 2 bytes out per element. Each lane
// handles 16 consecutive codes of one row (16-byte load, two 16-byte stores);
// 16 | 128 so the group lies in a single scale block. gfx950's
// v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly; the multiply is one fp32 RNE
// operation and v_cvt_pk_bf16_f32 rounds to nearest-even.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t dequant4(uint32_t codes, float s, uint32_t* hi) {
  floatx2 lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), false);
  floatx2 hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), true);
  *hi = pack_bf16x2(hi2[0] * s, hi2[1] * s);
  return pack_bf16x2(lo2[0] * s, lo2[1] * s);
}

__global__ __launch_bounds__(256) void dequant_fp8_block_kernel(const uint8_t* __restrict__ w,
                                                                const float* __restrict__ scale,
                                                                int64_t rows, int64_t cols,
                                                                uint16_t* __restrict__ out) {
  const int64_t groups_per_row = cols >> 4;
  const int64_t ngroups = rows * groups_per_row;
  const int64_t scols = (cols + 127) >> 7;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; gi < ngroups;
       gi += stride) {
    const int64_t i = gi / groups_per_row;
    const int64_t j = (gi - i * groups_per_row) << 4;
    const float s = scale[(i >> 7) * scols + (j >> 7)];
    const u32x4 c = ld16(w + i * cols + j);
    u32x4 o0, o1;
    uint32_t hi;
    o0[0] = dequant4(c[0], s, &hi);
    o0[1] = hi;
    o0[2] = dequant4(c[1], s, &hi);
    o0[3] = hi;
    o1[0] = dequant4(c[2], s, &hi);
    o1[1] = hi;
    o1[2] = dequant4(c[3], s, &hi);
    o1[3] = hi;
    uint16_t* dst = out + i * cols + j;
    st16(dst, o0);
    st16(dst + 8, o1);
  }
}

hipError_t launch_dequant_fp8_block(const uint8_t* w, const float* scale, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t stream) {
  const int64_t ngroups = rows * (cols >> 4);
  // enough blocks for ~8 waves per CU on 256 CUs; the loop strides the rest
  int64_t blocks = (ngroups + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(dequant_fp8_block_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, w, scale, rows, cols, out);
  return hipGetLastError();
}

}  // namespace mla
