// absorb.hip — fold W^UK into each head's content query.
//
// Operation ("DeepSeek-V3.2-Exp · Absorb key weights", equation and decode
// excerpt; "KV Reconstruction", How it works, first absorb identity):
//   q_lat[b,h,c] = sum_{d<128} q_nope[b,h,d] * wkv_b[h*256 + d, c]
//
// Per head this is a [B x 128] x [128 x 512] product; the 16 MiB of W^UK
// (n_h = 128, bf16) dominates the bytes, so the kernel is built to stream W
// once with wide loads and keep the contraction on MFMA.
//
// bf16 path: one wave per (head, 128-column quarter, 32-row batch tile),
// v_mfma_f32_32x32x16_bf16 with M = batch rows, N = latent columns,
// K = content features d. The contraction runs along W's row axis (its
// stride), so each lane loads 8 consecutive W rows x 4 consecutive columns
// (8-byte loads) and transposes that 8x4 block in registers into the B
// operands of four N-tiles. Tile j's column n is latent column 4n + j, which
// makes each lane's four accumulators four adjacent output columns: one
// 8-byte store per output row.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

__device__ __forceinline__ uint32_t lo_lo(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void absorb_q_bf16_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ q_lat, int B,
                                                            int n_h) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int nbt = (B + 31) >> 5;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // global wave id
  if (gw >= n_h * 4 * nbt) return;
  const int bt = gw % nbt;
  const int cq = (gw / nbt) & 3;
  const int h = gw / (nbt * 4);
  const int b = bt * 32 + n;  // this lane's A-operand row
  const int col0 = cq * 128 + 4 * n;
  const uint16_t* wh = w + static_cast<int64_t>(h) * ROWS_PER_HEAD * D_C + col0;
  const uint16_t* qrow = q_nope + (static_cast<int64_t>(b) * n_h + h) * D_N;

  floatx16 acc[4];
  for (int j = 0; j < 4; j++) acc[j] = floatx16{};
#pragma unroll 2
  for (int ks = 0; ks < D_N / 16; ks++) {
    const int d0 = ks * 16 + g * 8;
    u32x4 a = (b < B) ? ld16(qrow + d0) : u32x4{0, 0, 0, 0};
    u32x2 e[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      e[i] = *reinterpret_cast<const u32x2*>(wh + static_cast<int64_t>(d0 + i) * D_C);
    // e[i] holds W[d0+i][col0 .. col0+3]; operand j needs W[d0..d0+7][col0+j]
    u32x4 bj[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      bj[0][k] = lo_lo(e[2 * k][0], e[2 * k + 1][0]);
      bj[1][k] = hi_hi(e[2 * k][0], e[2 * k + 1][0]);
      bj[2][k] = lo_lo(e[2 * k][1], e[2 * k + 1][1]);
      bj[3][k] = hi_hi(e[2 * k][1], e[2 * k + 1][1]);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] = mfma32x32x16(as_bf16x8(a), as_bf16x8(bj[j]), acc[j]);
  }
  // accumulator r of lane (n, g) is batch row 8*(r/4) + 4*g + r%4, column col0 + j
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int bo = bt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
    if (bo < B) {
      u32x2 v;
      v[0] = pack_bf16x2(acc[0][r], acc[1][r]);
      v[1] = pack_bf16x2(acc[2][r], acc[3][r]);
      *reinterpret_cast<u32x2*>(q_lat + (static_cast<int64_t>(bo) * n_h + h) * D_C + col0) = v;
    }
  }
}

// fp32: one thread per output element, coalesced along the latent columns.
__global__ __launch_bounds__(256) void absorb_q_f32_kernel(const float* __restrict__ q_nope,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ q_lat, int n_h) {
  const int bh = blockIdx.x >> 1;  // (b, h) pair
  const int h = bh % n_h;
  const int c = (blockIdx.x & 1) * 256 + threadIdx.x;
  const float* q = q_nope + static_cast<int64_t>(bh) * D_N;
  const float* wh = w + static_cast<int64_t>(h) * ROWS_PER_HEAD * D_C + c;
  float acc = 0.f;
  for (int d = 0; d < D_N; d++) acc = fmaf(q[d], wh[static_cast<int64_t>(d) * D_C], acc);
  q_lat[static_cast<int64_t>(bh) * D_C + c] = acc;
}

hipError_t launch_absorb_q(const void* q_nope, const void* wkv_b, void* q_lat, int B, int n_h,
                           bool is_bf16, hipStream_t stream) {
  if (is_bf16) {
    const int waves = n_h * 4 * ((B + 31) / 32);
    hipLaunchKernelGGL(absorb_q_bf16_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(wkv_b),
                       static_cast<uint16_t*>(q_lat), B, n_h);
  } else {
    hipLaunchKernelGGL(absorb_q_f32_kernel, dim3(static_cast<unsigned>(B) * n_h * 2), dim3(256), 0,
                       stream, static_cast<const float*>(q_nope),
                       static_cast<const float*>(wkv_b), static_cast<float*>(q_lat), n_h);
  }
  return hipGetLastError();
}

}  // namespace mla
