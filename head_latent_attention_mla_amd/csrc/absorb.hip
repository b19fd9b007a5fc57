// absorb.hip — fold W^UK into each head's content query.
//
// Operation ("DeepSeek-V3.2-Exp · Absorb key weights", equation and decode
// excerpt; "KV Reconstruction", How it works, first absorb identity):
//   q_lat[b,h,c] = sum_{d<128} q_nope[b,h,d] * wkv_b[h*256 + d, c]
//
// Per head this is a [B x 128] x [128 x 512] product; the 16 MiB of W^UK
// (n_h = 128, bf16) dominates the bytes, so the kernel is built to have all
// of W in flight at once and keep the contraction on MFMA.
//
// bf16 path: one workgroup of 4 waves per (head, 128-column quarter, 32-row
// batch tile); wave w takes the content features d in [32w, 32w+32) (two
// k-steps of v_mfma_f32_32x32x16_bf16 with M = batch rows, N = latent
// columns) and issues all of its loads before the first multiply. The
// contraction runs along W's row axis (its stride), so each lane loads 8
// consecutive W rows x 4 consecutive columns (8-byte loads) per k-step and
// transposes that 8x4 block in registers into the B operands of four
// N-tiles; tile j's column n is latent column 4n + j, which makes each
// lane's four accumulators four adjacent output columns. The four partial
// sums meet in LDS and wave 0 stores 8-byte rows.
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
  __shared__ __attribute__((aligned(16))) floatx4 red[3][4][4][64];  // waves 1..3 partials
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int nbt = (B + 31) >> 5;
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; when the
  // heads split evenly, XCD x takes every workgroup of heads h = x (mod 8),
  // so the four quarters of each weight row are fetched by one XCD.
  int L = blockIdx.x;
  if ((n_h & 7) == 0) L = (L >> 3) + (L & 7) * (static_cast<int>(gridDim.x) >> 3);
  const int bt = L % nbt;
  const int cq = (L / nbt) & 3;
  const int hh = L / (nbt * 4);  // head index in XCD-grouped order
  const int h = (n_h & 7) == 0 ? (hh % (n_h >> 3)) * 8 + hh / (n_h >> 3) : hh;
  // rows past B load row B-1 (unconditional loads keep all of them in
  // flight); their results are never stored
  const int b = min(bt * 32 + n, B - 1);  // this lane's A-operand row
  const int col0 = cq * 128 + 4 * n;
  const uint16_t* wh = w + static_cast<int64_t>(h) * ROWS_PER_HEAD * D_C + col0;
  const uint16_t* qrow = q_nope + (static_cast<int64_t>(b) * n_h + h) * D_N;

  // all loads of this wave up front: 2 k-steps x (A: 16 bytes, B: 8 rows x 8 bytes)
  u32x4 a[2];
  u32x2 e[2][8];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int d0 = wave * 32 + k * 16 + g * 8;
    a[k] = ld16(qrow + d0);
#pragma unroll
    for (int i = 0; i < 8; i++)
      e[k][i] = *reinterpret_cast<const u32x2*>(wh + static_cast<int64_t>(d0 + i) * D_C);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load issued before the first wait
  floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = floatx16{};
#pragma unroll
  for (int k = 0; k < 2; k++) {
    // e[k][i] holds W[d0+i][col0 .. col0+3]; operand j needs W[d0..d0+7][col0+j]
    u32x4 bj[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      bj[0][r] = lo_lo(e[k][2 * r][0], e[k][2 * r + 1][0]);
      bj[1][r] = hi_hi(e[k][2 * r][0], e[k][2 * r + 1][0]);
      bj[2][r] = lo_lo(e[k][2 * r][1], e[k][2 * r + 1][1]);
      bj[3][r] = hi_hi(e[k][2 * r][1], e[k][2 * r + 1][1]);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] = mfma32x32x16(as_bf16x8(a[k]), as_bf16x8(bj[j]), acc[j]);
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++)
        red[wave - 1][j][q4][lane] = floatx4{acc[j][4 * q4], acc[j][4 * q4 + 1],
                                             acc[j][4 * q4 + 2], acc[j][4 * q4 + 3]};
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int wv = 0; wv < 3; wv++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const floatx4 v = red[wv][j][q4][lane];
        acc[j][4 * q4] += v[0];
        acc[j][4 * q4 + 1] += v[1];
        acc[j][4 * q4 + 2] += v[2];
        acc[j][4 * q4 + 3] += v[3];
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
    const int blocks = n_h * 4 * ((B + 31) / 32);
    hipLaunchKernelGGL(absorb_q_bf16_kernel, dim3(blocks), dim3(256), 0, stream,
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
