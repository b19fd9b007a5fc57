// absorb.hip — fold W^UK into each head's content query.
//
// Operation ("DeepSeek-V3.2-Exp · Absorb key weights", equation and decode
// excerpt; "KV Reconstruction", How it works, first absorb identity):
//   q_lat[b,h,c] = sum_{d<128} q_nope[b,h,d] * wkv_b[h*256 + d, c]
//
// Per head this is a [B x 128] x [128 x 512] product; the 16 MiB of W^UK
// (n_h = 128, bf16) dominates the bytes.
//
// bf16 path: one workgroup of 4 waves per (head, 128-column quarter). The
// workgroup's 128 x 128 block of W^UK (32 KB) is staged into LDS with
// 16-byte LDS-DMA loads (whole 256-byte row segments) and read back
// transposed with ds_read_b64_tr_b16, so W is fetched once, in full lines,
// whatever the batch size. Wave w owns latent columns 32w..32w+31 of the
// quarter and computes the transposed product
//   q_lat^T[32 columns x 32 rows] = W^T[columns x d] . q_nope^T[d x rows]
// (8 k-steps of v_mfma_f32_32x32x16_bf16 per 32-row batch tile; A = W^T from
// LDS, held in registers across batch tiles; B = the batch tile's q_nope
// rows, staged once per workgroup into LDS by LDS-DMA (the four waves read
// the same rows: staged once, the workgroup fetches 8 KB per tile instead of
// 32 KB), double-buffered across batch tiles). The column order tau makes
// accumulator r of lane half g column 16g + r, so every lane stores 32
// contiguous bytes. LDS rows of W are XOR-swizzled by 4 * (row mod 4)
// chunks, rows of q_nope by (row mod 16) chunks, which keeps both kinds of
// reads free of bank conflicts.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int AB_ROW_BYTES = 256;                  // 128 columns of bf16
constexpr int AB_BYTES = D_N * AB_ROW_BYTES;       // 32 KiB staged block
constexpr int AB_DMA = AB_BYTES / 1024 / 4;        // 8 wave-DMAs per wave

__device__ __forceinline__ int ab_tau(int beta) { return 4 * (beta & 1) + (beta >> 1); }

typedef __attribute__((address_space(3))) shortx4 ab_lds_shortx4;

__device__ __forceinline__ bf16x8 ab_tr_pair(const char* lo, const char* hi) {
  const shortx4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ab_lds_shortx4*)(lo));
  const shortx4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ab_lds_shortx4*)(hi));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

// swz_sq = 0: q_lat rows [B, n_h, 512]. swz_sq = s_q > 0: the decode's
// operand order for B / s_q sequences of s_q * n_h query rows (row j * n_h + h
// of sequence b is batch row b * s_q + j, head h): 16-byte slot
// ((((b * HG + hg) * 4 + hq) * 32 + ks) * 64 + g * 32 + (v & 31)) holds
// features 16ks + 8g of query row v = hg * 128 + hq * 32 + (v & 31),
// HG = s_q * n_h / 128.
__global__ __launch_bounds__(256) void absorb_q_bf16_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ q_lat, int B,
                                                            int n_h, int swz_sq) {
  __shared__ __attribute__((aligned(16))) char wl[AB_BYTES];
  __shared__ __attribute__((aligned(16))) char qt[2][32 * D_N * 2];  // q_nope batch tiles
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; when the
  // heads split evenly, XCD x takes the workgroups of heads
  // [x * n_h/8, (x+1) * n_h/8): the query rows of eight consecutive heads,
  // which share 128-byte lines in the operand-order output, are then written
  // through one L2 and leave it as whole lines.
  int L = blockIdx.x;
  if ((n_h & 7) == 0) L = (L >> 3) + (L & 7) * (static_cast<int>(gridDim.x) >> 3);
  const int cq = L & 3;
  const int h = L >> 2;

  // stage W^UK[h][0..127][128cq .. 128cq+127]: slot q of the block is row
  // q/16, chunk position q%16, holding global chunk position ^ 4*(row%4)
  {
    const i32x4 rs = make_rsrc(w + static_cast<int64_t>(h) * ROWS_PER_HEAD * D_C + cq * 128);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(wl));
#pragma unroll
    for (int j = 0; j < AB_DMA; j++) {
      const int q = (wave + 4 * j) * 64 + lane;
      const int r = q >> 4, pos = q & 15;
      const int c = pos ^ (4 * (r & 3));
      dma16(rs, dst + (wave + 4 * j) * 1024, static_cast<uint32_t>(r * D_C * 2 + c * 16), 0);
    }
  }
  // q_nope rows of batch tile bt into qt[bt & 1] (rows past B re-read row
  // B-1): LDS chunk p of row r holds the row's 16-byte chunk p ^ (r mod 16);
  // 1 KB block j = wave + 4k, k = 0, 1, of the 8 KB tile per DMA
  const int nbt = (B + 31) >> 5;
  const uint32_t qt_addr = __builtin_amdgcn_readfirstlane(lds_addr(qt));
  auto stage_q = [&](int bt) {
    const i32x4 rs = make_rsrc(q_nope + (static_cast<int64_t>(bt) * 32 * n_h + h) * D_N);
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int j = wave + 4 * k;
      const int pch = j * 64 + lane;
      const int r = pch >> 4, c = (pch & 15) ^ (r & 15);
      const int rr = min(bt * 32 + r, B - 1) - bt * 32;  // row within the tile's base
      dma16(rs, qt_addr + (bt & 1) * (32 * D_N * 2) + j * 1024,
            static_cast<uint32_t>(rr * n_h * (D_N * 2) + c * 16), 0);
    }
  };
  stage_q(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // A operands: W^T rows = columns 32*wave + 4*tau(4a + (jj>>2)) + (jj&3),
  // k = d rows 16ks + 8g + 0..7 (lo: +0..3, hi: +4..7)
  bf16x8 A[8];
  {
    const int jj = lane & 15, a = (lane >> 4) & 1;
    const int tau = ab_tau(4 * a + (jj & 3));
    const int r = 8 * g + (jj >> 2);
    const int off = r * AB_ROW_BYTES + 16 * ((4 * wave + (tau >> 1)) ^ (4 * (jj >> 2))) +
                    8 * (tau & 1);
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
      const char* lo = wl + off + 16 * ks * AB_ROW_BYTES;
      A[ks] = ab_tr_pair(lo, lo + 4 * AB_ROW_BYTES);
    }
  }
  const int col = cq * 128 + 32 * wave + 16 * g;  // first of this lane's 16 output columns
  for (int bt = 0; bt < nbt; bt++) {
    // the next tile's rows are staged into the other buffer (free: every
    // wave passed the barrier after reading it) while this one multiplies
    if (bt + 1 < nbt) stage_q(bt + 1);
    u32x4 qv[8];
    {
      const char* qrow = qt[bt & 1] + n * (D_N * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ks++) qv[ks] = ld_lds16(qrow + 16 * ((2 * ks + g) ^ (n & 15)));
    }
    floatx16 acc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) acc = mfma32x32x16(A[ks], as_bf16x8(qv[ks]), acc);
    const int b = bt * 32 + n;
    if (b < B) {
      u32x4 v0, v1;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v0[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        v1[i] = pack_bf16x2(acc[8 + 2 * i], acc[8 + 2 * i + 1]);
      }
      if (swz_sq == 0) {
        uint16_t* dst = q_lat + (static_cast<int64_t>(b) * n_h + h) * D_C + col;
        st16(dst, v0);
        st16(dst + 8, v1);
      } else {
        // the lane's 16 columns are k-step col/16, both lane halves
        const int seq = b / swz_sq;
        const int v = (b - seq * swz_sq) * n_h + h;
        const int hgs = swz_sq * n_h >> 7;
        uint16_t* dst = q_lat + ((((static_cast<int64_t>(seq) * hgs + (v >> 7)) * 4 +
                                   ((v >> 5) & 3)) * 32 + (col >> 4)) * 64 + (v & 31)) * 8;
        st16(dst, v0);
        st16(dst + 32 * 8, v1);
      }
    }
    if (bt + 1 < nbt) {
      // the next tile landed (the wait also covers this tile's stores)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
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
    const int blocks = n_h * 4;
    hipLaunchKernelGGL(absorb_q_bf16_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(wkv_b),
                       static_cast<uint16_t*>(q_lat), B, n_h, 0);
  } else {
    hipLaunchKernelGGL(absorb_q_f32_kernel, dim3(static_cast<unsigned>(B) * n_h * 2), dim3(256), 0,
                       stream, static_cast<const float*>(q_nope),
                       static_cast<const float*>(wkv_b), static_cast<float*>(q_lat), n_h);
  }
  return hipGetLastError();
}

hipError_t launch_absorb_q_swizzled(const void* q_nope, const void* wkv_b, void* q_lat, int B,
                                    int n_h, int s_q, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_bf16_kernel, dim3(n_h * 4), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(wkv_b),
                     static_cast<uint16_t*>(q_lat), B, n_h, s_q);
  return hipGetLastError();
}

}  // namespace mla
