// out_up.hip — W^UV applied after the probability-weighted latent sum.
//
// Operation ("KV Reconstruction", How it works, second absorb identity and
// Watch-outs: attend on the latent, then apply W^UV; "Absorb key weights",
// decode excerpt, last einsum; "Value up-projection", Explanation: value rows
// are 128..255 of each head's 256):
//   out[b,h,d] = sum_c out_lat[b,h,c] * wkv_b[h*256 + 128 + d, c]
//
// Per head a [B x 512] x [512 x 128] product bound by streaming the 16 MiB of
// W^UV. Here the contraction runs along W's contiguous axis, so both MFMA
// operands are straight 16-byte loads. One workgroup of 4 waves per (head,
// 32-wide value tile); wave w takes latent features [128w, 128w+128) (8
// k-steps of v_mfma_f32_32x32x16_bf16 with M = batch rows, N = value
// features), keeps its W operands in registers across the 32-row batch
// tiles (W is read once whatever the batch), and issues all loads before
// the first multiply; the four partial sums meet in LDS.
#include "common.hpp"
#include "launch.hpp"
#include "merge.hpp"

namespace mla {

__global__ __launch_bounds__(256) void out_up_bf16_kernel(const uint16_t* __restrict__ o_lat,
                                                          const uint16_t* __restrict__ w,
                                                          uint16_t* __restrict__ out, int B,
                                                          int n_h) {
  __shared__ __attribute__((aligned(16))) floatx4 red[3][4][64];  // waves 1..3 partials
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; when the
  // heads split evenly, XCD x takes every workgroup of heads h = x (mod 8),
  // so the four value tiles of each head are fetched by one XCD.
  int L = blockIdx.x;
  if ((n_h & 7) == 0) L = (L >> 3) + (L & 7) * (static_cast<int>(gridDim.x) >> 3);
  const int dt = L & 3;
  const int hh = L >> 2;  // head index in XCD-grouped order
  const int h = (n_h & 7) == 0 ? (hh % (n_h >> 3)) * 8 + hh / (n_h >> 3) : hh;
  const int d = dt * 32 + n;  // this lane's B-operand column (value feature)
  const uint16_t* wrow =
      w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + D_N + d) * D_C + wave * 128 + g * 8;
  // rows past B load row B-1 (unconditional loads keep all of them in
  // flight); their results are never stored
  auto load_o = [&](int bt, u32x4* a) {
    const int b = min(bt * 32 + n, B - 1);
    const uint16_t* orow = o_lat + (static_cast<int64_t>(b) * n_h + h) * D_C + wave * 128 + g * 8;
#pragma unroll
    for (int k = 0; k < 8; k++) a[k] = ld16(orow + 16 * k);
  };
  // the W^UV operands stay in registers for every batch tile
  u32x4 a[8], bw[8];
  load_o(0, a);
#pragma unroll
  for (int k = 0; k < 8; k++) bw[k] = ld16(wrow + 16 * k);
  __builtin_amdgcn_sched_barrier(0);  // keep every load issued before the first wait
  const int nbt = (B + 31) >> 5;
  for (int bt = 0; bt < nbt; bt++) {
    // next tile's rows into a second register set, issued before the
    // multiplies: a branch between the multiplies and the reads of their
    // accumulators has let an accumulator be read before the MFMA wrote it
    u32x4 an[8];
    if (bt + 1 < nbt) load_o(bt + 1, an);
    floatx16 acc = {};
#pragma unroll
    for (int k = 0; k < 8; k++) acc = mfma32x32x16(as_bf16x8(a[k]), as_bf16x8(bw[k]), acc);
#pragma unroll
    for (int k = 0; k < 8; k++) a[k] = an[k];
    if (bt > 0) __syncthreads();  // wave 0 done reading the previous tile's partials
    if (wave > 0) {
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++)
        red[wave - 1][q4][lane] =
            floatx4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int wv = 0; wv < 3; wv++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const floatx4 v = red[wv][q4][lane];
          acc[4 * q4] += v[0];
          acc[4 * q4 + 1] += v[1];
          acc[4 * q4 + 2] += v[2];
          acc[4 * q4 + 3] += v[3];
        }
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int bo = bt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (bo < B) out[(static_cast<int64_t>(bo) * n_h + h) * D_V + d] = float_to_bf16_bits(acc[r]);
      }
    }
  }
}

// Merge of the decode's split partials fused with W^UV (the one-call decode
// step): one workgroup of 8 waves per (head, 16-row batch tile), so a
// 32-row batch gives two workgroups per head and the chip is filled. The
// waves first merge the tile's rows (wave w: rows w and w+8, both loaded in
// one memory round trip, rows past the batch skipped; lane: 8 latent
// features, the arithmetic of the stand-alone merge) into a bf16 o_lat tile in LDS, then wave (dt, kh)
// multiplies it by value features 32dt..32dt+31 of W^UV over latent half kh
// (two 128-feature quarters; its W operands were loaded before the merge)
// and the partial sums meet in LDS, added in the stand-alone kernel's
// order. The merged rows never go to memory; the result has the bits of
// merge + out-up. The MFMA tile has 32 rows: rows 16..31 repeat 0..15 and
// are not stored. LDS rows are XOR-swizzled by (row mod 16) chunks so the
// 16 rows of an operand read hit distinct banks.
// With NV = 2 (a batch of at most 16 rows and fewer than 256 (head, tile)
// workgroups) the value features are split between two workgroups, so the
// whole chip streams W^UV and the partials (the second workgroup's partial
// rows come from L2): wave (dt, kq) then multiplies one 128-feature quarter
// kq for value block dt, and the quarter sums meet in LDS in the same order.
constexpr int MO_ROWS = 16;
template <int NV>
__global__ __launch_bounds__(512) void merge_out_up_bf16_kernel(
    const uint16_t* __restrict__ ws_o, const float* __restrict__ ws_lse, int S,
    const uint16_t* __restrict__ w, uint16_t* __restrict__ out, float* __restrict__ lse, int B,
    int n_h) {
  __shared__ __attribute__((aligned(16))) char ol[MO_ROWS * D_C * 2];   // merged rows
  __shared__ __attribute__((aligned(16))) floatx4 red[16][64];  // quarter sums of the other waves
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int nbt = (B + MO_ROWS - 1) / MO_ROWS;
  // the batch tiles of eight consecutive heads share an XCD (as in out-up)
  int L = blockIdx.x;
  const int G = gridDim.x;
  if ((n_h & 7) == 0) L = (L >> 3) + (L & 7) * (G >> 3);
  const int vp = L % NV;  // value part (the parts of a (head, tile) are adjacent)
  const int bt = (L / NV) % nbt;
  const int hh = L / (NV * nbt);
  const int h = (n_h & 7) == 0 ? (hh % (n_h >> 3)) * 8 + hh / (n_h >> 3) : hh;
  // NV = 1: wave (dt, kh) takes quarters 2kh, 2kh+1; NV = 2: wave (dt, kq)
  // quarter kq, value blocks 2vp, 2vp+1
  constexpr int NQ = 2 / NV;               // quarters per wave
  const int dt = NV == 1 ? (wave & 3) : 2 * vp + (wave & 1);
  const int q0 = NV == 1 ? 2 * (wave >> 2) : (wave >> 1);  // first quarter of this wave
  const int d = dt * 32 + n;

  u32x4 bw[8 * NQ];
  {
    const uint16_t* wrow =
        w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + D_N + d) * D_C + q0 * 128 + g * 8;
#pragma unroll
    for (int k = 0; k < 8 * NQ; k++) bw[k] = ld16(wrow + 16 * k);
  }
  const int64_t BH = static_cast<int64_t>(B) * n_h;
  if (S > MERGE_SPLIT_PARTS_ABOVE && B - bt * MO_ROWS <= 4) {
    // at most 4 rows of many splits: wave (part, r) folds part `part` of row
    // r, the part-1 states meet part 0 through `red` (free until the quarter
    // sums); the arithmetic of merge_rows8 for such rows, so the same bits.
    // Waves 0..3 write merged rows 0..3 of the tile, every other row is zeros.
    const int part = wave >> 2, r = wave & 3;
    const int bb = bt * MO_ROWS + r;
    const bool ok = bb < B;
    const int64_t bhr = static_cast<int64_t>(bb) * n_h + h;
    float mx = -INFINITY, wsum = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
    if (ok)
      merge_chunks<true, NV == 2 ? 4 : 2>(ws_o, ws_lse, S, BH, bhr, lane * 8,
                                          merge_part_begin(S, part), merge_part_end(S, part),
                                          mx, wsum, acc);
    float* const xs = reinterpret_cast<float*>(red);  // [4 rows][10][64]
    if (part == 1) {
      xs[(r * 10 + 0) * 64 + lane] = mx;
      xs[(r * 10 + 1) * 64 + lane] = wsum;
#pragma unroll
      for (int i = 0; i < 8; i++) xs[(r * 10 + 2 + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    u32x4 o = u32x4{0u, 0u, 0u, 0u};
    if (part == 0 && ok) {
      float a1[8], o8[8];
#pragma unroll
      for (int i = 0; i < 8; i++) a1[i] = xs[(r * 10 + 2 + i) * 64 + lane];
      merge_combine2(mx, wsum, acc, xs[(r * 10 + 0) * 64 + lane], xs[(r * 10 + 1) * 64 + lane],
                     a1);
      const float l = merge_finish(mx, wsum, acc, o8);
#pragma unroll
      for (int q = 0; q < 4; q++) o[q] = pack_bf16x2(o8[2 * q], o8[2 * q + 1]);
      if (lane == 0 && lse) lse[bhr] = l;
    }
    // rows `wave` (merged for waves 0..3) and wave + 8 (zeros)
    *reinterpret_cast<u32x4*>(ol + wave * (D_C * 2) + 16 * (lane ^ wave)) = o;
    *reinterpret_cast<u32x4*>(ol + (wave + 8) * (D_C * 2) + 16 * (lane ^ (wave + 8))) =
        u32x4{0u, 0u, 0u, 0u};
  } else {
    // rows wave and wave + 8 of the tile; rows past B are zeros in LDS (their
    // products are never stored)
    const int r0 = wave, r1 = wave + 8;
    const int b0 = bt * MO_ROWS + r0, b1 = bt * MO_ROWS + r1;
    float o8[2][8], l[2];
    int64_t bh[2] = {static_cast<int64_t>(b0) * n_h + h, static_cast<int64_t>(b1) * n_h + h};
    int nrows = 0;
    if (b1 < B) {
      merge_rows8<2, true>(ws_o, ws_lse, S, BH, bh, lane * 8, o8, l);
      nrows = 2;
    } else if (b0 < B) {
      merge_rows8<1, true>(ws_o, ws_lse, S, BH, bh, lane * 8, o8, l);
      nrows = 1;
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int r = wave + 8 * i;
      u32x4 o = u32x4{0u, 0u, 0u, 0u};
      if (i < nrows) {
#pragma unroll
        for (int q = 0; q < 4; q++) o[q] = pack_bf16x2(o8[i][2 * q], o8[i][2 * q + 1]);
        if (lane == 0 && lse) lse[bh[i]] = l[i];
      }
      *reinterpret_cast<u32x4*>(ol + r * (D_C * 2) + 16 * (lane ^ r)) = o;
    }
  }
  __syncthreads();
  // each quarter is one 8-k-step chain from zero; the quarters are summed in
  // the order the stand-alone W^UV kernel uses ((q0 + q1) + q2) + q3, so
  // both paths give the same bits
  floatx16 acc[NQ];
#pragma unroll
  for (int qq = 0; qq < NQ; qq++) acc[qq] = floatx16{};
  {
    const int r = n & 15;
    const char* arow = ol + r * (D_C * 2);
#pragma unroll
    for (int k = 0; k < 8 * NQ; k++) {
      const int c = q0 * 16 + 2 * k + g;
      const u32x4 a = ld_lds16(arow + 16 * (c ^ r));
      acc[k >> 3] = mfma32x32x16(as_bf16x8(a), as_bf16x8(bw[k]), acc[k >> 3]);
    }
  }
  // accumulators 0..7 of lane half g hold rows 8*(r/4) + 4g + r%4 < 16;
  // the quarters the first waves (those holding quarter 0) do not hold meet
  // in red: NV = 1 quarters 2, 3 of value block dt; NV = 2 quarters 1..3 of
  // block dt & 1 (two float4 per lane each)
  auto slot = [&](int q, int q4) {
    return NV == 1 ? ((q - 2) * 4 + dt) * 2 + q4 : ((q - 1) * 2 + (dt & 1)) * 2 + q4;
  };
  const bool first = q0 == 0;
  if (!first) {
#pragma unroll
    for (int qq = 0; qq < NQ; qq++)
#pragma unroll
      for (int q4 = 0; q4 < 2; q4++)
        red[slot(q0 + qq, q4)][lane] = floatx4{acc[qq][4 * q4], acc[qq][4 * q4 + 1],
                                                     acc[qq][4 * q4 + 2], acc[qq][4 * q4 + 3]};
  }
  __syncthreads();
  if (first) {
    float sum[8];
#pragma unroll
    for (int i = 0; i < 8; i++) sum[i] = NQ == 2 ? acc[0][i] + acc[NQ - 1][i] : acc[0][i];
#pragma unroll
    for (int q = NQ; q < 4; q++)
#pragma unroll
      for (int q4 = 0; q4 < 2; q4++) {
        const floatx4 v = red[slot(q, q4)][lane];
        sum[4 * q4] += v[0];
        sum[4 * q4 + 1] += v[1];
        sum[4 * q4 + 2] += v[2];
        sum[4 * q4 + 3] += v[3];
      }
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int bo = bt * MO_ROWS + 8 * (r >> 2) + 4 * g + (r & 3);
      if (bo < B) out[(static_cast<int64_t>(bo) * n_h + h) * D_V + d] = float_to_bf16_bits(sum[r]);
    }
  }
}

hipError_t launch_merge_out_up(const void* ws_o, const float* ws_lse, int S, const void* wkv_b,
                               void* out, float* lse, int B, int n_h, hipStream_t stream) {
  const int tiles = n_h * ((B + MO_ROWS - 1) / MO_ROWS);
  if (tiles < 256 && (n_h & 7) == 0)
    hipLaunchKernelGGL(merge_out_up_bf16_kernel<2>, dim3(2 * tiles), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(ws_o), ws_lse, S,
                       static_cast<const uint16_t*>(wkv_b), static_cast<uint16_t*>(out), lse, B,
                       n_h);
  else
    hipLaunchKernelGGL(merge_out_up_bf16_kernel<1>, dim3(tiles), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(ws_o), ws_lse, S,
                       static_cast<const uint16_t*>(wkv_b), static_cast<uint16_t*>(out), lse, B,
                       n_h);
  return hipGetLastError();
}

// fp32: one block per (b, h); thread d walks its W^UV row.
__global__ __launch_bounds__(128) void out_up_f32_kernel(const float* __restrict__ o_lat,
                                                         const float* __restrict__ w,
                                                         float* __restrict__ out, int n_h) {
  __shared__ float o[D_C];
  const int bh = blockIdx.x;
  const int h = bh % n_h;
  for (int c = threadIdx.x; c < D_C; c += 128) o[c] = o_lat[static_cast<int64_t>(bh) * D_C + c];
  __syncthreads();
  const int d = threadIdx.x;
  const float* wrow = w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + D_N + d) * D_C;
  float acc = 0.f;
  for (int c = 0; c < D_C; c++) acc = fmaf(o[c], wrow[c], acc);
  out[static_cast<int64_t>(bh) * D_V + d] = acc;
}

hipError_t launch_out_up(const void* o_lat, const void* wkv_b, void* out, int B, int n_h,
                         bool is_bf16, hipStream_t stream) {
  if (is_bf16) {
    const int blocks = n_h * 4;
    hipLaunchKernelGGL(out_up_bf16_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(o_lat), static_cast<const uint16_t*>(wkv_b),
                       static_cast<uint16_t*>(out), B, n_h);
  } else {
    hipLaunchKernelGGL(out_up_f32_kernel, dim3(static_cast<unsigned>(B) * n_h), dim3(128), 0,
                       stream, static_cast<const float*>(o_lat), static_cast<const float*>(wkv_b),
                       static_cast<float*>(out), n_h);
  }
  return hipGetLastError();
}

}  // namespace mla
