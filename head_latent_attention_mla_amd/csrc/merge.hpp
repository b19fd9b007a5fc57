// merge.hpp — combination of split partials of the decode (one softmax over
// all positions, computed per split): with per-split normalised outputs O_s
// and log-sum-exps lse_s,
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
// Shared by the stand-alone merge kernel and the merge fused into W^UV, so
// both produce the same bits.
#pragma once
#include "common.hpp"

namespace mla {

constexpr int MERGE_CHUNK = 8;  // splits per memory round trip

// One chunk of MERGE_CHUNK splits (s0 .. s0+7; log-sum-exps lv, partials v:
// 8 consecutive bf16 features) folded into the running state (mx, wsum,
// acc) of one row: the running maximum absorbs the chunk's, state and new
// terms are weighted by exp(lse - max). Entries past the last split (their
// indices were clamped by the caller) weigh zero; while no split has seen a
// position (cm = -inf: every index outside [0, T)) nothing is added.
__device__ __forceinline__ void merge_fold8(const float (&lv)[MERGE_CHUNK],
                                            const u32x4 (&v)[MERGE_CHUNK], int s0, int S,
                                            float& mx, float& wsum, float (&acc)[8]) {
  // no contraction beyond the explicit fmaf: the same bits in every caller
#pragma clang fp contract(off)
  float cm = mx;
#pragma unroll
  for (int j = 0; j < MERGE_CHUNK; j++) cm = fmaxf(cm, lv[j]);
  // f is 0 on the first chunk (mx = -inf)
  const float f = cm != -INFINITY ? __expf(mx - cm) : 1.f;
  wsum *= f;
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] *= f;
  mx = cm;
#pragma unroll
  for (int j = 0; j < MERGE_CHUNK; j++) {
    const float w = s0 + j < S && cm != -INFINITY ? __expf(lv[j] - mx) : 0.f;
    wsum += w;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      acc[2 * i] = fmaf(w, __uint_as_float(v[j][i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(w, __uint_as_float(v[j][i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
  }
}

// The merged values (fp32, before rounding) and the row's log-sum-exp from
// the state after the last chunk; a row whose splits all saw no position
// merges to zero with lse -inf (the empty sum).
__device__ __forceinline__ float merge_finish(float mx, float wsum, const float (&acc)[8],
                                              float (&out)[8]) {
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = acc[i] * inv;
  return mx + logf(wsum);
}

// Rows of more than MERGE_SPLIT_PARTS_ABOVE splits are merged in two parts:
// part 0 folds chunks [0, h), part 1 chunks [h, nch) (nch chunks of
// MERGE_CHUNK splits, h = ceil(nch / 2)), each from an empty state, and the
// two states are combined by merge_combine2. A caller may give the parts to
// two waves (few rows of many splits: long positions over a small batch) or
// run both in one wave; the arithmetic, and so the bits, are the same.
constexpr int MERGE_SPLIT_PARTS_ABOVE = 4 * MERGE_CHUNK;

__device__ __forceinline__ int merge_part_begin(int S, int part) {
  const int nch = (S + MERGE_CHUNK - 1) / MERGE_CHUNK;
  return part == 0 ? 0 : (nch + 1) / 2;
}
__device__ __forceinline__ int merge_part_end(int S, int part) {
  const int nch = (S + MERGE_CHUNK - 1) / MERGE_CHUNK;
  return part == 0 ? (nch + 1) / 2 : nch;
}

// Chunks [cb, ce) of one row folded in order from the state (mx, wsum, acc)
// with AHEAD chunks of loads in flight: chunk c + AHEAD is loaded right
// after chunk c is folded, so the result has the bits of one chunk per
// memory round trip (AHEAD only trades registers for round trips). NT:
// non-temporal partial loads.
template <bool NT, int AHEAD = 4>
__device__ __forceinline__ void merge_chunks(const uint16_t* __restrict__ ws_o,
                                             const float* __restrict__ ws_lse, int S, int64_t BH,
                                             int64_t bh, int c0, int cb, int ce, float& mx,
                                             float& wsum, float (&acc)[8]) {
  constexpr int MERGE_AHEAD = AHEAD;
  u32x4 v[MERGE_AHEAD][MERGE_CHUNK];
  float lv[MERGE_AHEAD][MERGE_CHUNK];
  auto load = [&](int c, float (&l)[MERGE_CHUNK], u32x4 (&x)[MERGE_CHUNK]) {
#pragma unroll
    for (int j = 0; j < MERGE_CHUNK; j++) {
      const int64_t sj = min(c * MERGE_CHUNK + j, S - 1);
      l[j] = ws_lse[sj * BH + bh];
      const uint16_t* src = ws_o + (sj * BH + bh) * D_C + c0;
      x[j] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)) : ld16(src);
    }
  };
#pragma unroll
  for (int k = 0; k < MERGE_AHEAD; k++)
    if (cb + k < ce) load(cb + k, lv[k], v[k]);
  for (int c = cb; c < ce; c += MERGE_AHEAD) {
#pragma unroll
    for (int k = 0; k < MERGE_AHEAD; k++) {
      if (c + k < ce) {
        merge_fold8(lv[k], v[k], (c + k) * MERGE_CHUNK, S, mx, wsum, acc);
        if (c + k + MERGE_AHEAD < ce) load(c + k + MERGE_AHEAD, lv[k], v[k]);
      }
    }
  }
}

// The state of part 1 (mx1, wsum1, acc1) combined into that of part 0: both
// weighted by exp(mx_k - max); a part that saw no position (mx = -inf, zero
// sums) adds nothing, and two such parts leave the empty state.
__device__ __forceinline__ void merge_combine2(float& mx, float& wsum, float (&acc)[8], float mx1,
                                               float wsum1, const float (&acc1)[8]) {
  // no contraction beyond the explicit fmaf: the same bits in every caller
#pragma clang fp contract(off)
  const float M = fmaxf(mx, mx1);
  const float f0 = M != -INFINITY ? __expf(mx - M) : 1.f;
  const float f1 = M != -INFINITY ? __expf(mx1 - M) : 1.f;
  wsum = fmaf(wsum1, f1, wsum * f0);
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = fmaf(acc1[i], f1, acc[i] * f0);
  mx = M;
}

// 8 consecutive latent features (c0..c0+7) of NR query rows bh[0..NR-1]:
// partials are [S][BH][512] bf16, lse [S][BH] fp32. Splits are taken
// MERGE_CHUNK at a time; a chunk's log-sum-exps and partials of all NR rows
// are loaded together (one memory round trip per chunk, or for one row of 9
// to 16 splits both chunks in one round trip; indices past the last split
// are clamped) and folded in with merge_fold8; rows of more than
// MERGE_SPLIT_PARTS_ABOVE splits are merged in two parts (both here, one
// after the other). The arithmetic of a row does not depend on NR or on how
// its chunks were loaded. NT: the partials are read non-temporally (each is
// read once; the split kernels write them non-temporally too). Measured:
// 25 -> 22 us per sparse top-2048 attention call with the stand-alone merge,
// ~0.8 us per B=32 T=4096 step with the merge fused into W^UV.
template <int NR, bool NT = false>
__device__ __forceinline__ void merge_rows8(const uint16_t* __restrict__ ws_o,
                                            const float* __restrict__ ws_lse, int S, int64_t BH,
                                            const int64_t* bh, int c0, float out[NR][8],
                                            float* lse) {
  float mx[NR], wsum[NR], acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; r++) {
    mx[r] = -INFINITY;
    wsum[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[r][i] = 0.f;
  }
  auto load = [&](int r, int s0, float (&lv)[MERGE_CHUNK], u32x4 (&v)[MERGE_CHUNK]) {
#pragma unroll
    for (int j = 0; j < MERGE_CHUNK; j++) {
      const int64_t sj = min(s0 + j, S - 1);
      lv[j] = ws_lse[sj * BH + bh[r]];
      const uint16_t* src = ws_o + (sj * BH + bh[r]) * D_C + c0;
      v[j] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)) : ld16(src);
    }
  };
  if (NR == 1 && S > MERGE_CHUNK && S <= 2 * MERGE_CHUNK) {
    // two chunks of one row: both in one memory round trip
    u32x4 v0[MERGE_CHUNK], v1[MERGE_CHUNK];
    float l0[MERGE_CHUNK], l1[MERGE_CHUNK];
    load(0, 0, l0, v0);
    load(0, MERGE_CHUNK, l1, v1);
    merge_fold8(l0, v0, 0, S, mx[0], wsum[0], acc[0]);
    merge_fold8(l1, v1, MERGE_CHUNK, S, mx[0], wsum[0], acc[0]);
  } else if (S > MERGE_SPLIT_PARTS_ABOVE) {
    // (two loads ahead with two rows: the callers of two rows hold other
    // operands in registers)
    constexpr int AH = NR == 1 ? 4 : 2;
#pragma unroll
    for (int r = 0; r < NR; r++) {
      merge_chunks<NT, AH>(ws_o, ws_lse, S, BH, bh[r], c0, merge_part_begin(S, 0),
                           merge_part_end(S, 0), mx[r], wsum[r], acc[r]);
      float mx1 = -INFINITY, wsum1 = 0.f, acc1[8];
#pragma unroll
      for (int i = 0; i < 8; i++) acc1[i] = 0.f;
      merge_chunks<NT, AH>(ws_o, ws_lse, S, BH, bh[r], c0, merge_part_begin(S, 1),
                           merge_part_end(S, 1), mx1, wsum1, acc1);
      merge_combine2(mx[r], wsum[r], acc[r], mx1, wsum1, acc1);
    }
  } else if (NR == 1 && S > 2 * MERGE_CHUNK) {
    merge_chunks<NT>(ws_o, ws_lse, S, BH, bh[0], c0, 0, (S + MERGE_CHUNK - 1) / MERGE_CHUNK,
                     mx[0], wsum[0], acc[0]);
  } else {
    for (int s0 = 0; s0 < S; s0 += MERGE_CHUNK) {
      u32x4 v[NR][MERGE_CHUNK];
      float lv[NR][MERGE_CHUNK];
#pragma unroll
      for (int r = 0; r < NR; r++) load(r, s0, lv[r], v[r]);
#pragma unroll
      for (int r = 0; r < NR; r++) merge_fold8(lv[r], v[r], s0, S, mx[r], wsum[r], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; r++) lse[r] = merge_finish(mx[r], wsum[r], acc[r], out[r]);
}

}  // namespace mla
