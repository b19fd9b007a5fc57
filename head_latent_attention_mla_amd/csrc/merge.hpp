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

// 8 consecutive latent features (c0..c0+7) of NR query rows bh[0..NR-1]:
// partials are [S][BH][512] bf16, lse [S][BH] fp32. Splits are taken
// MERGE_CHUNK at a time; a chunk's log-sum-exps and partials of all NR rows
// are loaded together (one memory round trip per chunk, or for one row of 9
// to 16 splits both chunks in one round trip; indices past the last split
// are clamped) and folded in with merge_fold8. The arithmetic of a row does
// not depend on NR or on how its chunks were loaded. NT: the partials are
// read non-temporally (each is read once; the split kernels write them
// non-temporally too). Measured: 25 -> 22 us per sparse top-2048 attention
// call with the stand-alone merge, ~0.8 us per B=32 T=4096 step with the
// merge fused into W^UV.
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
  } else if (NR == 1 && S > 2 * MERGE_CHUNK) {
    // one row of many splits (long positions over few sequences): MERGE_AHEAD
    // chunks in flight, chunk c + MERGE_AHEAD loaded right after chunk c is
    // folded; the chunks are folded in order, so the result is the bits of
    // one chunk per round trip (measured at B=4 T=32768, 64 splits: the
    // round trips were the merge's time)
    constexpr int MERGE_AHEAD = 4;
    u32x4 v[MERGE_AHEAD][MERGE_CHUNK];
    float lv[MERGE_AHEAD][MERGE_CHUNK];
    const int nch = (S + MERGE_CHUNK - 1) / MERGE_CHUNK;
#pragma unroll
    for (int k = 0; k < MERGE_AHEAD; k++)
      if (k < nch) load(0, k * MERGE_CHUNK, lv[k], v[k]);
    for (int c = 0; c < nch; c += MERGE_AHEAD) {
#pragma unroll
      for (int k = 0; k < MERGE_AHEAD; k++) {
        if (c + k < nch) {
          merge_fold8(lv[k], v[k], (c + k) * MERGE_CHUNK, S, mx[0], wsum[0], acc[0]);
          if (c + k + MERGE_AHEAD < nch)
            load(0, (c + k + MERGE_AHEAD) * MERGE_CHUNK, lv[k], v[k]);
        }
      }
    }
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
