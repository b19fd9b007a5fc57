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

// 8 consecutive latent features (c0..c0+7) of NR query rows bh[0..NR-1]:
// partials are [S][BH][512] bf16, lse [S][BH] fp32. Splits are taken
// MERGE_CHUNK at a time; a chunk's log-sum-exps and partials of all NR rows
// are loaded together (one memory round trip per chunk; indices past the
// last split are clamped and weighted zero) and folded in with a running
// maximum. Returns the merged values (fp32, before rounding) and each row's
// log-sum-exp; a row whose splits all saw no position (lse -inf) merges to
// zero with lse -inf. The arithmetic of a row does not depend on NR.
template <int NR>
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
  for (int s0 = 0; s0 < S; s0 += MERGE_CHUNK) {
    u32x4 v[NR][MERGE_CHUNK];
    float lv[NR][MERGE_CHUNK];
#pragma unroll
    for (int r = 0; r < NR; r++)
#pragma unroll
      for (int j = 0; j < MERGE_CHUNK; j++) {
        const int64_t sj = min(s0 + j, S - 1);
        lv[r][j] = ws_lse[sj * BH + bh[r]];
        v[r][j] = ld16(ws_o + (sj * BH + bh[r]) * D_C + c0);
      }
#pragma unroll
    for (int r = 0; r < NR; r++) {
      float cm = mx[r];
#pragma unroll
      for (int j = 0; j < MERGE_CHUNK; j++) cm = fmaxf(cm, lv[r][j]);
      // f is 0 on the first chunk (mx = -inf); while no split has seen a
      // position (cm = -inf: every index outside [0, T)) nothing is added
      const float f = cm != -INFINITY ? __expf(mx[r] - cm) : 1.f;
      wsum[r] *= f;
#pragma unroll
      for (int i = 0; i < 8; i++) acc[r][i] *= f;
      mx[r] = cm;
#pragma unroll
      for (int j = 0; j < MERGE_CHUNK; j++) {
        const float w = s0 + j < S && cm != -INFINITY ? __expf(lv[r][j] - mx[r]) : 0.f;
        wsum[r] += w;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          acc[r][2 * i] = fmaf(w, __uint_as_float(v[r][j][i] << 16), acc[r][2 * i]);
          acc[r][2 * i + 1] = fmaf(w, __uint_as_float(v[r][j][i] & 0xFFFF0000u), acc[r][2 * i + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; r++) {
    const float inv = wsum[r] > 0.f ? 1.f / wsum[r] : 0.f;  // the empty sum is 0
#pragma unroll
    for (int i = 0; i < 8; i++) out[r][i] = acc[r][i] * inv;
    lse[r] = mx[r] + logf(wsum[r]);
  }
}

}  // namespace mla
