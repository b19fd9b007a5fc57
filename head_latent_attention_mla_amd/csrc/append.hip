// append.hip — writes a new token's entries into the compressed cache.
//
// Operation ("DeepSeek-V3.2-Exp · Key–value latent", section "Key–value
// down-projection": the joint down-projection output is split into the
// 512-feature latent and the 64-feature rotary key, the latent is normalised
// and the key rotated; section "Key–value latent RMSNorm": float32
// arithmetic, mean of squares, x * rsqrt(mean + eps), per-feature gain, one
// cast back to the storage type; "DeepSeek V3" inference notes, "Decoupled
// RoPE": the rotated key is cached once per token and shared by all heads):
//   latent[s,p,c] = cast( gamma[c] * (x[c] * rsqrt(mean_c x^2 + eps)) )
//   rope[s,p,2i]   = cast( k[2i] cos_i - k[2i+1] sin_i )
//   rope[s,p,2i+1] = cast( k[2i] sin_i + k[2i+1] cos_i )
// with (cos_i, sin_i) = freqs[p][i] and (s, p) = (seq_idx[n], pos[n]).
//
// HBM-bound: per row 576 elements in, 576 out, plus 256 B of the rotation
// table. A wave handles a few rows, one row across its 64 lanes at a time.
// For bf16 each lane reads 8 latent features of a row (one 16-byte load; the
// wave covers the 1 KB row in one instruction); for fp32
// two 16-byte loads 1 KB apart keep every instruction contiguous across the
// wave. The sum of squares is reduced across the wave with lane shuffles.
// Lanes 0..15 each also rotate two pairs of the rotary key.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

#ifndef MLA_APPEND_WAVES
#define MLA_APPEND_WAVES 4
#endif
#ifndef MLA_APPEND_ROWS
#define MLA_APPEND_ROWS 1
#endif
constexpr int APPEND_WAVES = MLA_APPEND_WAVES;  // waves per workgroup
constexpr int APPEND_ROWS = MLA_APPEND_ROWS;    // rows per wave

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// 8 latent features of this lane: bf16 at feature 8*lane; fp32 at features
// 4*lane + {0..3} and 256 + 4*lane + {0..3}.
template <bool BF16>
__device__ __forceinline__ int lat_feature(int lane, int k) {
  return BF16 ? 8 * lane + k : (k < 4 ? 4 * lane + k : 256 + 4 * lane + (k - 4));
}

template <bool BF16>
__device__ __forceinline__ void load_lat(const void* row, int lane, float x[8]) {
  if constexpr (BF16) {
    const u32x4 v = ld16(static_cast<const uint16_t*>(row) + 8 * lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(v[k] << 16);
      x[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
    }
  } else {
    const float* r = static_cast<const float*>(row);
    const floatx4 a = *reinterpret_cast<const floatx4*>(r + 4 * lane);
    const floatx4 b = *reinterpret_cast<const floatx4*>(r + 256 + 4 * lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = b[k];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store_lat(void* row, int lane, const float y[8]) {
  if constexpr (BF16) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
    st16(static_cast<uint16_t*>(row) + 8 * lane, v);
  } else {
    float* r = static_cast<float*>(row);
    *reinterpret_cast<floatx4*>(r + 4 * lane) = floatx4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<floatx4*>(r + 256 + 4 * lane) = floatx4{y[4], y[5], y[6], y[7]};
  }
}

// Each wave handles ROWS consecutive rows, all of their loads issued before
// any arithmetic. One row per wave and four waves per workgroup measured
// fastest on MI355X (within 11% of a plain device copy of the same bytes);
// more rows per wave lower the occupancy more than they add bytes in flight.
template <bool BF16, int ROWS>
__global__ __launch_bounds__(64 * APPEND_WAVES) void cache_append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t n0 =
      (static_cast<int64_t>(blockIdx.x) * APPEND_WAVES + (threadIdx.x >> 6)) * ROWS;
  const int esz = BF16 ? 2 : 4;
  // loads in two rounds: (1) the row indices, the rows themselves and the
  // gains (none depends on another); (2) the rotation-table rows, which need
  // the positions. The loaded vectors are kept raw until both rounds are out.
  u32x4 raw[ROWS][2];  // bf16: raw[r][0] = 8 latent features; fp32: [0], [1] = two halves
  u32x4 kraw[ROWS];    // rotary key: bf16 4 features in .x/.y; fp32 4 floats
  floatx4 cs[ROWS];
  int64_t dst_lat[ROWS], dst_rope[ROWS];
  bool ok[ROWS];
  int tpos[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int64_t n = n0 + r;
    const bool in = n < p.N;
    const int s = !in ? -1 : (p.seq_idx ? p.seq_idx[n] : static_cast<int>(n));
    const int t = in ? p.pos[n] : -1;
    tpos[r] = t;
    // rows addressed outside the cache or the rotation table are not written
    ok[r] = in && s >= 0 && s < p.B_cache && t >= 0 && t < p.T_cache && t < p.n_pos;
    dst_lat[r] = s * p.lat_bs + t * p.lat_rs;
    dst_rope[r] = s * p.rope_bs + t * p.rope_rs;
    // the row itself depends only on n: its loads go out with the index loads
    const int64_t nn = in ? n : 0;
    const char* src = static_cast<const char*>(p.kv_a) + nn * p.in_rstride * esz;
    if constexpr (BF16) {
      raw[r][0] = ld16(static_cast<const uint16_t*>(static_cast<const void*>(src)) + 8 * lane);
      raw[r][1] = raw[r][0];
    } else {
      raw[r][0] = ld16(reinterpret_cast<const float*>(src) + 4 * lane);
      raw[r][1] = ld16(reinterpret_cast<const float*>(src) + 256 + 4 * lane);
    }
    kraw[r] = u32x4{0u, 0u, 0u, 0u};
    if (lane < D_R / 4) {  // 16 lanes x 4 rotary features (2 pairs)
      if constexpr (BF16) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(
            reinterpret_cast<const uint16_t*>(src) + D_C + 4 * lane);
        kraw[r] = u32x4{v[0], v[1], 0u, 0u};
      } else {
        kraw[r] = ld16(reinterpret_cast<const float*>(src) + D_C + 4 * lane);
      }
    }
  }
  float g[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) g[k] = p.gamma[lat_feature<BF16>(lane, k)];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    // (cos, sin) of pairs 2*lane and 2*lane + 1
    cs[r] = floatx4{1.f, 0.f, 1.f, 0.f};
    if (ok[r] && lane < D_R / 4)
      cs[r] = *reinterpret_cast<const floatx4*>(p.freqs + static_cast<int64_t>(tpos[r]) * D_R +
                                                4 * lane);
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (!ok[r]) continue;
    float x[8];
    if constexpr (BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(raw[r][0][k] << 16);
        x[2 * k + 1] = __uint_as_float(raw[r][0][k] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = __uint_as_float(raw[r][0][k]);
        x[4 + k] = __uint_as_float(raw[r][1][k]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += x[k] * x[k];
    ss = wave_sum(ss);
    // 1/512 is a power of two: the mean is exact in fp32
    const float inv = rsqrtf(ss * (1.0f / D_C) + p.eps);
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = g[k] * (x[k] * inv);
    store_lat<BF16>(static_cast<char*>(p.latent) + dst_lat[r] * esz, lane, y);
    if (lane < D_R / 4) {
      float kk[4];
      if constexpr (BF16) {
        kk[0] = __uint_as_float(kraw[r][0] << 16);
        kk[1] = __uint_as_float(kraw[r][0] & 0xFFFF0000u);
        kk[2] = __uint_as_float(kraw[r][1] << 16);
        kk[3] = __uint_as_float(kraw[r][1] & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) kk[k] = __uint_as_float(kraw[r][k]);
      }
      const floatx4 c = cs[r];
      const float o0 = kk[0] * c[0] - kk[1] * c[1];
      const float o1 = kk[0] * c[1] + kk[1] * c[0];
      const float o2 = kk[2] * c[2] - kk[3] * c[3];
      const float o3 = kk[2] * c[3] + kk[3] * c[2];
      char* rdst = static_cast<char*>(p.rope) + dst_rope[r] * esz;
      if constexpr (BF16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(rdst) + 4 * lane) =
            u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      } else {
        *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(rdst) + 4 * lane) =
            floatx4{o0, o1, o2, o3};
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, bool is_bf16, hipStream_t stream) {
  constexpr int per_block = APPEND_WAVES * APPEND_ROWS;
  const int64_t blocks = (p.N + per_block - 1) / per_block;
  auto kern = is_bf16 ? cache_append_kernel<true, APPEND_ROWS>
                      : cache_append_kernel<false, APPEND_ROWS>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(64 * APPEND_WAVES), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace mla
