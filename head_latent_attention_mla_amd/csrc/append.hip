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
// table. One wave per row. For bf16 each lane reads 8 latent features (one
// 16-byte load; the wave covers the 1 KB row in one instruction); for fp32
// two 16-byte loads 1 KB apart keep every instruction contiguous across the
// wave. The sum of squares is reduced across the wave with lane shuffles.
// Lanes 0..15 each also rotate two pairs of the rotary key.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int APPEND_ROWS_PER_BLOCK = 4;  // one 64-lane wave per row

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

template <bool BF16>
__global__ __launch_bounds__(64 * APPEND_ROWS_PER_BLOCK) void cache_append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * APPEND_ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (n >= p.N) return;
  const int s = p.seq_idx ? p.seq_idx[n] : static_cast<int>(n);
  const int t = p.pos[n];
  // rows addressed outside the cache or the rotation table are not written
  if (s < 0 || s >= p.B_cache || t < 0 || t >= p.T_cache || t >= p.n_pos) return;
  const int esz = BF16 ? 2 : 4;
  const char* src = static_cast<const char*>(p.kv_a) + n * p.in_rstride * esz;

  float x[8];
  load_lat<BF16>(src, lane, x);
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += x[k] * x[k];
  ss = wave_sum(ss);
  // 1/512 is a power of two: the mean is exact in fp32
  const float inv = rsqrtf(ss * (1.0f / D_C) + p.eps);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = p.gamma[lat_feature<BF16>(lane, k)] * (x[k] * inv);
  char* dst = static_cast<char*>(p.latent) + (s * p.lat_bs + t * p.lat_rs) * esz;
  store_lat<BF16>(dst, lane, y);

  if (lane < D_R / 4) {  // 16 lanes x 4 rotary features (2 pairs)
    float k4[4];
    if constexpr (BF16) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(
          reinterpret_cast<const uint16_t*>(src) + D_C + 4 * lane);
      k4[0] = __uint_as_float(v[0] << 16);
      k4[1] = __uint_as_float(v[0] & 0xFFFF0000u);
      k4[2] = __uint_as_float(v[1] << 16);
      k4[3] = __uint_as_float(v[1] & 0xFFFF0000u);
    } else {
      const floatx4 v = *reinterpret_cast<const floatx4*>(
          reinterpret_cast<const float*>(src) + D_C + 4 * lane);
      for (int k = 0; k < 4; ++k) k4[k] = v[k];
    }
    // (cos, sin) of pairs 2*lane and 2*lane + 1
    const floatx4 cs =
        *reinterpret_cast<const floatx4*>(p.freqs + static_cast<int64_t>(t) * D_R + 4 * lane);
    float r[4];
    r[0] = k4[0] * cs[0] - k4[1] * cs[1];
    r[1] = k4[0] * cs[1] + k4[1] * cs[0];
    r[2] = k4[2] * cs[2] - k4[3] * cs[3];
    r[3] = k4[2] * cs[3] + k4[3] * cs[2];
    char* rdst = static_cast<char*>(p.rope) + (s * p.rope_bs + t * p.rope_rs) * esz;
    if constexpr (BF16) {
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(rdst) + 4 * lane) =
          u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    } else {
      *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(rdst) + 4 * lane) =
          floatx4{r[0], r[1], r[2], r[3]};
    }
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, bool is_bf16, hipStream_t stream) {
  const int64_t blocks = (p.N + APPEND_ROWS_PER_BLOCK - 1) / APPEND_ROWS_PER_BLOCK;
  auto kern = is_bf16 ? cache_append_kernel<true> : cache_append_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(64 * APPEND_ROWS_PER_BLOCK),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
