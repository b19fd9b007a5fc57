// reconstruct.hip — the literal ("naive") key/value reconstruction.
//
// Operation ("KV Reconstruction", How it works: k^C = W^UK c, v^C = W^UV c,
// key = [k^C ; k^R]; "Value up-projection", prefill excerpt: wkv_b applied to
// the latent, viewed per head, split into k_nope / v, shared k^R broadcast
// and concatenated):
//   kv[n,h,e] = sum_c wkv_b[h*256 + e, c] * c[n,c]
//   K[n,h,:] = [kv[n,h,0:128] ; k_rope[n,:]],   V[n,h,:] = kv[n,h,128:256]
//
// A [N x 512] x [512 x n_h*256] GEMM (K = 512 is short) that writes 671 MB at
// N = 8192, n_h = 128: its floor is the MFMA work and the output writes
// together, so the kernel keeps both busy at once.
//
// bf16 path: a persistent kernel, one workgroup of 4 waves per CU, looping
// over tiles of one head (256 features: the 128 k_nope rows then the 128 v
// rows) x 256 tokens. Wave (wm, wn) accumulates features 128wm.. x tokens
// 128wn.. (4 x 4 v_mfma_f32_32x32x16_bf16 tiles, 256 accumulator registers;
// M = features, N = tokens, K = latent). The latent axis is staged in
// 32-wide slices (32 KB: 256 weight rows + 256 token rows, 64 bytes each)
// into four LDS buffers by LDS-DMA issued from inline assembly, three slices
// ahead of the multiplies and across tile boundaries, so ~96 KB per CU stay
// in flight. The tile's rotary rows ride along with slices 4..11 into a
// fifth 32 KB buffer. A tile's epilogue issues its stores (K, V and the
// rotary copy) and moves straight on: they drain while the next tile
// multiplies. Every wave issues the same number of memory instructions in
// the same order (tail tokens re-read and re-write the last token's row with
// identical values), which makes the vmcnt bookkeeping exact.
// The A-row permutation pi gives each lane 16 consecutive output features
// of one token, i.e. two 16-byte stores.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int RC_TOK = 256;                 // tokens per tile
constexpr int RC_FEAT = ROWS_PER_HEAD;      // 256 features per tile (one head)
constexpr int RC_KC = 32;                   // latent features per stage
constexpr int RC_NSTAGE = D_C / RC_KC;      // 16 stages per tile
constexpr int RC_NBUF = 4;                  // stage buffers
constexpr int RC_AHEAD = RC_NBUF - 1;       // stages in flight ahead of the multiplies
constexpr int RC_STAGE_BYTES = (RC_FEAT + RC_TOK) * RC_KC * 2;  // 32 KiB
constexpr int RC_ROPE_BYTES = RC_TOK * D_R * 2;                 // 32 KiB
constexpr int RC_LOADS = RC_STAGE_BYTES / 1024 / 4;             // 8 DMA per wave per stage
constexpr int RC_ROPE_FIRST = 4;            // stages 4..11 also carry one rotary DMA
constexpr int RC_STORES = 4 * 4 * 2 + RC_TOK * D_R * 2 / 16 / 256;  // 40 per wave per tile

__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int pi_row(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// DMA instructions per wave of the group that stages slice s of a tile
constexpr int rc_loads(int s) {
  return RC_LOADS + (s >= RC_ROPE_FIRST && s < RC_ROPE_FIRST + 8 ? 1 : 0);
}
// s_waitcnt vmcnt(N) at the top of stage s: the group of stage s must have
// landed; the newer memory instructions allowed in flight are the groups of
// stages s+1 and s+2 and, in the first three stages of a tile, the previous
// tile's epilogue stores (issued after group s+2 of tile i-1 = group 2 of
// tile i, before group 3). `prev` is false on a workgroup's first tile (no
// previous stores), `last` true on its last tile (no groups past stage 15).
constexpr int rc_wait(int s, bool prev, bool last) {
  auto L = [&](int t) { return (last && t >= RC_NSTAGE) ? 0 : rc_loads(t % RC_NSTAGE); };
  const int S = prev ? RC_STORES : 0;
  if (s == 0) return L(1) + L(2) + S;
  if (s == 1) return L(2) + S + L(3);
  if (s == 2) return S + L(3) + L(4);
  return L(s + 1) + L(s + 2);
}
}  // namespace

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Output stores: whole 256-byte rows of one token and head (128-byte rows
// for the rotary copy), non-temporal: the 671 MB of outputs at N = 8192 then
// do not displace the weight and latent rows later tiles re-read from L2
// (measured 323 against 362 us with ordinary stores; with the 16-byte
// pieces of the MFMA layout, non-temporal stores were slower, since L2 then
// cannot merge the pieces of a line).
__device__ __forceinline__ void rc_store(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate out of range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Stage slice k0..k0+31 of the head's 256 weight rows (w_d) and the tile's
// 256 token rows (x_d; rows past last_row re-read it) into `stage`: chunk j
// (16 bytes) of row r lands at LDS chunk 4r + (j ^ swz4(r)), weight rows
// first. Eight DMA instructions per wave.
__device__ __forceinline__ void rc_stage(i32x4 w_d, i32x4 x_d, int last_row, int k0,
                                         uint32_t stage, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int blk = k * 4 + wave;  // 1 KB block of the stage
    const int pch = (blk & 15) * 64 + lane;
    const int row = pch >> 2;
    const int c = (pch & 3) ^ swz4(row);
    if (k < 4) {
      dma16(w_d, stage + blk * 1024, static_cast<uint32_t>(row * (D_C * 2) + k0 * 2 + c * 16), 0);
    } else {
      const int r = row < last_row ? row : last_row;
      dma16(x_d, stage + blk * 1024, static_cast<uint32_t>(r * (D_C * 2) + k0 * 2 + c * 16), 0);
    }
  }
}

// Rotary rows of the tile (contiguous 256 x 128 bytes; rows past last_row
// re-read it): 1 KB block q = 4j + wave, one DMA instruction.
__device__ __forceinline__ void rc_rope(i32x4 r_d, int last_row, int j, uint32_t rope,
                                        int wave, int lane) {
  const int q = 4 * j + wave;
  const int tok = q * 8 + (lane >> 3);
  const int t = tok < last_row ? tok : last_row;
  dma16(r_d, rope + q * 1024, static_cast<uint32_t>(t * (D_R * 2) + (lane & 7) * 16), 0);
}

__global__ __launch_bounds__(256, 1) void kv_reconstruct_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ k_rope,
    const uint16_t* __restrict__ w, uint16_t* __restrict__ Kout, uint16_t* __restrict__ Vout,
    int64_t N, int n_h) {
  __shared__ __attribute__((aligned(16))) char lds[RC_NBUF * RC_STAGE_BYTES + RC_ROPE_BYTES];
  const int ntt = static_cast<int>((N + RC_TOK - 1) / RC_TOK);
  const int ntiles = ntt * n_h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;  // feature half (k_nope / v), token half
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const uint32_t rope_lds = lds0 + RC_NBUF * RC_STAGE_BYTES;
  const char* rope_buf = lds + RC_NBUF * RC_STAGE_BYTES;
  // this workgroup's tiles: t = blockIdx.x + i * gridDim.x, i < my_tiles;
  // tile t = (head t / ntt, token tile t % ntt)
  const int my_tiles = (ntiles - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                       static_cast<int>(gridDim.x);
  if (my_tiles <= 0) return;

  struct Tile {
    i32x4 w_d, x_d, r_d;
    int last_row, h;
    int64_t tok0;
  };
  auto tile_of = [&](int i) {
    Tile T;
    const int t = static_cast<int>(blockIdx.x) + i * static_cast<int>(gridDim.x);
    T.h = t / ntt;
    T.tok0 = static_cast<int64_t>(t % ntt) * RC_TOK;
    T.w_d = make_rsrc(w + static_cast<int64_t>(T.h) * ROWS_PER_HEAD * D_C);
    T.x_d = make_rsrc(x + T.tok0 * D_C);
    T.r_d = make_rsrc(k_rope + T.tok0 * D_R);
    T.last_row = static_cast<int>(N - 1 - T.tok0 < RC_TOK - 1 ? N - 1 - T.tok0 : RC_TOK - 1);
    return T;
  };
  // the DMA group of stage s of tile T into buffer slot
  auto issue = [&](const Tile& T, int s, int slot) {
    rc_stage(T.w_d, T.x_d, T.last_row, s * RC_KC, lds0 + slot * RC_STAGE_BYTES, wave, lane);
    if (s >= RC_ROPE_FIRST && s < RC_ROPE_FIRST + 8)
      rc_rope(T.r_d, T.last_row, s - RC_ROPE_FIRST, rope_lds, wave, lane);
  };

  floatx16 acc[4][4];
  Tile cur = tile_of(0);
  // prologue: groups of stages 0..2 of the first tile (slots 0..2)
#pragma unroll
  for (int s = 0; s < RC_AHEAD; s++) issue(cur, s, s);

  int gstage = 0;  // stages begun so far (the buffer slot is gstage % RC_NBUF)
  for (int i = 0; i < my_tiles; i++) {
    const bool prev = i > 0, last = i + 1 == my_tiles;
    Tile nxt = last ? cur : tile_of(i + 1);
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int b = 0; b < 4; b++) acc[a][b] = floatx16{};
    static_for<0, RC_NSTAGE>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      // group s landed; stage s-1's buffer is free for the group 3 ahead
      if (prev && !last) wait_vm<rc_wait(s, true, false)>();
      else if (prev) wait_vm<rc_wait(s, true, true)>();
      else if (!last) wait_vm<rc_wait(s, false, false)>();
      else wait_vm<rc_wait(s, false, true)>();
      __syncthreads();
      const int ahead = s + RC_AHEAD;
      const int slot_ahead = (gstage + RC_AHEAD) & (RC_NBUF - 1);
      if (ahead < RC_NSTAGE)
        issue(cur, ahead, slot_ahead);
      else if (!last)
        issue(nxt, ahead - RC_NSTAGE, slot_ahead);
      const char* buf = lds + (gstage & (RC_NBUF - 1)) * RC_STAGE_BYTES;
      gstage++;
#pragma unroll
      for (int ks = 0; ks < RC_KC / 16; ks++) {
        const int c = 2 * ks + g;
        bf16x8 av[4], bv[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          const int row = wm * 128 + mt * 32 + pi_row(n);
          av[mt] = as_bf16x8(ld_lds16(buf + (row * 4 + (c ^ swz4(row))) * 16));
        }
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
          const int row = wn * 128 + nt * 32 + n;
          bv[nt] = as_bf16x8(ld_lds16(buf + RC_FEAT * RC_KC * 2 + (row * 4 + (c ^ swz4(row))) * 16));
        }
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
          for (int nt = 0; nt < 4; nt++) acc[mt][nt] = mfma32x32x16(av[mt], bv[nt], acc[mt][nt]);
      }
    });
    // K[n,h,128:192] = k_rope[n,:] from the staged rows: 8 chunks per token
#pragma unroll
    for (int k = 0; k < RC_TOK * 8 / 256; k++) {
      const int idx = k * 256 + static_cast<int>(threadIdx.x);
      const int tl = min(idx >> 3, cur.last_row);
      const u32x4 v = ld_lds16(rope_buf + (idx >> 3) * 128 + (idx & 7) * 16);
      rc_store(Kout + ((cur.tok0 + tl) * n_h + cur.h) * (D_N + D_R) + D_N + (idx & 7) * 8, v);
    }
    // every wave is done with the rotary rows: the buffer now stages each
    // wave's outputs (8 KB per wave), so that every store instruction writes
    // whole 256-byte rows (4 tokens) instead of 64 separate 16-byte pieces.
    // The buffer is next written by the rotary DMA issued after the barrier
    // of the next tile's stage 1.
    __syncthreads();
    char* stg = const_cast<char*>(rope_buf) + wave * 8192;
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      // lane (token n of N-tile nt, half g) holds features 32mt + 16g .. +15
      // of half wm: chunks 4mt + 2g, +1 of the token's 16-chunk row,
      // XOR-swizzled by token
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        u32x4 v0, v1;
#pragma unroll
        for (int w2 = 0; w2 < 4; w2++) {
          v0[w2] = pack_bf16x2(acc[mt][nt][2 * w2], acc[mt][nt][2 * w2 + 1]);
          v1[w2] = pack_bf16x2(acc[mt][nt][8 + 2 * w2], acc[mt][nt][8 + 2 * w2 + 1]);
        }
        const int c0 = 4 * mt + 2 * g;
        *reinterpret_cast<u32x4*>(stg + n * 256 + ((c0 ^ (n & 15)) << 4)) = v0;
        *reinterpret_cast<u32x4*>(stg + n * 256 + (((c0 + 1) ^ (n & 15)) << 4)) = v1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // 16 lanes per token row: tokens 4i + lane/16, chunk lane % 16; tail
      // tokens rewrite the last token's row with identical values
      u32x4 rows[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int r = 4 * i + (lane >> 4), c = lane & 15;
        rows[i] = ld_lds16(stg + r * 256 + ((c ^ (r & 15)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int r = 4 * i + (lane >> 4), c = lane & 15;
        const int64_t tk = cur.tok0 + min(wn * 128 + nt * 32 + r, cur.last_row);
        uint16_t* dst = wm == 0 ? Kout + (tk * n_h + cur.h) * (D_N + D_R) + c * 8
                                : Vout + (tk * n_h + cur.h) * D_V + c * 8;
        rc_store(dst, rows[i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    cur = nxt;
  }
}

// fp32: one block per (token, head); thread e computes feature e of the 256.
__global__ __launch_bounds__(256) void kv_reconstruct_f32_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ k_rope,
                                                                 const float* __restrict__ w,
                                                                 float* __restrict__ Kout,
                                                                 float* __restrict__ Vout,
                                                                 int n_h) {
  __shared__ float xs[D_C];
  const int64_t tk = blockIdx.x / n_h;
  const int h = blockIdx.x % n_h;
  for (int c = threadIdx.x; c < D_C; c += 256) xs[c] = x[tk * D_C + c];
  __syncthreads();
  const int e = threadIdx.x;
  const float* wrow = w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + e) * D_C;
  float acc = 0.f;
  for (int c = 0; c < D_C; c++) acc = fmaf(wrow[c], xs[c], acc);
  if (e < D_N)
    Kout[(tk * n_h + h) * (D_N + D_R) + e] = acc;
  else
    Vout[(tk * n_h + h) * D_V + (e - D_N)] = acc;
  if (e < D_R) Kout[(tk * n_h + h) * (D_N + D_R) + D_N + e] = k_rope[tk * D_R + e];
}

// Compute units of the current device (cached per device).
static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static int cache[64] = {0};
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  return cus;
}

hipError_t launch_kv_reconstruct(const void* c, const void* k_rope, const void* wkv_b, void* K,
                                 void* V, int64_t N, int n_h, bool is_bf16, hipStream_t stream) {
  if (is_bf16) {
    const int64_t tiles = (N + RC_TOK - 1) / RC_TOK * n_h;
    const int64_t grid = tiles < cu_count() ? tiles : cu_count();
    hipLaunchKernelGGL(kv_reconstruct_bf16_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(c),
                       static_cast<const uint16_t*>(k_rope), static_cast<const uint16_t*>(wkv_b),
                       static_cast<uint16_t*>(K), static_cast<uint16_t*>(V), N, n_h);
  } else {
    hipLaunchKernelGGL(kv_reconstruct_f32_kernel, dim3(static_cast<unsigned>(N * n_h)), dim3(256), 0,
                       stream, static_cast<const float*>(c), static_cast<const float*>(k_rope),
                       static_cast<const float*>(wkv_b), static_cast<float*>(K),
                       static_cast<float*>(V), n_h);
  }
  return hipGetLastError();
}

}  // namespace mla
