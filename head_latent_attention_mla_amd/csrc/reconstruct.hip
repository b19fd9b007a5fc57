// reconstruct.hip — the literal ("naive") key/value reconstruction.
//
// Operation ("KV Reconstruction", How it works: k^C = W^UK c, v^C = W^UV c,
// key = [k^C ; k^R]; "Value up-projection", prefill excerpt: wkv_b applied to
// the latent, viewed per head, split into k_nope / v, shared k^R broadcast
// and concatenated):
//   kv[n,h,e] = sum_c wkv_b[h*256 + e, c] * c[n,c]
//   K[n,h,:] = [kv[n,h,0:128] ; k_rope[n,:]],   V[n,h,:] = kv[n,h,128:256]
//
// A [N x 512] x [512 x n_h*256] GEMM (K = 512 is short) whose epilogue routes
// each 128-feature half of a head to K or V, plus a 64-feature copy of k_rope
// into every head's key. bf16 path: workgroup tile = 128 features (one half
// of one head) x 256 tokens, 4 waves of 64 x 128, v_mfma_f32_32x32x16_bf16
// with M = features, N = tokens, K = latent. Both operands are K-contiguous
// in memory; 32-wide K slices are staged HBM -> LDS with
// global_load_lds_dwordx4 (double-buffered, XOR-swizzled against bank
// conflicts). The A-row permutation pi gives each lane 16 consecutive output
// features of one token, i.e. two 16-byte stores.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int RT_TOK = 256;                  // tokens per workgroup
constexpr int RT_FEAT = 128;                 // features per workgroup
constexpr int RT_KC = 32;                    // latent features per stage
constexpr int A_CHUNKS = RT_FEAT * RT_KC / 8;  // 512 16-byte chunks
constexpr int B_CHUNKS = RT_TOK * RT_KC / 8;   // 1024
constexpr int STAGE_BYTES = (A_CHUNKS + B_CHUNKS) * 16;  // 24 KiB

__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int pi_row(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
}  // namespace

__device__ __forceinline__ void rc_issue_stage(const uint16_t* wsrc, const uint16_t* xsrc,
                                               int64_t N, int64_t tok0, int k0, char* stage,
                                               int wave, int lane) {
  // A: 128 feature rows x 4 chunks; B: 256 token rows x 4 chunks
#pragma unroll
  for (int k = 0; k < A_CHUNKS / 256; k++) {
    const int blk = k * 4 + wave;
    const int pch = blk * 64 + lane;
    const int row = pch >> 2;
    const int c = (pch & 3) ^ swz4(row);
    __builtin_amdgcn_global_load_lds(wsrc + static_cast<int64_t>(row) * D_C + k0 + c * 8,
                                     (lds_void*)(stage + blk * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < B_CHUNKS / 256; k++) {
    const int blk = k * 4 + wave;
    const int pch = blk * 64 + lane;
    const int row = pch >> 2;
    const int c = (pch & 3) ^ swz4(row);
    int64_t tk = tok0 + row;
    tk = tk < N ? tk : N - 1;  // tail tokens load a valid row; results are not stored
    __builtin_amdgcn_global_load_lds(xsrc + tk * D_C + k0 + c * 8,
                                     (lds_void*)(stage + A_CHUNKS * 16 + blk * 1024),
                                     16, 0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void kv_reconstruct_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ k_rope,
    const uint16_t* __restrict__ w, uint16_t* __restrict__ Kout, uint16_t* __restrict__ Vout,
    int64_t N, int n_h) {
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE_BYTES];
  const int ntt = static_cast<int>((N + RT_TOK - 1) / RT_TOK);
  const int tt = blockIdx.x % ntt;
  const int hh = blockIdx.x / ntt;  // head * 2 + half
  const int h = hh >> 1, half = hh & 1;
  const int64_t tok0 = static_cast<int64_t>(tt) * RT_TOK;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int wf = wave & 1, wn = wave >> 1;
  const uint16_t* wsrc = w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + half * 128) * D_C;

  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = floatx16{};

  rc_issue_stage(wsrc, x, N, tok0, 0, lds, wave, lane);
  constexpr int NSTAGE = D_C / RT_KC;  // 16
  for (int st = 0; st < NSTAGE; st++) {
    char* cur = lds + (st & 1) * STAGE_BYTES;
    if (st + 1 < NSTAGE) {
      rc_issue_stage(wsrc, x, N, tok0, (st + 1) * RT_KC, lds + ((st + 1) & 1) * STAGE_BYTES, wave,
                     lane);
      __builtin_amdgcn_s_waitcnt(0xF70 | ((A_CHUNKS + B_CHUNKS) / 256));
    } else {
      __builtin_amdgcn_s_waitcnt(0xF70);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < RT_KC / 16; ks++) {
      const int c = 2 * ks + g;
      bf16x8 a[2], bb[4];
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        const int row = wf * 64 + mt * 32 + pi_row(n);
        a[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(cur + (row * 4 + (c ^ swz4(row))) * 16));
      }
#pragma unroll
      for (int nt = 0; nt < 4; nt++) {
        const int row = wn * 128 + nt * 32 + n;
        bb[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(cur + A_CHUNKS * 16 +
                                                           (row * 4 + (c ^ swz4(row))) * 16));
      }
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < 4; nt++) acc[mt][nt] = mfma32x32x16(a[mt], bb[nt], acc[mt][nt]);
    }
    __syncthreads();
  }

  // epilogue: lane (token n of N-tile nt, half g) holds features 16g..16g+15
  // of M-tile mt
#pragma unroll
  for (int nt = 0; nt < 4; nt++) {
    const int64_t tk = tok0 + wn * 128 + nt * 32 + n;
    if (tk >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int e = wf * 64 + mt * 32 + 16 * g;  // feature within the half
      u32x4 v0, v1;
#pragma unroll
      for (int w2 = 0; w2 < 4; w2++) {
        v0[w2] = pack_bf16x2(acc[mt][nt][2 * w2], acc[mt][nt][2 * w2 + 1]);
        v1[w2] = pack_bf16x2(acc[mt][nt][8 + 2 * w2], acc[mt][nt][8 + 2 * w2 + 1]);
      }
      uint16_t* dst = half == 0 ? Kout + (tk * n_h + h) * (D_N + D_R) + e
                                : Vout + (tk * n_h + h) * D_V + e;
      st16(dst, v0);
      st16(dst + 8, v1);
    }
  }
  if (half == 0) {
    // K[n,h,128:192] = k_rope[n,:]: 8 chunks of 16 bytes per token
#pragma unroll
    for (int k = 0; k < RT_TOK * 8 / 256; k++) {
      const int idx = k * 256 + threadIdx.x;
      const int64_t tk = tok0 + (idx >> 3);
      const int c = idx & 7;
      if (tk < N) st16(Kout + (tk * n_h + h) * (D_N + D_R) + D_N + c * 8, ld16(k_rope + tk * D_R + c * 8));
    }
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

hipError_t launch_kv_reconstruct(const void* c, const void* k_rope, const void* wkv_b, void* K,
                                 void* V, int64_t N, int n_h, bool is_bf16, hipStream_t stream) {
  if (is_bf16) {
    const int64_t ntt = (N + RT_TOK - 1) / RT_TOK;
    hipLaunchKernelGGL(kv_reconstruct_bf16_kernel, dim3(static_cast<unsigned>(ntt * n_h * 2)),
                       dim3(256), 0, stream, static_cast<const uint16_t*>(c),
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
