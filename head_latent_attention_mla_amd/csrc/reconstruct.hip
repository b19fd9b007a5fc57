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
// bf16 path: one workgroup of 8 waves (two per SIMD) per (head, token chunk);
// wave w owns output features 32w..32w+31 of the head (waves 0-3 the k_nope
// rows, 4-7 the v rows) and holds those 32 rows of wkv_b, the MFMA A
// operands of all 32 k-steps, in registers for the whole kernel (128
// registers a lane): every weight byte is fetched once per workgroup. The
// chunk's tokens stream through LDS in stages of 32 whole latent rows (1 KB
// each, full cache lines; the rotary rows ride along), RW_LEAD stages ahead
// of the multiplies; per stage a wave runs one chain of 32
// v_mfma_f32_32x32x16_bf16 (B = the stage's token rows). The A-row order pi
// gives each lane 16 consecutive features of one token, which go to an LDS
// output stage (double-buffered) so that every store instruction writes
// whole rows. Roles split the memory work: waves 0-3 issue all the LDS-DMA
// (and copy the rotary rows into the output stage), waves 4-7 issue all the
// stores, five per stage, between their multiplies of the next stage. A
// loader wave's vector-memory counter then holds only its own DMA, so each
// stage waits exactly for its group; the storers never wait for a store.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int RW_WAVES = 8;                           // waves per workgroup
constexpr int RW_TOK = 32;                            // tokens per stage
constexpr int RW_NBUF = 3;                            // staged token buffers
constexpr int RW_LEAD = RW_NBUF - 1;                  // stages in flight ahead
constexpr int RW_PITCH = 68 * 16;                     // bytes per staged latent row
constexpr int RW_LAT_BYTES = RW_TOK * RW_PITCH;       // 34,816
constexpr int RW_ROPE_BYTES = RW_TOK * D_R * 2;       // 4,096
constexpr int RW_BUF_BYTES = RW_LAT_BYTES + RW_ROPE_BYTES;
constexpr int RW_OPITCH = 17 * 16;                    // bytes per staged 128-feature output row
constexpr int RW_OUT_BYTES = 2 * RW_TOK * RW_OPITCH + RW_ROPE_BYTES;  // k_nope, v, rotary
constexpr int RW_DMA = RW_TOK / 4 + 1;                // DMA per loader wave and stage
constexpr int RW_STORES = (2 * RW_TOK * 16 + RW_TOK * 8) / 64 / 4;  // 5 per storer and stage
constexpr int RW_RING = 4;                            // token operands read ahead
static_assert(RW_NBUF * RW_BUF_BYTES + 2 * RW_OUT_BYTES <= 160 * 1024, "LDS budget");

// Latent row t of a stage starts at chunk rw_shift(t) of its 68-chunk slot: a
// 16-byte B-operand read of 16 consecutive rows at one chunk then lands in
// 16 distinct bank quarters ((4t + shift + c) mod 16 is a permutation).
__device__ __forceinline__ int rw_shift(int t) { return (t >> 2) & 3; }
// A-operand row i holds feature pi(i) of the wave's 32: accumulator r of lane
// half g is then feature 16g + r.
__device__ __forceinline__ int rw_pi(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
}  // namespace

// One stage of the loader wave w (0..3): latent rows 8w..8w+7 of the stage
// (one DMA each, the row's offset a scalar) and rotary rows 8w..8w+7 (one
// DMA); tokens past the last re-read it. The buffer descriptors are based at
// the stage's first token, so every offset stays below 32 KB however long
// the sequence.
__device__ __forceinline__ void rw_stage(const uint16_t* x, const uint16_t* k_rope, int64_t tok0,
                                         int64_t last, uint32_t buf, int w, int lane) {
  const i32x4 c_d = make_rsrc(x + tok0 * D_C);
  const i32x4 r_d = make_rsrc(k_rope + tok0 * D_R);
  const int lastr = static_cast<int>(last - tok0 < RW_TOK - 1 ? last - tok0 : RW_TOK - 1);
#pragma unroll
  for (int k = 0; k < RW_TOK / 4; k++) {
    const int t = 8 * w + k;
    const int tr = t < lastr ? t : lastr;
    dma16(c_d, buf + t * RW_PITCH + 16 * rw_shift(t), static_cast<uint32_t>(lane * 16),
          __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(tr * (D_C * 2))));
  }
  const int t = 8 * w + (lane >> 3);
  const int tr = t < lastr ? t : lastr;
  dma16(r_d, buf + RW_LAT_BYTES + w * 1024,
        static_cast<uint32_t>(tr * (D_R * 2) + (lane & 7) * 16), 0);
}

__global__ __launch_bounds__(RW_WAVES * 64, 1) void kv_reconstruct_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ k_rope,
    const uint16_t* __restrict__ w, uint16_t* __restrict__ Kout, uint16_t* __restrict__ Vout,
    int64_t N, int n_h, int chunks, int64_t chunk_tok) {
  __shared__ __attribute__((aligned(16))) char lds[RW_NBUF * RW_BUF_BYTES + 2 * RW_OUT_BYTES];
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; renumber
  // them so that the chunks of one head share an XCD (its weights are then
  // fetched into one L2).
  int h, ck;
  {
    const int G = static_cast<int>(gridDim.x), L = static_cast<int>(blockIdx.x);
    const int j = (G & 7) == 0 ? (L & 7) * (G >> 3) + (L >> 3) : L;
    h = j / chunks;
    ck = j - h * chunks;
  }
  const int64_t tok_begin = static_cast<int64_t>(ck) * chunk_tok;
  const int64_t tok_end = tok_begin + chunk_tok < N ? tok_begin + chunk_tok : N;
  if (tok_begin >= tok_end) return;  // (uniform over the workgroup)
  const int nst = static_cast<int>((tok_end - tok_begin + RW_TOK - 1) / RW_TOK);
  const int64_t last = N - 1;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const bool loader = wave < 4;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  auto buf_addr = [&](int s) { return lds0 + (s % RW_NBUF) * RW_BUF_BYTES; };
  char* const outs = lds + RW_NBUF * RW_BUF_BYTES;

  // the first RW_LEAD stages in flight, then this wave's 32 weight rows
  if (loader) {
#pragma unroll
    for (int s = 0; s < RW_LEAD; s++)
      if (s < nst) rw_stage(x, k_rope, tok_begin + s * RW_TOK, last, buf_addr(s), wave, lane);
  }
  bf16x8 A[D_C / 16];
  {
    const uint16_t* wr =
        w + (static_cast<int64_t>(h) * ROWS_PER_HEAD + 32 * wave + rw_pi(n)) * D_C + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D_C / 16; ks++) A[ks] = as_bf16x8(ld16(wr + 16 * ks));
  }
  // consume the weight loads here (the wait also covers the older DMA)
#pragma unroll
  for (int ks = 0; ks < D_C / 16; ks++) asm volatile("" : : "v"(A[ks]));

  // B operands: token row n, chunk 2ks + g
  const int b_off = n * RW_PITCH + 16 * (rw_shift(n) + g);
  // output stage row of this lane: token n, chunks 4(wave % 4) + 2g, +1
  const int o_off = (loader ? 0 : RW_TOK * RW_OPITCH) + n * RW_OPITCH;
  const int o_c0 = 4 * (wave & 3) + 2 * g;

  // the storers' five stores of one stage: instruction j = 4i + (wave - 4)
  // of 20 (8 k_nope, 8 v, 4 rotary). Per instruction the lane's token t of
  // the stage, its source in the output stage and its destination for the
  // chunk's first stage (later stages: + 32 tokens of rows each)
  int st_t[RW_STORES], st_src[RW_STORES];
  uint16_t* sp[RW_STORES];
  int64_t st_step[RW_STORES];
#pragma unroll
  for (int i = 0; i < RW_STORES; i++) {
    const int j = 4 * i + ((wave - 4) & 3);
    int c;
    if (j < 16) {  // k_nope (j < 8) or v rows: 4 tokens x 16 chunks
      st_t[i] = 4 * (j & 7) + (lane >> 4);
      c = lane & 15;
      st_src[i] = (j < 8 ? 0 : RW_TOK * RW_OPITCH) + st_t[i] * RW_OPITCH + 16 * c;
    } else {  // rotary rows: 8 tokens x 8 chunks
      st_t[i] = 8 * (j - 16) + (lane >> 3);
      c = lane & 7;
      st_src[i] = 2 * RW_TOK * RW_OPITCH + st_t[i] * 128 + 16 * c;
    }
    const int64_t row = (tok_begin + st_t[i]) * n_h + h;
    sp[i] = j < 8 ? Kout + row * (D_N + D_R) + 8 * c
          : j < 16 ? Vout + row * D_V + 8 * c
                   : Kout + row * (D_N + D_R) + D_N + 8 * c;
    st_step[i] = static_cast<int64_t>(RW_TOK) * n_h * (j >= 8 && j < 16 ? D_V : D_N + D_R);
  }
  u32x4 sv[RW_STORES];
  bool sok[RW_STORES];
  // outputs of stage s (s = 0, 1, ... in order): read from the output stage
  auto load_stores = [&](int s) {
    const char* ob = outs + (s & 1) * RW_OUT_BYTES;
    const int64_t left = tok_end - (tok_begin + static_cast<int64_t>(s) * RW_TOK);
#pragma unroll
    for (int i = 0; i < RW_STORES; i++) {
      sok[i] = st_t[i] < left;
      sv[i] = ld_lds16(ob + st_src[i]);
    }
  };
  // store i, then on to the same rows of the next stage
  auto store = [&](int i) {
    if (sok[i]) __builtin_nontemporal_store(sv[i], reinterpret_cast<u32x4*>(sp[i]));
    sp[i] += st_step[i];
  };

  // this wave's 32 features of the 32 tokens of stage s into output stage s & 1
  auto write_out = [&](int s, const floatx16& acc) {
    char* ob = outs + (s & 1) * RW_OUT_BYTES;
    u32x4 v0, v1;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v0[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
      v1[k] = pack_bf16x2(acc[8 + 2 * k], acc[8 + 2 * k + 1]);
    }
    *reinterpret_cast<u32x4*>(ob + o_off + 16 * o_c0) = v0;
    *reinterpret_cast<u32x4*>(ob + o_off + 16 * (o_c0 + 1)) = v1;
  };
  // loaders: rotary rows 8w..8w+7 of stage s, from its token buffer into
  // output stage s & 1
  auto read_rope = [&](int s) {
    return ld_lds16(lds + (s % RW_NBUF) * RW_BUF_BYTES + RW_LAT_BYTES + wave * 1024 + 16 * lane);
  };
  auto write_rope = [&](int s, u32x4 v) {
    *reinterpret_cast<u32x4*>(outs + (s & 1) * RW_OUT_BYTES + 2 * RW_TOK * RW_OPITCH +
                              wave * 1024 + 16 * lane) = v;
  };

  // Stage s. The outputs of stage s-1 (accumulators `prev`) go to the output
  // stage between the first multiplies of stage s, and the storers store
  // those of stage s-2 (complete since the barrier) between the multiplies;
  // the loaders move stage s-1's rotary rows out of its token buffer before
  // they refill that buffer with stage s+RW_LEAD.
  auto body = [&](int s, floatx16& acc, const floatx16& prev) {
    // stage s landed (a loader's counter holds only its DMA: the groups of
    // stages s .. s+RW_LEAD-1 that exist)
    if (loader) {
      if (s + 1 < nst)
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(RW_DMA) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // stage s published; every wave is done with stage s-1's token buffer and
    // the output stage of s-2 is complete
    __syncthreads();
    const bool st = !loader && s >= 2;
    if (st) load_stores(s - 2);
    u32x4 rope = {};
    if (loader && s >= 1) rope = read_rope(s - 1);
    const char* bp = lds + (s % RW_NBUF) * RW_BUF_BYTES + b_off;
    u32x4 ring[RW_RING];
#pragma unroll
    for (int j = 0; j < RW_RING; j++) ring[j] = ld_lds16(bp + 32 * j);
#pragma unroll
    for (int ks = 0; ks < D_C / 16; ks++) {
      const u32x4 b = ring[ks % RW_RING];
      if (ks + RW_RING < D_C / 16) ring[ks % RW_RING] = ld_lds16(bp + 32 * (ks + RW_RING));
      if (ks == 1 && s >= 1) {
        write_out(s - 1, prev);
        if (loader) write_rope(s - 1, rope);
      }
      // (the rotary rows were read and written back at ks = 1: the buffer
      // is free for the DMA)
      if (ks == 4 && loader && s + RW_LEAD < nst)
        rw_stage(x, k_rope, tok_begin + static_cast<int64_t>(s + RW_LEAD) * RW_TOK, last,
                 buf_addr(s + RW_LEAD), wave, lane);
      if (st && ks % 6 == 3 && ks / 6 < RW_STORES) store(ks / 6);
      acc = mfma32x32x16(A[ks], as_bf16x8(b), ks == 0 ? floatx16{} : acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  floatx16 acc0 = {}, acc1 = {};
  for (int s = 0; s < nst; s += 2) {
    body(s, acc0, acc1);
    if (s + 1 < nst) body(s + 1, acc1, acc0);
  }
  // the last two stages' outputs: nst-2 (written during stage nst-1) and
  // nst-1 (still in registers)
  __syncthreads();
  if (!loader && nst >= 2) {
    load_stores(nst - 2);
#pragma unroll
    for (int i = 0; i < RW_STORES; i++) store(i);
  }
  {
    const floatx16 lastacc = (nst - 1) & 1 ? acc1 : acc0;
    u32x4 rope = {};
    if (loader) rope = read_rope(nst - 1);
    write_out(nst - 1, lastacc);
    if (loader) write_rope(nst - 1, rope);
  }
  __syncthreads();
  if (!loader) {
    load_stores(nst - 1);
#pragma unroll
    for (int i = 0; i < RW_STORES; i++) store(i);
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
    // token chunks per head: enough (head, chunk) workgroups to fill the CUs,
    // each chunk a whole number of 32-token stages
    const int cus = cu_count();
    int64_t chunks = n_h < cus ? cus / n_h : 1;
    const int64_t stages = (N + RW_TOK - 1) / RW_TOK;
    if (chunks > stages) chunks = stages;
    const int64_t chunk_tok = (stages + chunks - 1) / chunks * RW_TOK;
    chunks = (N + chunk_tok - 1) / chunk_tok;
    const int64_t grid = static_cast<int64_t>(n_h) * chunks;
    hipLaunchKernelGGL(kv_reconstruct_bf16_kernel, dim3(static_cast<unsigned>(grid)),
                       dim3(RW_WAVES * 64), 0, stream, static_cast<const uint16_t*>(c),
                       static_cast<const uint16_t*>(k_rope), static_cast<const uint16_t*>(wkv_b),
                       static_cast<uint16_t*>(K), static_cast<uint16_t*>(V), N, n_h,
                       static_cast<int>(chunks), chunk_tok);
  } else {
    hipLaunchKernelGGL(kv_reconstruct_f32_kernel, dim3(static_cast<unsigned>(N * n_h)), dim3(256), 0,
                       stream, static_cast<const float*>(c), static_cast<const float*>(k_rope),
                       static_cast<const float*>(wkv_b), static_cast<float*>(K),
                       static_cast<float*>(V), n_h);
  }
  return hipGetLastError();
}

}  // namespace mla
