// attention.hip — ordinary (naive-path) attention over reconstructed keys and
// values.
//
// Operation ("Value up-projection", prefill excerpt): per head,
// q = [q_nope ; q_pe] (192 features) and k = [k_nope ; k^R] (192), v (128);
//   z[s,t] = scale * q[s] . k[t]
//   z = -inf where t is outside query s's own index set (the index mask is a
//       scatter of each query token's indices into a -inf row) and, with the
//       causal mask, where t > T - S + s (queries sit at the end of the keys)
//   out[s] = sum_t softmax_t(z[s,:]) v[t]
//
// bf16 kernel: flash-style, one workgroup of 8 waves per (sequence, head,
// block of 256 queries); wave w owns queries 32w..32w+31 of the block. Keys
// stream in 64-key tiles (k: 64 x 192, v: 64 x 128) from HBM/L2 into LDS
// rings with buffer_load ... lds (the tile after next is in flight while one
// is consumed): keys three tiles deep, values four (odd waves mix a tile's
// values one tile later than even waves). Per 32-key half-tile each wave computes
//   S^T[32 keys x 32 queries] = K . Q^T   (12 k-steps of 32x32x16 bf16 MFMA;
//       A = key rows read from LDS in the row order pi, so accumulator r of
//       lane half g is key 16g + r; B = the wave's queries, in registers)
//   online softmax in the log2 domain, per lane (each lane holds one query
//       and 16 keys; one cross-half exchange per max); the running max is
//       raised lazily (only when a score beats it by 2^8), so the output
//       accumulators are rescaled rarely, and tiles wholly visible to the
//       wave skip the mask
//   O^T[128 x 32] += V^T . P^T   (8 MFMAs; A = value rows read with the
//       gfx950 transposing LDS load ds_read_b64_tr_b16; B = P straight from
//       the score accumulators)
// LDS rows are XOR-swizzled by 16-byte chunk so that both the score reads and
// the transposing reads are free of bank conflicts.
//
// Workgroups are renumbered so that the query blocks of one (sequence, head)
// run on one XCD at the same time and share its L2: every key/value tile is
// fetched from HBM about once and then served from L2 to all of them. With
// the causal mask the blocks with the most keys are dispatched first.
//
// The index sets arrive as int32 [B, S, K]; a scatter kernel turns them into
// one bit per (query, key) in the workspace, laid out [B, key word, query]
// (word w holds keys 32w..32w+31): the words of one key tile for a block of
// queries are contiguous and are staged into LDS with the tile.
//
// fp32 kernel: a plain per-(sequence, query, head) VALU kernel (a
// correctness path for the float32 interface).
#include <algorithm>
#include <climits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int AT_WAVES = 8;
constexpr int AT_QBLOCK = 32 * AT_WAVES;       // queries per workgroup
constexpr int AT_KT = 64;                       // keys per tile
constexpr int AT_DQK = 192;                     // query/key features
constexpr int AT_DV = 128;                      // value features
constexpr int AT_K_PITCH = AT_DQK * 2;          // 384 bytes per key row in LDS
constexpr int AT_V_PITCH = AT_DV * 2;           // 256 bytes per value row
constexpr int AT_K_BYTES = AT_KT * AT_K_PITCH;  // 24 KiB
constexpr int AT_V_BYTES = AT_KT * AT_V_PITCH;  // 16 KiB
constexpr int AT_M_BYTES = 2 * AT_QBLOCK * 4;    // 2 mask words per query
// LDS rings: keys and mask words 3 tiles deep, values 4 deep (the second
// wave of each SIMD mixes a tile's values one tile later)
constexpr int AT_NK = 3;
constexpr int AT_NV = 4;
constexpr int AT_V0 = AT_NK * AT_K_BYTES;
constexpr int AT_M0 = AT_V0 + AT_NV * AT_V_BYTES;
constexpr int AT_LDS = AT_M0 + AT_NK * AT_M_BYTES;
constexpr int AT_K_DMA = AT_K_BYTES / 1024 / AT_WAVES;  // 3 wave-DMAs per wave and tile
constexpr int AT_V_DMA = AT_V_BYTES / 1024 / AT_WAVES;  // 2
constexpr int AT_DMA = AT_K_DMA + AT_V_DMA;        // + 1 mask DMA on waves 0, 1 (index sets)
constexpr float AT_LOG2E = 1.4426950408889634f;
constexpr float AT_LN2 = 0.6931471805599453f;
constexpr float AT_SLACK = 8.0f;  // log2 units by which a score may exceed the running max
#ifndef MLA_AT_AHEAD
#define MLA_AT_AHEAD 6
#endif
constexpr int AT_SCORE_AHEAD = MLA_AT_AHEAD;  // key operands read ahead of the score multiplies
constexpr int AT_MIX_AHEAD = MLA_AT_AHEAD;    // value operands read ahead of the mix multiplies

static_assert(AT_K_BYTES % (1024 * AT_WAVES) == 0 && AT_V_BYTES % (1024 * AT_WAVES) == 0,
              "tiles must split into whole wave-DMAs");

// Key rows: 24 chunks of 16 bytes; chunk c of row r is stored at chunk
// position c ^ kswz(r). The score read of lane (i, g) touches row pi(i):
// rows {0..3,16..19,4..7,20..23} (+8) meet distinct bank groups.
__device__ __forceinline__ int kswz(int r) {
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 4) & 1) << 2);
}
// Value rows: 16 chunks; chunk c of row r at position c ^ (4 * (r & 3)).
__device__ __forceinline__ int vswz(int r) { return 4 * (r & 3); }

// Score A-operand row i reads key pi(i) of the half-tile; accumulator r of
// lane half g is then key 16g + r.
__device__ __forceinline__ int at_pi(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }
// Value A-operand feature blocks: block beta holds features 4*tau(beta)..+3
// of a 32-feature tile, so accumulator r of lane half g is feature 16g + r.
__device__ __forceinline__ int at_tau(int beta) { return 4 * (beta & 1) + (beta >> 1); }

typedef __attribute__((address_space(3))) shortx4 at_lds_shortx4;

__device__ __forceinline__ bf16x8 at_tr_pair(const char* lo, const char* hi) {
  const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_shortx4*)(lo));
  const shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_shortx4*)(hi));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// max / sum over the two lane halves (lanes l and l ^ 32 hold the same query)
__device__ __forceinline__ float half_max(float v) {
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float half_sum(float v) { return v + __shfl_xor(v, 32, 64); }

// DMA of key/value tile `tile` (keys t0..t0+63, rows past T re-read row T-1)
// into the LDS slots at byte addresses dst_k (keys), dst_v (values) and dst_m
// (mask words): wave w issues wave-DMAs w, w+8, w+16 of the key tile and
// w, w+8 of the value tile; each covers 1 KB of its slot (64 lanes x 16
// bytes) and the lane loads the global chunk the swizzle puts at its LDS
// position. With index sets, waves 0 and 1 also stage mask words t0/32 and
// t0/32 + 1 of the block's 256 queries.
template <bool SPARSE>
__device__ __forceinline__ void at_issue_tile(const AttnParams& p, int b, int h, int q0, int t0,
                                              uint32_t dst_k, uint32_t dst_v, uint32_t dst_m,
                                              int wave, int lane) {
  const int64_t row_elems = static_cast<int64_t>(p.n_h) * AT_DQK;
  const int64_t vrow_elems = static_cast<int64_t>(p.n_h) * AT_DV;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) +
                       (static_cast<int64_t>(b) * p.T + t0) * row_elems +
                       static_cast<int64_t>(h) * AT_DQK;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v) +
                       (static_cast<int64_t>(b) * p.T + t0) * vrow_elems +
                       static_cast<int64_t>(h) * AT_DV;
  const i32x4 krs = make_rsrc(kb);
  const i32x4 vrs = make_rsrc(vb);
  const int last = p.T - 1 - t0;  // last valid row of this tile
#pragma unroll
  for (int j = 0; j < AT_K_DMA; j++) {
    const int q = (wave + AT_WAVES * j) * 64 + lane;  // 16-byte slot of the stage
    const int r = q / 24, pos = q % 24;
    const int rr = min(r, last);
    const int c = pos ^ kswz(r);
    const uint32_t voff = static_cast<uint32_t>(rr * row_elems * 2 + c * 16);
    dma16(krs, dst_k + (wave + AT_WAVES * j) * 1024, voff, 0);
  }
#pragma unroll
  for (int j = 0; j < AT_V_DMA; j++) {
    const int q = (wave + AT_WAVES * j) * 64 + lane;
    const int r = q >> 4, pos = q & 15;
    const int rr = min(r, last);
    const int c = pos ^ vswz(r);
    const uint32_t voff = static_cast<uint32_t>(rr * vrow_elems * 2 + c * 16);
    dma16(vrs, dst_v + (wave + AT_WAVES * j) * 1024, voff, 0);
  }
  if (SPARSE && wave < 2) {
    const uint32_t* mb = p.mask + (static_cast<int64_t>(b) * p.mask_words + (t0 >> 5) + wave) *
                                      p.s_pad + q0;
    dma16(make_rsrc(mb), dst_m + wave * 1024, 16 * lane, 0);
  }
}

template <bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(64 * AT_WAVES, 1) void attention_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char at_lds[AT_LDS];

  // ---- workgroup -> (sequence, head, query block) ----
  int qb, h, b;
  {
    const int G = gridDim.x;
    const int L = blockIdx.x;
    const int j = (G & 7) == 0 ? (L & 7) * (G >> 3) + (L >> 3) : L;
    const int nqb = p.nqb;
    qb = j % nqb;
    if (CAUSAL) qb = nqb - 1 - qb;  // blocks with the most keys first
    h = (j / nqb) % p.n_h;
    b = j / (nqb * p.n_h);
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int q0 = qb * AT_QBLOCK;
  const int qw = q0 + 32 * wave;          // first query of this wave
  const int q = qw + n;                   // this lane's query
  const int qc = min(q, p.S - 1);         // clamped for loads
  const int shift = p.T - p.S;            // query s sits at position shift + s

  // keys this workgroup needs: all (dense), or up to the last query's position
  int kend = p.T;
  if (CAUSAL) kend = min(p.T, shift + min(q0 + AT_QBLOCK, p.S));
  const int ntiles = (kend + AT_KT - 1) / AT_KT;
  // keys this wave needs (wave-uniform)
  const int wkend = CAUSAL ? min(p.T, shift + min(qw + 32, p.S)) : p.T;
  const bool wave_live = qw < p.S;

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(at_lds));
  auto issue = [&](int tile) {
    at_issue_tile<SPARSE>(p, b, h, q0, tile * AT_KT, lds_base + (tile % AT_NK) * AT_K_BYTES,
                          lds_base + AT_V0 + (tile % AT_NV) * AT_V_BYTES,
                          lds_base + AT_M0 + (tile % AT_NK) * AT_M_BYTES, wave, lane);
  };
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);

  // queries of this lane as score B operands: features 16ks + 8g .. +7
  u32x4 qv[12];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((static_cast<int64_t>(b) * p.S + qc) * p.n_h + h) * AT_DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 12; ks++) qv[ks] = ld16(qp + 16 * ks);
  }

  // per-lane LDS byte offsets (stage-relative)
  // score reads: key row at_pi(n) of the half-tile, chunk (2ks + g) ^ kswz
  int k_off[4];
  {
    const int r = at_pi(n);
#pragma unroll
    for (int bb = 0; bb < 4; bb++) k_off[bb] = r * AT_K_PITCH + 16 * ((2 * bb + g) ^ kswz(r));
  }
  // transposing value reads: row 16g + (j >> 2) (+ 32 half + 8kk (+4)),
  // features 32mt + 4*tau(4a + (j & 3))
  int v_off[4];
  {
    const int jj = lane & 15, a = (lane >> 4) & 1;
    const int tau = at_tau(4 * a + (jj & 3));
    const int r = 16 * g + (jj >> 2);
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
      v_off[mt] = r * AT_V_PITCH + 16 * ((4 * mt + (tau >> 1)) ^ vswz(r)) + 8 * (tau & 1);
  }

  floatx16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) o[mt] = floatx16{};
  float m = -INFINITY;  // running max of scale*log2(e)*z for this lane's query
  float l = 0.f;        // this lane's share of the running sum
  const float sl2 = p.scale * AT_LOG2E;
  const int qpos = shift + q;  // causal: last visible key of this lane's query
  // odd waves mix each tile one tile later than even waves, so that waves
  // sharing a SIMD tend to be in different phases (one multiplying while the
  // other runs the softmax); measured a few per cent faster than all waves
  // in step
  const bool late = (wave & 1) != 0;
  bool pending = false;         // a late wave holds the weights of an unmixed tile
  u32x4 P[2][2];                // weights of the tile being mixed, bf16 [half][k-step]
  // O^T += V^T . P^T over the 64 keys of the value tile at vbase: 16
  // multiplies, step j = (half, kk, mt), so consecutive multiplies update
  // different accumulators; each accumulator still adds its four products in
  // the order (half, kk). The transposing operand reads run AT_MIX_AHEAD
  // steps ahead of their multiplies (an LDS round trip lasts several
  // multiplies), each read kept with its multiply.
  auto mix = [&](const u32x4 (&Pm)[2][2], const char* vbase) {
    auto operand = [&](int j) {
      const int half = j >> 3, kk = (j >> 2) & 1, mt = j & 3;
      const char* lo = vbase + 32 * half * AT_V_PITCH + v_off[mt] + 8 * kk * AT_V_PITCH;
      return at_tr_pair(lo, lo + 4 * AT_V_PITCH);
    };
    bf16x8 ring[AT_MIX_AHEAD];
#pragma unroll
    for (int j = 0; j < AT_MIX_AHEAD; j++) ring[j] = operand(j);
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int half = j >> 3, kk = (j >> 2) & 1, mt = j & 3;
      const bf16x8 A = ring[j % AT_MIX_AHEAD];
      if (j + AT_MIX_AHEAD < 16) ring[j % AT_MIX_AHEAD] = operand(j + AT_MIX_AHEAD);
      o[mt] = mfma32x32x16(A, as_bf16x8(Pm[half][kk]), o[mt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int it = 0; it < ntiles; it++) {
    // tile it resident for every wave; every wave done with tile it-1
    if (it + 1 >= ntiles)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (SPARSE && wave < 2)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(AT_DMA + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(AT_DMA) : "memory");
    __syncthreads();
    if (it + 2 < ntiles)
      issue(it + 2);
    // the second wave of each SIMD mixes the previous tile now, while the
    // first one computes this tile's scores
    if (late && pending) {
      mix(P, at_lds + AT_V0 + ((it - 1) % AT_NV) * AT_V_BYTES);
      pending = false;
    }
    const int t0 = it * AT_KT;
    if (!wave_live || t0 >= wkend) continue;  // nothing of this tile is visible to the wave
    const char* kst = at_lds + (it % AT_NK) * AT_K_BYTES;

    // scores of both 32-key halves as two independent MFMA chains (a half
    // wholly past the wave's keys is computed and masked to weight 0)
    // (key operands read AT_SCORE_AHEAD multiplies ahead, each read kept
    // with its multiply)
    floatx16 s[2] = {floatx16{}, floatx16{}};
    {
      auto operand = [&](int j) {
        const int ks = j >> 1, half = j & 1;
        return ld_lds16(kst + 32 * half * AT_K_PITCH + k_off[ks & 3] + 128 * (ks >> 2));
      };
      u32x4 ring[AT_SCORE_AHEAD];
#pragma unroll
      for (int j = 0; j < AT_SCORE_AHEAD; j++) ring[j] = operand(j);
#pragma unroll
      for (int j = 0; j < 24; j++) {
        const int ks = j >> 1, half = j & 1;
        const u32x4 A = ring[j % AT_SCORE_AHEAD];
        if (j + AT_SCORE_AHEAD < 24) ring[j % AT_SCORE_AHEAD] = operand(j + AT_SCORE_AHEAD);
        s[half] = mfma32x32x16(as_bf16x8(A), as_bf16x8(qv[ks]), s[half]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // mask: keys past T, past the query's position (causal), or outside the
    // query's index set. A tile wholly visible to the wave (all dense tiles
    // but the last and the causal diagonal) needs no mask.
    const bool all_visible =
        !SPARSE && t0 + AT_KT <= p.T && (!CAUSAL || t0 + AT_KT - 1 <= shift + qw);
    if (!all_visible) {
#pragma unroll
      for (int half = 0; half < 2; half++) {
        uint32_t bits = 0xFFFFu;
        if (SPARSE) {
          const uint32_t* ms =
              reinterpret_cast<const uint32_t*>(at_lds + AT_M0 + (it % AT_NK) * AT_M_BYTES) +
              half * AT_QBLOCK;
          bits = (ms[32 * wave + n] >> (16 * g)) & 0xFFFFu;
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int t = t0 + 32 * half + 16 * g + r;
          bool vis = t < p.T;
          if (CAUSAL) vis = vis && t <= qpos;
          if (SPARSE) vis = vis && ((bits >> r) & 1u);
          s[half][r] = vis ? s[half][r] : -INFINITY;
        }
      }
    }
    // one running-max update per 64-key tile, in the log2 domain; the scale
    // is positive, so the max of the scaled scores is the scaled max. The max
    // is raised lazily (only when a score beats it by 2^8), so the output
    // accumulators are rescaled only then; weights stay below 2^8.
    float smax = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; half++)
#pragma unroll
      for (int r = 0; r < 16; r++) smax = fmaxf(smax, s[half][r]);
    const float tmax = half_max(smax) * sl2;
    const bool rescaled = __any(tmax > m + AT_SLACK);
    const float m_new = rescaled ? fmaxf(m, tmax) : m;
    // a query that has seen no visible key yet keeps m = -inf: factor 1,
    // weights exp2(-inf) = 0
    if (rescaled) {
      const float f = m_new != -INFINITY ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
      l *= f;
#pragma unroll
      for (int mt = 0; mt < 4; mt++) o[mt] *= f;
    }
    m = m_new;
    const float nm = m != -INFINITY ? -m : 0.f;
#pragma unroll
    for (int half = 0; half < 2; half++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
#pragma unroll
        for (int w2 = 0; w2 < 4; w2++) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[half][8 * kk + 2 * w2], sl2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[half][8 * kk + 2 * w2 + 1], sl2, nm));
          P[half][kk][w2] = pack_bf16x2(p0, p1);
          // the denominator sums the rounded weights the mix uses
          l += __uint_as_float(P[half][kk][w2] << 16) +
               __uint_as_float(P[half][kk][w2] & 0xFFFF0000u);
        }
      }
    if (late)
      pending = true;
    else
      mix(P, at_lds + AT_V0 + (it % AT_NV) * AT_V_BYTES);
  }
  if (late && pending) mix(P, at_lds + AT_V0 + ((ntiles - 1) % AT_NV) * AT_V_BYTES);

  // ---- epilogue: normalise, write out and the log-sum-exp ----
  const float l_tot = half_sum(l);
  if (!wave_live || q >= p.S) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;  // no visible key: zero output
  uint16_t* dst = static_cast<uint16_t*>(p.out) +
                  ((static_cast<int64_t>(b) * p.S + q) * p.n_h + h) * AT_DV + 16 * g;
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    u32x4 v0, v1;
#pragma unroll
    for (int w2 = 0; w2 < 4; w2++) {
      v0[w2] = pack_bf16x2(o[mt][2 * w2] * inv, o[mt][2 * w2 + 1] * inv);
      v1[w2] = pack_bf16x2(o[mt][8 + 2 * w2] * inv, o[mt][8 + 2 * w2 + 1] * inv);
    }
    st16(dst + 32 * mt, v0);
    st16(dst + 32 * mt + 8, v1);
  }
  if (g == 0 && p.lse)
    p.lse[(static_cast<int64_t>(b) * p.S + q) * p.n_h + h] =
        l_tot > 0.f ? (m + log2f(l_tot)) * AT_LN2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// index sets -> bit mask: word (b, t/32, s), bit t%32 set iff t is in the
// set of query s. Entries outside [0, T) are ignored; repeats set the same bit.
__global__ __launch_bounds__(256) void mask_clear_kernel(uint32_t* __restrict__ m, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    m[i] = 0u;
}

__global__ __launch_bounds__(256) void mask_scatter_kernel(const int32_t* __restrict__ idx, int S,
                                                           int64_t rows, int K, int T, int words,
                                                           int s_pad, uint32_t* __restrict__ m) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t n = rows * K;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int64_t row = i / K;  // b * S + s
    const int64_t bb = row / S, ss = row - bb * S;
    const int t = idx[i];
    if (t < 0 || t >= T) continue;
    atomicOr(m + (bb * words + (t >> 5)) * s_pad + ss, 1u << (t & 31));
  }
}

// ---------------------------------------------------------------------------
// fp32: one block of 256 threads per (query, head, sequence)
__global__ __launch_bounds__(256) void attention_f32_kernel(AttnParams p) {
  __shared__ float qs[AT_DQK];
  __shared__ float ps[256];
  __shared__ float red[8];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t row = (static_cast<int64_t>(b) * p.S + s) * p.n_h + h;
  const float* qp = static_cast<const float*>(p.q) + row * AT_DQK;
  for (int c = tid; c < AT_DQK; c += 256) qs[c] = qp[c];
  const float* kb = static_cast<const float*>(p.k);
  const float* vb = static_cast<const float*>(p.v);
  const int64_t kstride = static_cast<int64_t>(p.n_h) * AT_DQK;
  const int64_t vstride = static_cast<int64_t>(p.n_h) * AT_DV;
  const int qpos = p.T - p.S + s;
  const uint32_t* mcol = p.mask ? p.mask + static_cast<int64_t>(b) * p.mask_words * p.s_pad + s
                                : nullptr;
  const int kend = p.causal ? min(p.T, qpos + 1) : p.T;
  __syncthreads();
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int r0 = 0; r0 < kend; r0 += 256) {
    const int t = r0 + tid;
    float z = -INFINITY;
    if (t < kend && (!mcol || ((mcol[static_cast<int64_t>(t >> 5) * p.s_pad] >> (t & 31)) & 1u))) {
      const float* kr = kb + (static_cast<int64_t>(b) * p.T + t) * kstride + h * AT_DQK;
      float d = 0.f;
      for (int c = 0; c < AT_DQK; c++) d = fmaf(qs[c], kr[c], d);
      z = p.scale * d;
    }
    float v = z;
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const float tmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m, tmax);
    const float f = m_new != -INFINITY ? expf(m - m_new) : 1.f;
    const float pv = z != -INFINITY ? expf(z - m_new) : 0.f;
    ps[tid] = pv;
    float sv = pv;
    for (int o = 32; o > 0; o >>= 1) sv += __shfl_xor(sv, o);
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = sv;
    __syncthreads();
    l = l * f + (red[4] + red[5] + red[6] + red[7]);
    acc *= f;
    m = m_new;
    const int nr = min(256, kend - r0);
    if (tid < AT_DV)
      for (int j = 0; j < nr; j++)
        if (ps[j] != 0.f)
          acc = fmaf(ps[j], vb[(static_cast<int64_t>(b) * p.T + r0 + j) * vstride + h * AT_DV + tid],
                     acc);
    __syncthreads();
  }
  if (tid < AT_DV) static_cast<float*>(p.out)[row * AT_DV + tid] = l > 0.f ? acc / l : 0.f;
  if (tid == 0 && p.lse) p.lse[row] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

int attention_query_block() { return AT_QBLOCK; }
int attention_key_tile() { return AT_KT; }

hipError_t launch_attention(AttnParams p, const int32_t* idx, int K, bool is_bf16,
                            hipStream_t stream) {
  if (idx) {
    const int64_t words = static_cast<int64_t>(p.B) * p.mask_words * p.s_pad;
    const int64_t cb = std::min<int64_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(mask_clear_kernel, dim3(static_cast<unsigned>(cb)), dim3(256), 0, stream,
                       p.mask, words);
    const int64_t n = static_cast<int64_t>(p.B) * p.S * K;
    const int64_t sb = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(mask_scatter_kernel, dim3(static_cast<unsigned>(sb)), dim3(256), 0, stream,
                       idx, p.S, static_cast<int64_t>(p.B) * p.S, K, p.T, p.mask_words, p.s_pad,
                       p.mask);
  } else {
    p.mask = nullptr;
  }
  if (is_bf16) {
    const int64_t grid = static_cast<int64_t>(p.nqb) * p.n_h * p.B;
    auto kern = p.causal ? (idx ? attention_bf16_kernel<true, true> : attention_bf16_kernel<true, false>)
                         : (idx ? attention_bf16_kernel<false, true> : attention_bf16_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * AT_WAVES), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attention_f32_kernel, dim3(p.S, p.n_h, p.B), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
