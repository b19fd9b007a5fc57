// decode.hip — latent attention of the absorbed MLA decode path.
//
// Operation ("DeepSeek-V3.2-Exp · Absorb key weights", decode excerpt;
// "KV Reconstruction", How it works):
//   z[b,h,t] = scale * (q_lat[b,h,:] . latent[b,t,:] + q_pe[b,h,:] . rope[b,t,:])
//   z = -inf at positions outside the top-k set (one set per sequence, shared
//   by all heads), p = softmax_t z, out_lat[b,h,:] = sum_t p[b,h,t] latent[b,t,:]
//
// bf16 kernel (the hot path). One workgroup of 8 waves (2 per SIMD) per
// (sequence, group of 128 heads, split of the attended rows). The workgroup
// streams its rows in 32-row tiles (latent 512 + rotary 64 features) from HBM
// into LDS with buffer_load ... lds (double-buffered: the next tile is in
// flight while the current one is consumed), so each cached byte is read
// from HBM once and shared by all 128 heads. LDS read bandwidth, not MFMA,
// is the scarce resource on gfx950, so the work is split to maximise reuse
// of every LDS read:
//   scores   wave (hq, kh) computes the partial S^T[32 rows x 32 heads]
//            of head quarter hq over feature half kh (18 k-steps of
//            v_mfma_f32_32x32x16_bf16; A = cache rows via ds_read_b128,
//            B = its queries, held in registers). The two halves meet in LDS.
//   softmax  the kh = 1 wave of each pair owns the online softmax of its 32
//            heads: each lane holds one head and 16 rows, so a tile max is 15
//            in-lane maxima plus one cross-half exchange; the running max is
//            raised lazily (only when a row beats it by 2^8), keeping the
//            accumulator rescale off the common path. It publishes P (bf16,
//            already in MFMA operand layout) and any rescale factors.
//   mix      wave w owns latent features 64w..64w+63 of all 128 heads:
//            O^T[64 x 128] += C^T[64 x 32 rows] . P^T[32 rows x 128 heads],
//            16 MFMAs whose A operand (read with ds_read_b64_tr_b16, the
//            gfx950 transposing LDS load) is reused across 4 head tiles.
// Row and feature permutations (pi, tau) make each lane's score
// accumulators 16 consecutive rows (exactly the P^T operand layout) and its
// output accumulators 16 consecutive latent features (32-byte stores). LDS
// tiles are XOR-swizzled per row (swz_lat / swz_rope) so the 16-byte score
// reads and the transposing reads hit distinct banks.
//
// Splits: with S > 1 each split writes its normalised partial output (bf16)
// and log-sum-exp to the workspace and a merge kernel combines them:
//   lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * out_s.
//
// fp32 kernel: a plain per-(sequence, head, split) VALU kernel used for the
// float32 interface (a correctness path, not a performance path).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "merge.hpp"

namespace mla {

constexpr int TILE = 32;                          // rows per tile
constexpr int NWAVES = 8;                         // waves per workgroup
constexpr int LAT_PITCH = 68 * 16;                // bytes per latent row in LDS
constexpr int LAT_BYTES = TILE * LAT_PITCH;       // 34 KiB latent region
constexpr int ROPE_BYTES = TILE * D_R * 2;        // 4 KiB rotary region
constexpr int BUF_BYTES = LAT_BYTES + ROPE_BYTES; // one staged tile
constexpr int NBUF = 3;                           // tiles in LDS (2 in flight)
constexpr int MAX_SPARSE_ROWS = 1024;             // staged top-k indices per split
constexpr int QK_P_STEPS = 21;                    // latent k-steps of the partner wave
constexpr int QK_O_STEPS = D_C / 16 - QK_P_STEPS; // latent k-steps of the owner wave
constexpr int QK_ROPE_STEPS = D_R / 16;           // 4 rotary k-steps (partner wave)
#ifndef MLA_P_RING
#define MLA_P_RING 2
#endif
#ifndef MLA_O_RING
#define MLA_O_RING 2
#endif
constexpr int P_RING = MLA_P_RING;  // tile-operand read-ahead of the partner's k-steps
constexpr int O_RING = MLA_O_RING;  // and of the owner's
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units


// LDS tile layout.
// Latent: row r occupies a 68-chunk (1088-byte) slot and its 64 data chunks
// start at chunk lat_shift(r) of the slot. With 64 four-byte banks a 16-byte
// chunk at slot chunk position x of row r lands in bank quarter
// (4r + x) mod 16, so:
//   * a 16-byte score read (16 lanes, rows {0..3,16..19,4..7,20..23} or the
//     +8 set, one chunk) hits 16 distinct quarters, and
//   * a transposing read (4 consecutive rows x 4 consecutive chunks) does too,
// while every address stays affine in the tile coordinates (one base register
// per lane plus instruction immediates).
// Rotary: rows of 8 chunks, chunk index XOR-swizzled by swz_rope (row parity
// supplies the 4th bit); only the score reads touch it, one row per lane.
__device__ __forceinline__ int lat_shift(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }
__device__ __forceinline__ int swz_rope(int r) {
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
}
// Score A-operand row i reads tile row pi(i): accumulator r of lane half g is
// then tile row 16g + r.
__device__ __forceinline__ int pi_row(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// Mix A-operand rows come in blocks of 4 latent features; block beta holds
// features 4*tau(beta)..+3 of a 32-feature tile, so accumulator r of lane
// half g is feature 16g + r.
__device__ __forceinline__ int tau_blk(int beta) { return 4 * (beta & 1) + (beta >> 1); }

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ bf16x8 tr_pair(const char* lo, const char* hi) {
  const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lo));
  const shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(hi));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// dma16 with the non-temporal hint, for rows that are read once and not again
// soon (a decode step's cache tiles).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16nt(i32x4 rsrc, uint32_t lds_dst, uint32_t voff,
                                        uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Staging of rows [row0, row0+32) of this split into the LDS tile at byte
// address `dst` by NW waves (w = 0..NW-1), one instruction per call: step
// k < 32/NW stages latent row NW*k + w (64 chunks of 16 bytes; the row's
// global offset is a scalar); step 32/NW stages the rotary rows 8w..8w+7
// (waves w < 4). Rows at or beyond row_end re-read row row_end-1 (their
// probabilities are zero). The loads carry the non-temporal hint: a step
// reads each cached row once (measured ~0.7 us per step at B=32, T=4096).
template <bool SPARSE, int NW>
__device__ __forceinline__ void stage_step(int k, i32x4 lat_d, i32x4 rope_d, uint32_t lat_rb,
                                           uint32_t rope_rb, const int* idx_lds, int row0,
                                           int row_end, int row_begin, uint32_t dst, int w,
                                           int lane) {
  const int valid = row_end - row0;
  if (k < TILE / NW) {
    const int R = NW * k + w;  // wave-uniform tile row
    const int Rc = R < valid ? R : valid - 1;
    uint32_t grow;
    if (SPARSE)
      grow = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(idx_lds[row0 - row_begin + Rc]));
    else
      grow = static_cast<uint32_t>(row0 + Rc);
    dma16nt(lat_d, dst + R * LAT_PITCH + 16 * lat_shift(R), static_cast<uint32_t>(lane * 16),
          __builtin_amdgcn_readfirstlane(grow * lat_rb));
  } else if (w < 4) {
    const int R = 8 * w + (lane >> 3);
    const int Rc = R < valid ? R : valid - 1;
    const uint32_t c = static_cast<uint32_t>((lane & 7) ^ swz_rope(R));
    uint32_t vo, so;
    if (SPARSE) {
      vo = static_cast<uint32_t>(idx_lds[row0 - row_begin + Rc]) * rope_rb + c * 16;
      so = 0;
    } else {
      vo = static_cast<uint32_t>(Rc) * rope_rb + c * 16;
      so = static_cast<uint32_t>(row0) * rope_rb;
    }
    dma16nt(rope_d, dst + LAT_BYTES + w * 1024, vo, __builtin_amdgcn_readfirstlane(so));
  }
}

// The whole staging of a tile by all NWAVES waves (prologue).
template <bool SPARSE>
__device__ __forceinline__ void issue_tile(i32x4 lat_d, i32x4 rope_d, uint32_t lat_rb,
                                           uint32_t rope_rb, const int* idx_lds, int row0,
                                           int row_end, int row_begin, uint32_t dst, int wave,
                                           int lane) {
#pragma unroll
  for (int k = 0; k <= TILE / NWAVES; k++)
    stage_step<SPARSE, NWAVES>(k, lat_d, rope_d, lat_rb, rope_rb, idx_lds, row0, row_end,
                               row_begin, dst, wave, lane);
}

// max / sum of a value over lanes l and l^32 (the two lane halves hold the
// same head), on the VALU: v_permlane32_swap exchanges the halves.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Partial scores S^T[32 rows x 32 heads] of one wave over its k-steps of a
// staged tile: NL latent k-steps from byte offset s_off of the tile (32 bytes
// per k-step), then, for the partner (ROPE), the 4 rotary k-steps. Query
// operands q[] are registers, the rotary ones (qpe_w) LDS. Tile operands are read RING k-steps ahead into
// distinct registers (an LDS round trip is several MFMA durations). With
// PINNED, sched_barrier keeps each (read ahead, multiply) pair in place;
// without, the scheduler may interleave other independent work (the owner's
// softmax) between them. hook(j) runs before multiply j (the owner issues
// its share of the tile DMA there).
template <int NL, bool ROPE, int RING, bool PINNED, class Hook>
__device__ __forceinline__ floatx16 partial_scores(const char* buf, int s_off, const bf16x8* q,
                                                   const u32x4* qpe_w, int lane, Hook&& hook) {
  constexpr int N = NL + (ROPE ? QK_ROPE_STEPS : 0);
  floatx16 sacc = {};
  const char* sp = buf + s_off;
  // rotary rows: chunk 2j+g of row pi(n), XOR-swizzled; recomputed here from
  // an opaque lane id rather than kept live across the tile loop
  const char* rp = buf;
  int r_x = 0;
  if (ROPE) {
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int srow = pi_row(lid & 31);
    rp = buf + LAT_BYTES + srow * 128;
    r_x = (lid >> 5) ^ swz_rope(srow);
  }
  auto operand = [&](int j) -> u32x4 {
    if (j < NL) return *reinterpret_cast<const u32x4*>(sp + 32 * j);
    return *reinterpret_cast<const u32x4*>(rp + (((2 * (j - NL)) ^ r_x) << 4));
  };
  u32x4 ring[RING];
#pragma unroll
  for (int j = 0; j < RING; j++) ring[j] = operand(j);
#pragma unroll
  for (int j = 0; j < N; j++) {
    const u32x4 a = ring[j % RING];
    if (j + RING < N) ring[j % RING] = operand(j + RING);
    // rotary query operands come from LDS (registers are full)
    const bf16x8 b = j < NL ? q[j] : as_bf16x8(qpe_w[(j - NL) * 64 + lane]);
    hook(j);
    sacc = mfma32x32x16(as_bf16x8(a), b, sacc);
    if (PINNED) __builtin_amdgcn_sched_barrier(0);
  }
  return sacc;
}

// FULL: every 128-head group holds 128 real heads (n_h % 128 == 0), which
// removes the code for head quarters without heads.
// CAUSAL (dense only): per-head visible row limit of multi-token queries.
template <bool FULL, bool CAUSAL>
__global__ __launch_bounds__(NWAVES * 64, 1) void decode_bf16_kernel(DecodeParams p) {
  constexpr bool SPARSE = false;  // top-k rows go to attend64_bf16_kernel
  __shared__ __attribute__((aligned(16))) char tiles[NBUF * BUF_BYTES];
  __shared__ __attribute__((aligned(16))) float sx[4 * 16 * 64];  // partner partial scores
  __shared__ __attribute__((aligned(16))) u32x4 qpe[4 * 4 * 64];  // rotary query operands
  __shared__ __attribute__((aligned(16))) u32x4 pb[4 * 2 * 64];   // P operands [hq][kk][lane]
  __shared__ float fac[128];                                       // rescale factor per head
  __shared__ __attribute__((aligned(16))) int flag[4];             // head quarter rescaled
  __shared__ float linv[128];                                      // 1 / sum per head
  const int* const idx_lds = nullptr;  // (no index rows: dense attention)

  // Workgroups are dealt to the 8 XCDs round-robin in launch order. Renumber
  // them so that the splits of one (sequence, head group) run on one XCD and
  // share its L2: the query rows they all read are then fetched once.
  int s, hg, b;
  {
    const int S = gridDim.x, HG = gridDim.y;
    const int G = S * HG * gridDim.z;
    const int L = blockIdx.x + S * (blockIdx.y + HG * blockIdx.z);
    const int j = (G & 7) == 0 ? (L & 7) * (G >> 3) + (L >> 3) : L;
    s = j % S;
    hg = (j / S) % HG;
    b = j / (S * HG);
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int hq = wave & 3, kh = wave >> 2;  // score role: head quarter, 0 partner / 1 owner
  const int head = hg * 128 + hq * 32 + n;  // score-role head of this lane
  const int headc = min(head, p.n_h - 1);   // clamped for loads

  const int row_begin = s * p.tiles_per_split * TILE;
  const int row_end = min(p.rows, row_begin + p.tiles_per_split * TILE);
  const int ntiles = (row_end - row_begin + TILE - 1) / TILE;
  // Rows [row_begin, row_vis) are visible to this lane's head. Heads are
  // numbered token * n_h_tok + head; with the causal limit, query token j
  // (position T - s_q + j) sees positions up to its own.
  const int row_vis = CAUSAL ? min(row_end, p.T - p.s_q + headc / p.n_h_tok + 1) : row_end;

  const i32x4 lat_d =
      make_rsrc(static_cast<const uint16_t*>(p.latent) + static_cast<int64_t>(b) * p.lat_bs);
  const i32x4 rope_d =
      make_rsrc(static_cast<const uint16_t*>(p.rope) + static_cast<int64_t>(b) * p.rope_bs);
  const uint32_t lat_rb = static_cast<uint32_t>(p.lat_rs * 2);  // row strides in bytes
  const uint32_t rope_rb = static_cast<uint32_t>(p.rope_rs * 2);
  const uint32_t tiles_addr = __builtin_amdgcn_readfirstlane(lds_addr(tiles));

  // prologue DMA of tile 0; the query loads that follow are waited for
  // (by the compiler) before the rest of the prologue DMA is issued
  issue_tile<SPARSE>(lat_d, rope_d, lat_rb, rope_rb, idx_lds, row_begin, row_end, row_begin,
                     tiles_addr, wave, lane);

  // per-lane LDS byte offsets inside a tile buffer (tile-independent)
  const int srow = pi_row(n);
  const int s_off = srow * LAT_PITCH + 16 * (lat_shift(srow) + g) + 32 * QK_P_STEPS * kh;
  int m_off;  // transposing reads: + 8704kk + 4368rd + 64mt
  {
    const int tau = tau_blk(4 * ((lane >> 4) & 1) + (lane & 3));
    const int row0 = 16 * g + ((lane & 15) >> 2);
    m_off = row0 * LAT_PITCH + 16 * (2 * g + (tau >> 1)) + 8 * (tau & 1) + 64 * 2 * wave;
  }
  const int64_t qrow = static_cast<int64_t>(b) * p.n_h + headc;
  // this lane's query operands: k-step ks is ql[16 * ks] (rows) or
  // ql[512 * ks] (operand order: one contiguous KiB per wave and k-step)
  const uint16_t* ql;
  int ql_step;
  if (FULL && p.q_swz) {
    ql = static_cast<const uint16_t*>(p.q_lat) +
         ((static_cast<int64_t>(b) * (p.n_h >> 7) + hg) * 4 + hq) * (32 * 512) + 8 * lane;
    ql_step = 512;
  } else {
    ql = static_cast<const uint16_t*>(p.q_lat) + qrow * D_C + 8 * g;
    ql_step = 16;
  }

  floatx16 acc[2][4];  // mix accumulators [feature tile][head tile]
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = floatx16{};
  float m = -INFINITY;  // owner waves: running max of scale*log2(e)*score
  float l = 0.f;        // owner waves: this lane's share of the running sum
  const float sl2 = p.scale * LOG2E;
  // head quarters of this group that hold real heads (n_h need not fill
  // 128): waves of the other quarters compute no scores and no softmax, and
  // the mix skips their head tiles; they still stage their share of tiles
  const int nact = FULL ? 4 : min(4, (p.n_h - hg * 128 + 31) >> 5);
  const bool active = FULL || hq < nact;

  // ---- software-pipelined tile loop ---------------------------------------------
  // Entering iteration it: the owner waves hold the complete scores S of tile
  // it; tile it and (if any) tile it+1 are in LDS or in flight. Per iteration:
  //   barrier A   tile it+1 resident, mix of tile it-1 done
  //   phase 1     owner: softmax(it) -> P, rescale factors; then its own
  //               partial scores of tile it+1 (registers), issuing between
  //               those multiplies the DMA of tile it+2 into tile it-1's buffer
  //               partner: partial scores of tile it+1 -> LDS
  //   barrier B
  //   phase 2     everyone: mix(it); owner: S of tile it+1 = own partial
  //               scores plus the partner's
  // The two roles run separate copies of the prologue and loop (kh is
  // wave-uniform) with their own query registers; both pass the same
  // barriers in the same order.
  // After the query registers have arrived (and with them tile 0): DMA of
  // tile 1 by all waves, then the barrier that publishes tile 0 (and the
  // staged rotary queries). In the loop only the owner waves stage tiles.
  auto tile0_wait = [&]() {
    if (threadIdx.x < 4) flag[threadIdx.x] = 0;
    if (ntiles > 1)
      issue_tile<SPARSE>(lat_d, rope_d, lat_rb, rope_rb, idx_lds, row_begin + TILE, row_end,
                         row_begin, tiles_addr + BUF_BYTES, wave, lane);
    // tile 0 resident (in practice already waited for with the queries)
    if (ntiles == 1)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (kh == 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(TILE / NWAVES) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(TILE / NWAVES + 1) : "memory");
    __syncthreads();
  };
  // Top of iteration it: tile it+1 resident (staged by the owners during
  // iteration it-1, or by everyone in the prologue) and every wave done with
  // tile it-1.
  auto top_of_tile = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto mix = [&](const char* buf) {
    const i32x4 fl = *reinterpret_cast<const i32x4*>(flag);
    if (fl[0] | fl[1] | fl[2] | fl[3]) {
#pragma unroll
      for (int nt = 0; nt < 4; nt++) {
        if (nt < nact && fl[nt]) {
          const float fn = fac[nt * 32 + n];
          acc[0][nt] *= fn;
          acc[1][nt] *= fn;
        }
      }
    }
    const char* mp = buf + m_off;
    bf16x8 A[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++)
        A[mt][kk] = tr_pair(mp + 8704 * kk + 64 * mt, mp + 8704 * kk + 4368 + 64 * mt);
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      if (nt >= nact) break;
      const bf16x8 B0 = as_bf16x8(pb[(nt * 2 + 0) * 64 + lane]);
      const bf16x8 B1 = as_bf16x8(pb[(nt * 2 + 1) * 64 + lane]);
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        acc[mt][nt] = mfma32x32x16(A[mt][0], B0, acc[mt][nt]);
        acc[mt][nt] = mfma32x32x16(A[mt][1], B1, acc[mt][nt]);
      }
    }
  };
  float4* const sx_w = reinterpret_cast<float4*>(sx) + hq * 256 + lane;

  if (!active) {
    // ======== waves of a head quarter without heads: staging and mix only ========
    tile0_wait();
    __syncthreads();  // (partner scores of tile 0 published)
    for (int it = 0; it < ntiles; it++) {
      top_of_tile();
      if (it + 2 < ntiles) {
        const uint32_t dst = tiles_addr + ((it + 2) % NBUF) * BUF_BYTES;
        const int srow0 = row_begin + (it + 2) * TILE;
#pragma unroll
        for (int j = 0; j < TILE / NWAVES; j++)
          stage_step<SPARSE, NWAVES>(j, lat_d, rope_d, lat_rb, rope_rb, idx_lds, srow0, row_end,
                                     row_begin, dst, wave, lane);
        if (kh == 1)  // the owners stage the rotary rows 8(wave-4)..+7
          stage_step<SPARSE, NWAVES>(TILE / NWAVES, lat_d, rope_d, lat_rb, rope_rb, idx_lds,
                                     srow0, row_end, row_begin, dst, wave - 4, lane);
      }
      __syncthreads();  // barrier B
      mix(tiles + (it % NBUF) * BUF_BYTES);
    }
  } else if (kh == 0) {
    // ======== partner waves: the first QK_P_STEPS latent k-steps and the rotary ones ==
    // query operands: k-step ks covers features 16ks..16ks+15, lane half g the
    // 8 at 16ks + 8g; rotary operands staged in LDS as [hq][k-step][lane]
    bf16x8 q[QK_P_STEPS];
#pragma unroll
    for (int j = 0; j < QK_P_STEPS; j++) q[j] = as_bf16x8(ld16(ql + ql_step * j));
    {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q_pe) + qrow * D_R + 8 * g;
#pragma unroll
      for (int j = 0; j < QK_ROPE_STEPS; j++) qpe[(hq * 4 + j) * 64 + lane] = ld16(qp + 16 * j);
    }
    // consume the loads here so the compiler's vmcnt waits stay out of the
    // tile loop (where they would also wait on tile DMA)
#pragma unroll
    for (int j = 0; j < QK_P_STEPS; j++) asm volatile("" : : "v"(q[j]));
    const u32x4* qpe_w = qpe + hq * 4 * 64;

    tile0_wait();
    {
      const floatx16 Sp = partial_scores<QK_P_STEPS, true, P_RING, true>(tiles, s_off, q, qpe_w, lane,
                                                                         [](int) {});
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++)
        sx_w[64 * j4] = make_float4(Sp[4 * j4], Sp[4 * j4 + 1], Sp[4 * j4 + 2], Sp[4 * j4 + 3]);
    }
    __syncthreads();  // partner scores of tile 0 published
    for (int it = 0; it < ntiles; it++) {
      top_of_tile();
      if (it + 1 < ntiles) {
        const char* buf = tiles + ((it + 1) % NBUF) * BUF_BYTES;
        floatx16 Sp;
        if (it + 2 < ntiles) {
          // this wave's share of the DMA of tile it+2 (latent rows 8k+wave)
          // between its multiplies; the owners stage the rest
          const uint32_t dst = tiles_addr + ((it + 2) % NBUF) * BUF_BYTES;
          const int srow0 = row_begin + (it + 2) * TILE;
          Sp = partial_scores<QK_P_STEPS, true, P_RING, true>(buf, s_off, q, qpe_w, lane,
                                                              [&](int j) {
            if (j < TILE / NWAVES)
              stage_step<SPARSE, NWAVES>(j, lat_d, rope_d, lat_rb, rope_rb, idx_lds, srow0,
                                         row_end, row_begin, dst, wave, lane);
          });
        } else {
          Sp = partial_scores<QK_P_STEPS, true, P_RING, true>(buf, s_off, q, qpe_w, lane,
                                                              [](int) {});
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; j4++)
          sx_w[64 * j4] = make_float4(Sp[4 * j4], Sp[4 * j4 + 1], Sp[4 * j4 + 2], Sp[4 * j4 + 3]);
      }
      __syncthreads();  // barrier B
      mix(tiles + (it % NBUF) * BUF_BYTES);
    }
  } else {
    // ======== owner waves: the last QK_O_STEPS latent k-steps and the softmax ========
    bf16x8 q[QK_O_STEPS];
#pragma unroll
    for (int j = 0; j < QK_O_STEPS; j++) q[j] = as_bf16x8(ld16(ql + ql_step * (QK_P_STEPS + j)));
#pragma unroll
    for (int j = 0; j < QK_O_STEPS; j++) asm volatile("" : : "v"(q[j]));

    tile0_wait();
    floatx16 S = partial_scores<QK_O_STEPS, false, O_RING, true>(tiles, s_off, q, nullptr, lane,
                                                                  [](int) {});
    __syncthreads();  // partner scores of tile 0 published
#pragma unroll
    for (int j4 = 0; j4 < 4; j4++) {
      const float4 o = sx_w[64 * j4];
      S[4 * j4] += o.x;
      S[4 * j4 + 1] += o.y;
      S[4 * j4 + 2] += o.z;
      S[4 * j4 + 3] += o.w;
    }
    for (int it = 0; it < ntiles; it++) {
      top_of_tile();
      // ---- phase 1: online softmax of tile it (log2 domain), then the own
      // partial scores of tile it+1 (on the last tile they read a stale
      // buffer and are discarded); the partner's multiplies fill the
      // SIMD's MFMA pipe meanwhile ----
      {
        const int valid = row_vis - (row_begin + it * TILE);  // visible rows of this tile
        // (without the causal limit only a split's last tile can be partial:
        // whole tiles skip the mask)
        if (CAUSAL || valid < TILE) {
#pragma unroll
          for (int r = 0; r < 16; r++) S[r] = 16 * g + r < valid ? S[r] : -INFINITY;
        }
      }
      float smax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r++) smax = fmaxf(smax, S[r]);
      // scale > 0, so the max of the scaled scores is the scaled max
      const float tmax = pair_max(smax * sl2);
      const bool rescaled = __any(tmax > m + RESCALE_SLACK);
      const float m_new = rescaled ? fmaxf(m, tmax) : m;
      // 0 on the first tile; a head that has seen no visible row yet (causal
      // limit) keeps m = -inf, factor 1 and weights exp2(-inf) = 0
      constexpr bool MAYBE_EMPTY = CAUSAL;
      const float f = rescaled && (!MAYBE_EMPTY || m_new != -INFINITY)
                          ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
      l *= f;
      m = m_new;
      const float nm = !MAYBE_EMPTY || m != -INFINITY ? -m : 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        u32x4 P;
#pragma unroll
        for (int w2 = 0; w2 < 4; w2++) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * kk + 2 * w2], sl2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * kk + 2 * w2 + 1], sl2, nm));
          P[w2] = pack_bf16x2(p0, p1);
          // the denominator sums the rounded weights the mix actually uses
          l += __uint_as_float(P[w2] << 16) + __uint_as_float(P[w2] & 0xFFFF0000u);
        }
        pb[(hq * 2 + kk) * 64 + lane] = P;
      }
      if (g == 0) fac[hq * 32 + n] = f;
      if (lane == 0) flag[hq] = rescaled;
      // Between its multiplies this wave stages its share of tile it+2
      // (latent rows 8k+wave and the rotary rows) into the buffer tile it-1
      // used (free since barrier A): the time an instruction waits to enter
      // the vector-memory pipeline then overlaps MFMAs instead of stalling
      // every wave after the barrier. The partner waves stage the other
      // latent rows.
      floatx16 Sn;
      {
        const char* buf = tiles + ((it + 1) % NBUF) * BUF_BYTES;
        if (it + 2 < ntiles) {
          const uint32_t dst = tiles_addr + ((it + 2) % NBUF) * BUF_BYTES;
          const int srow0 = row_begin + (it + 2) * TILE;
          Sn = partial_scores<QK_O_STEPS, false, O_RING, true>(buf, s_off, q, nullptr, lane,
                                                               [&](int j) {
            if (j < TILE / NWAVES)
              stage_step<SPARSE, NWAVES>(j, lat_d, rope_d, lat_rb, rope_rb, idx_lds, srow0,
                                         row_end, row_begin, dst, wave, lane);
            else if (j == TILE / NWAVES)  // the rotary rows 8(wave-4)..+7
              stage_step<SPARSE, NWAVES>(j, lat_d, rope_d, lat_rb, rope_rb, idx_lds, srow0,
                                         row_end, row_begin, dst, wave - 4, lane);
          });
        } else {
          Sn = partial_scores<QK_O_STEPS, false, O_RING, true>(buf, s_off, q, nullptr, lane,
                                                               [](int) {});
        }
      }
      __syncthreads();  // barrier B
      // ---- phase 2: mix of tile it; scores of tile it+1 completed ----
      mix(tiles + (it % NBUF) * BUF_BYTES);
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const float4 o = sx_w[64 * j4];
        S[4 * j4] = Sn[4 * j4] + o.x;
        S[4 * j4 + 1] = Sn[4 * j4 + 1] + o.y;
        S[4 * j4 + 2] = Sn[4 * j4 + 2] + o.z;
        S[4 * j4 + 3] = Sn[4 * j4 + 3] + o.w;
      }
    }
  }

  // ---- epilogue -----------------------------------------------------------------
  const int64_t BH = static_cast<int64_t>(p.B) * p.n_h;
  if (kh == 1 && active) {
    const float l_tot = pair_sum(l);
    // a head with no visible row in this split: zero partial, lse -inf
    if (g == 0) linv[hq * 32 + n] = !CAUSAL || l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (g == 0 && head < p.n_h) {
      const float lse_v = (m + log2f(l_tot)) * LN2;  // natural log of sum exp(z)
      const int64_t bh = static_cast<int64_t>(b) * p.n_h + head;
      if (p.num_splits == 1) {
        if (p.lse) p.lse[bh] = lse_v;
      } else {
        p.ws_lse[static_cast<int64_t>(s) * BH + bh] = lse_v;
      }
    }
  }
  __syncthreads();
  uint16_t* out_base = p.num_splits == 1
                           ? static_cast<uint16_t*>(p.out_lat)
                           : static_cast<uint16_t*>(p.ws_o) + static_cast<int64_t>(s) * BH * D_C;
  // The normalised rows go out in two halves of 64 heads staged in the (now
  // free) tile buffers: LDS row r holds head 64*half + r, its 16-byte chunk c
  // at position c ^ (r & 63), so that every store writes one whole 1 KB row,
  // non-temporally (64.3 -> 63.1 us per B=32 T=4096 step; the stores of the
  // 16-byte pieces of the MFMA layout were slower non-temporal, 68.3 us)
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int nt = 2 * half + t;
      const int r = 32 * t + n;  // stage row
      const float inv = linv[nt * 32 + n];
      char* const srow_p = tiles + r * (D_C * 2);
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        u32x4 v0, v1;
#pragma unroll
        for (int w2 = 0; w2 < 4; w2++) {
          v0[w2] = pack_bf16x2(acc[mt][nt][2 * w2] * inv, acc[mt][nt][2 * w2 + 1] * inv);
          v1[w2] = pack_bf16x2(acc[mt][nt][8 + 2 * w2] * inv, acc[mt][nt][8 + 2 * w2 + 1] * inv);
        }
        const int c0 = 8 * wave + 4 * mt + 2 * g;  // features 64 wave + 32 mt + 16 g
        *reinterpret_cast<u32x4*>(srow_p + ((c0 ^ (r & 63)) << 4)) = v0;
        *reinterpret_cast<u32x4*>(srow_p + (((c0 + 1) ^ (r & 63)) << 4)) = v1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 8 * wave + i;
      const int hr = hg * 128 + 64 * half + r;
      if (hr < p.n_h) {
        const u32x4 v = ld_lds16(tiles + r * (D_C * 2) + ((lane ^ (r & 63)) << 4));
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4*>(out_base + (static_cast<int64_t>(b) * p.n_h + hr) * D_C +
                                        8 * lane));
      }
    }
    if (half == 0) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for top-k rows, 64 heads per workgroup. A top-k split holds few
// rows (config B=8, K=2048: 128 per workgroup), so what a workgroup reads
// and writes besides its gathered rows matters: with 64 heads it loads half
// the queries and writes half the partial output of a 128-head workgroup,
// and the split merge reads half as much. (For dense rows the 128-head
// kernel above is faster: one wave per SIMD here leaves the LDS latency and
// the softmax exposed, which two waves per SIMD hide.)
// One workgroup of 4 waves (one per SIMD) per (sequence, group of 64 heads,
// split of the index rows). Each iteration stages 64 gathered rows (two
// 32-row halves, each laid out as a tile above) into one of two LDS buffers
// by LDS-DMA while the other is consumed; the rows of the iteration after
// that are touched once with plain loads so they are in flight to L2.
// Wave (ph, hb): head block hb (32 heads), row half ph.
//   scores   S^T[32 rows x 32 heads] of its row half in one 576-deep MFMA
//            chain (all 36 query k-steps of its heads held in registers);
//   softmax  the two row-half waves of a head block share one running max:
//            each publishes its tile maximum, both take the larger, so both
//            hold the same max and the same rescale decisions; each turns
//            its own rows into P (bf16, MFMA operand layout) and hands them
//            to the other through the rotary region of its half (free once
//            every wave's scores are done);
//   mix      O^T[256 x 32 heads] += C^T[256 x 64 rows] . P^T over latent
//            features [256 ph, 256 ph + 256) and both row halves.
// Three barriers per iteration: tile resident, maxima published, P
// published.
constexpr int A4_HEADS = 64;
constexpr int A4_WAVES = 4;
constexpr int A4_HALF = BUF_BYTES;       // 32 rows (latent + rotary)
constexpr int A4_ITER = 2 * BUF_BYTES;   // 64 rows
constexpr int A4_STEPS = TILE / A4_WAVES + 1;  // DMA instructions per wave and half
#ifndef MLA_A4_SRING
#define MLA_A4_SRING 4
#endif
#ifndef MLA_A4_PF_LOADS
#define MLA_A4_PF_LOADS 3
#endif
constexpr int A4_PF_LOADS = MLA_A4_PF_LOADS;  // L2 prefetch loads per wave and iteration
constexpr int A4_SRING = MLA_A4_SRING;  // score operands read ahead

__global__ __launch_bounds__(A4_WAVES * 64, 1) void attend64_bf16_kernel(DecodeParams p) {
  constexpr bool SPARSE = true;
  __shared__ __attribute__((aligned(16))) char tiles[2 * A4_ITER];
  __shared__ float xmax[A4_WAVES * 64];  // published tile maxima
  __shared__ int idx_lds[MAX_SPARSE_ROWS];
  // bit r of word k: row 32k + r of this split is a position of the index set
  __shared__ uint32_t vmask[MAX_SPARSE_ROWS / 32];

  // Workgroups are dealt to the 8 XCDs round-robin in launch order. Renumber
  // them so that the splits and head groups of one sequence run on one XCD:
  // the head groups of a split read the same rows, which the second then
  // finds in that XCD's L2.
  int s, hg, b;
  {
    const int S = gridDim.x, HG = gridDim.y;
    const int G = S * HG * gridDim.z;
    const int L = blockIdx.x + S * (blockIdx.y + HG * blockIdx.z);
    const int j = (G & 7) == 0 ? (L & 7) * (G >> 3) + (L >> 3) : L;
    s = j % S;
    hg = (j / S) % HG;
    b = j / (S * HG);
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ph = wave >> 1;      // row half of every iteration, and feature half of the mix
  const int hb = wave & 1;       // head block of the group
  const int hblk = hg * 2 + hb;  // global 32-head block
  const int head = hblk * 32 + n;
  const int headc = min(head, p.n_h - 1);

  const int row_begin = s * p.tiles_per_split * TILE;
  const int row_end = min(p.rows, row_begin + p.tiles_per_split * TILE);
  const int niter = (row_end - row_begin + 2 * TILE - 1) / (2 * TILE);

  const i32x4 lat_d =
      make_rsrc(static_cast<const uint16_t*>(p.latent) + static_cast<int64_t>(b) * p.lat_bs);
  const i32x4 rope_d =
      make_rsrc(static_cast<const uint16_t*>(p.rope) + static_cast<int64_t>(b) * p.rope_bs);
  const uint32_t lat_rb = static_cast<uint32_t>(p.lat_rs * 2);
  const uint32_t rope_rb = static_cast<uint32_t>(p.rope_rs * 2);
  const uint32_t tiles_addr = __builtin_amdgcn_readfirstlane(lds_addr(tiles));

  // queries of this lane's head (loaded below, with the index entries)
  const int64_t qrow = static_cast<int64_t>(b) * p.n_h + headc;
  bf16x8 q[D_QK / 16];
  {
    // The index set is a scatter into a -inf row: an entry outside [0, T)
    // addresses no position. Such entries are staged as row 0 (so every
    // fetch stays inside the cache) and cleared in vmask (weight zero).
    const int* src = p.idx + static_cast<int64_t>(b) * p.K + row_begin;
    const int n_rows = row_end - row_begin;
    // the first chunk of entries, then the queries: the query loads stay in
    // flight while the entries are checked and published, so their latency
    // overlaps the round trip of the entries
    const int v_first = static_cast<int>(threadIdx.x) < n_rows ? src[threadIdx.x] : -1;
    // queries of this lane's head: 32 latent k-steps (rows layout: features
    // 16ks + 8g of the row; operand order: one contiguous KiB per k-step and
    // 32-head block) and the 4 rotary k-steps
    {
      const uint16_t* ql;
      int step;
      if (p.q_swz) {
        ql = static_cast<const uint16_t*>(p.q_lat) +
             ((static_cast<int64_t>(b) * (p.n_h >> 7) + (hblk >> 2)) * 4 + (hblk & 3)) * (32 * 512) +
             8 * lane;
        step = 512;
      } else {
        ql = static_cast<const uint16_t*>(p.q_lat) + qrow * D_C + 8 * g;
        step = 16;
      }
#pragma unroll
      for (int j = 0; j < D_C / 16; j++) q[j] = as_bf16x8(ld16(ql + step * j));
      const uint16_t* qp = static_cast<const uint16_t*>(p.q_pe) + qrow * D_R + 8 * g;
#pragma unroll
      for (int j = 0; j < D_R / 16; j++) q[D_C / 16 + j] = as_bf16x8(ld16(qp + 16 * j));
    }
    for (int i0 = 0; i0 < n_rows; i0 += A4_WAVES * 64) {
      const int i = i0 + threadIdx.x;
      const int v = i0 == 0 ? v_first : (i < n_rows ? src[i] : -1);
      const bool ok = v >= 0 && v < p.T;
      if (i < n_rows) idx_lds[i] = ok ? v : 0;
      const uint64_t bal = __ballot(ok);
      if (lane == 0 && i < MAX_SPARSE_ROWS) {  // i is a multiple of 64 on lane 0
        vmask[i >> 5] = static_cast<uint32_t>(bal);
        vmask[(i >> 5) + 1] = static_cast<uint32_t>(bal >> 32);
      }
    }
    __syncthreads();
  }
  // DMA step k (0 .. 2*A4_STEPS-1) of this wave for iteration it: half
  // k / A4_STEPS, step k % A4_STEPS of that half. A half past the split's
  // rows is filled with copies of its last row: its weights are zero, and
  // the mix must not multiply them by stale (possibly non-finite) bytes.
  // With a zero-range descriptor (no next iteration) every load of a step is
  // out of range: nothing is fetched and zeros land in the free buffer, so
  // the steps need no branch between the score multiplies.
  i32x4 lat_z = lat_d, rope_z = rope_d;
  lat_z[2] = 0;
  rope_z[2] = 0;
  // Row indices of an iteration's staging and prefetch, read from idx_lds
  // in a few loads at the top of the iteration before the score multiplies:
  // an index read inside the multiply chain would make its wait (the LDS
  // counter is in order) wait for every tile operand read issued before it.
  //   lat   lane j < 16: the global row of latent step (half j / 8, k j % 8),
  //         i.e. tile row 4k + wave of that half (handed out by readlane);
  //   rope  the row of this lane's rotary chunk in half 0 / 1;
  //   pf    the row of this lane's prefetch line k.
  struct Rows {
    int lat, rope[2], pf[A4_PF_LOADS];
  };
  auto rows_of = [&](int it) {
    Rows r;
    auto grow = [&](int half, int R) {  // index-set row R of a half (clamped)
      const int row0 = min(row_begin + it * 2 * TILE + half * TILE, row_end - 1);
      const int valid = row_end - row0;
      return idx_lds[row0 - row_begin + (R < valid ? R : valid - 1)];
    };
    r.lat = grow((lane >> 3) & 1, 4 * (lane & 7) + wave);
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) r.rope[h2] = grow(h2, 8 * wave + (lane >> 3));
#pragma unroll
    for (int k = 0; k < A4_PF_LOADS; k++) {
      const int L = 64 * k + lane;
      const int row = min(row_begin + it * 2 * TILE + 16 * wave + min(L / 9, 15), row_end - 1);
      r.pf[k] = idx_lds[row - row_begin];
    }
    return r;
  };
  // DMA step k (0 .. 2*A4_STEPS-1) of this wave for iteration it into buffer
  // it & 1: half k / A4_STEPS; steps 0..7 of a half stage latent rows
  // 4k + wave, step 8 the rotary rows 8 wave .. 8 wave + 7 (8 lanes per row).
  // A half past the split's rows holds copies of its last row (weights zero;
  // the mix must not multiply them by stale, possibly non-finite, bytes).
  auto stage = [&](int it, int k, bool live, const Rows& r) {
    const int half = k / A4_STEPS, kk = k % A4_STEPS;
    i32x4 ld = lat_d, rd = rope_d;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      ld[e] = live ? lat_d[e] : lat_z[e];
      rd[e] = live ? rope_d[e] : rope_z[e];
    }
    const uint32_t dst = tiles_addr + (it & 1) * A4_ITER + half * A4_HALF;
    if (kk < TILE / A4_WAVES) {
      const int R = A4_WAVES * kk + wave;
      const uint32_t grow =
          static_cast<uint32_t>(__builtin_amdgcn_readlane(r.lat, half * 8 + kk));
      dma16(ld, dst + R * LAT_PITCH + 16 * lat_shift(R), static_cast<uint32_t>(lane * 16),
            __builtin_amdgcn_readfirstlane(grow * lat_rb));
    } else {
      const int R = 8 * wave + (lane >> 3);
      const uint32_t c = static_cast<uint32_t>((lane & 7) ^ swz_rope(R));
      dma16(rd, dst + LAT_BYTES + wave * 1024,
            static_cast<uint32_t>(r.rope[half]) * rope_rb + c * 16, 0);
    }
  };
  {
    const Rows r0 = rows_of(0);
#pragma unroll
    for (int k = 0; k < 2 * A4_STEPS; k++) stage(0, k, true, r0);
  }

  // L2 prefetch of iteration it: wave w touches the 9 lines (8 latent, 1
  // rotary) of rows [16w, 16w + 16) of that iteration with A4_PF_LOADS
  // 4-byte loads per lane (rows past the split re-read its last row). The
  // LDS buffers hold one iteration ahead; these loads put the next one in
  // flight too, so the staging DMA later finds its lines in L2. Their
  // values are only folded into `sink`, PF iterations later, when the
  // loads have long completed.
  const uint16_t* lat_b = static_cast<const uint16_t*>(p.latent) + static_cast<int64_t>(b) * p.lat_bs;
  const uint16_t* rope_b = static_cast<const uint16_t*>(p.rope) + static_cast<int64_t>(b) * p.rope_bs;
  auto prefetch = [&](int k, const Rows& r) -> uint32_t {
    const int L = 64 * k + lane;
    const int ln = L - (L / 9) * 9;
    const int row = r.pf[k];
    const uint16_t* a = ln < 8 ? lat_b + static_cast<int64_t>(row) * p.lat_rs + 64 * ln
                               : rope_b + static_cast<int64_t>(row) * p.rope_rs;
    return *reinterpret_cast<const uint32_t*>(a);
  };
  uint32_t pf_old[A4_PF_LOADS], pf_pend[A4_PF_LOADS];
#pragma unroll
  for (int k = 0; k < A4_PF_LOADS; k++) pf_old[k] = 0u;

  {
    const Rows r1 = rows_of(1);
#pragma unroll
    for (int k = 0; k < A4_PF_LOADS; k++) pf_pend[k] = prefetch(k, r1);
  }
  uint32_t sink = 0u;

  // per-lane LDS byte offsets inside a 32-row half (tile-independent)
  const int srow = pi_row(n);
  const int s_off = srow * LAT_PITCH + 16 * (lat_shift(srow) + g);
  const int r_off = LAT_BYTES + srow * 128;
  const int r_x = g ^ swz_rope(srow);
  int m_off;  // transposing reads of this wave's feature half
  {
    const int tau = tau_blk(4 * ((lane >> 4) & 1) + (lane & 3));
    const int row0 = 16 * g + ((lane & 15) >> 2);
    m_off = row0 * LAT_PITCH + 16 * (2 * g + (tau >> 1)) + 8 * (tau & 1) + 512 * ph;
  }

  constexpr int NFB = D_C / 2 / 32;  // 8 feature blocks of 32 per wave
  floatx16 O[NFB];                   // O^T accumulators: feature block, this lane's head
#pragma unroll
  for (int i = 0; i < NFB; i++) O[i] = floatx16{};
  float m = -INFINITY;  // running max of scale*log2(e)*score (shared with the other row half)
  float l = 0.f;        // this lane's share of the running sum (both row halves)
  const float sl2 = p.scale * LOG2E;
  constexpr int NKS = D_QK / 16;  // 36 k-steps

  for (int it = 0; it < niter; it++) {
    // buffer it & 1 complete (this wave's DMA, then everyone's; only the
    // A4_PF_LOADS prefetches issued after it may still be in flight); every
    // wave is done with iteration it-1, whose buffer the DMA of it+1
    // overwrites
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(A4_PF_LOADS) : "memory");
    __syncthreads();
    // prefetches issued two iterations ago have completed
#pragma unroll
    for (int k = 0; k < A4_PF_LOADS; k++) {
      sink ^= pf_old[k];
      pf_old[k] = pf_pend[k];
    }
    const bool next = it + 1 < niter;
    const int row0 = row_begin + it * 2 * TILE + ph * TILE;  // first row of this wave's half
    const char* buf = tiles + (it & 1) * A4_ITER;
    const char* half = buf + ph * A4_HALF;
    // ---- scores: one 36-deep chain; the DMA of the next iteration and the
    // L2 prefetch of the one after are issued between the first multiplies.
    // Lanes of heads past n_h compute on clamped heads (every wave runs the
    // same code; nothing of theirs is stored). ----
    // row indices of the next iteration's staging and of the prefetch after
    // it, before the first tile operand read
    const Rows rs = rows_of(it + 1);
    const Rows rp = rows_of(it + 2);
    floatx16 S;
    {
      // two accumulators (even and odd k-steps): consecutive multiplies are
      // independent, so the chain is not held to the latency of a multiply
      // that waits for the previous result (one wave per SIMD: nothing else
      // would fill the gap)
      floatx16 S2[2] = {floatx16{}, floatx16{}};
      auto operand = [&](int j) -> u32x4 {
        if (j < D_C / 16) return *reinterpret_cast<const u32x4*>(half + s_off + 32 * j);
        return *reinterpret_cast<const u32x4*>(half + r_off +
                                               (((2 * (j - D_C / 16)) ^ r_x) << 4));
      };
      u32x4 ring[A4_SRING];
#pragma unroll
      for (int j = 0; j < A4_SRING; j++) ring[j] = operand(j);
#pragma unroll
      for (int j = 0; j < NKS; j++) {
        const u32x4 a = ring[j % A4_SRING];
        if (j + A4_SRING < NKS) ring[j % A4_SRING] = operand(j + A4_SRING);
        if (j < 2 * A4_STEPS) stage(it + 1, j, next, rs);
        if (j >= 2 * A4_STEPS && j < 2 * A4_STEPS + A4_PF_LOADS)
          pf_pend[j - 2 * A4_STEPS] = prefetch(j - 2 * A4_STEPS, rp);
        S2[j & 1] = mfma32x32x16(as_bf16x8(a), q[j], S2[j & 1]);
        // keep each read-ahead with its multiply: the scheduler would
        // otherwise sink the reads next to their use and expose the LDS
        // latency on every k-step
        __builtin_amdgcn_sched_barrier(0);
      }
      S = S2[0] + S2[1];
    }
    // ---- this half's visible rows and its maximum ----
    {
      // rows of this lane: 16g..16g+15 of its half (rows past the split are
      // clear in vmask too)
      const int w = (row0 - row_begin) >> 5;
      const uint32_t bits = row0 < row_end ? vmask[w] >> (16 * g) : 0u;
#pragma unroll
      for (int r = 0; r < 16; r++) S[r] = (bits >> r) & 1u ? S[r] : -INFINITY;
    }
    float smax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) smax = fmaxf(smax, S[r]);
    // scale > 0, so the max of the scaled scores is the scaled max
    const float tmax_own = pair_max(smax * sl2);
    xmax[wave * 64 + lane] = tmax_own;
    __syncthreads();  // maxima published; every wave's scores are done
    const float tmax = fmaxf(tmax_own, xmax[(wave ^ 2) * 64 + lane]);
    const bool rescaled = __any(tmax > m + RESCALE_SLACK);
    const float m_new = rescaled ? fmaxf(m, tmax) : m;
    // 0 on the first visible rows; a head that has seen no visible row yet
    // keeps m = -inf, factor 1 and weights exp2(-inf) = 0
    const float f = rescaled && m_new != -INFINITY ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
    l *= f;
    m = m_new;
    const float nm = m != -INFINITY ? -m : 0.f;
    u32x4 Pown[2];
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
#pragma unroll
      for (int w2 = 0; w2 < 4; w2++) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * kk + 2 * w2], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * kk + 2 * w2 + 1], sl2, nm));
        Pown[kk][w2] = pack_bf16x2(p0, p1);
      }
    }
    // P of this half into its rotary region (read by the scores only)
    u32x4* const pw = reinterpret_cast<u32x4*>(const_cast<char*>(half) + LAT_BYTES);
    pw[hb * 128 + lane] = Pown[0];
    pw[hb * 128 + 64 + lane] = Pown[1];
    __syncthreads();  // P published
    const u32x4* const po =
        reinterpret_cast<const u32x4*>(buf + (1 - ph) * A4_HALF + LAT_BYTES) + hb * 128;
    u32x4 P[2][2];  // [row half][k-step]
    P[ph][0] = Pown[0];
    P[ph][1] = Pown[1];
    P[1 - ph][0] = po[lane];
    P[1 - ph][1] = po[64 + lane];
    // the denominator sums the rounded weights the mix actually uses
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++)
#pragma unroll
        for (int w2 = 0; w2 < 4; w2++)
          l += __uint_as_float(P[hh][kk][w2] << 16) +
               __uint_as_float(P[hh][kk][w2] & 0xFFFF0000u);
    // ---- mix: O^T[256 x 32 heads] += C^T[256 x 64 rows] . P^T; when the
    // running max was raised each block is rescaled right before its first
    // multiply (a second copy of the loop: the accumulators stay in the
    // registers the multiplies use) ----
    {
      auto mixop = [&](int fb, int hh, int kk) -> bf16x8 {
        const char* mp = buf + hh * A4_HALF + m_off + 8704 * kk + 64 * fb;
        return tr_pair(mp, mp + 4368);
      };
      // sub-step st = (block pair fp = st / 2, row half hh = st % 2): the four
      // multiplies (block 2fp, 2fp+1) x (k-step 0, 1) alternate between the
      // two blocks, so no multiply waits for the one just before it; the
      // operands of the next sub-step are read meanwhile
      auto mix = [&](auto rescale) {
        auto load4 = [&](int st, bf16x8 (&A)[4]) {
          const int fp = st >> 1, hh = st & 1;
#pragma unroll
          for (int c = 0; c < 4; c++) A[c] = mixop(2 * fp + (c & 1), hh, c >> 1);
        };
        bf16x8 A[2][4];
        load4(0, A[0]);
#pragma unroll
        for (int st = 0; st < 2 * NFB / 2; st++) {
          const int fp = st >> 1, hh = st & 1;
          if (st + 1 < NFB) load4(st + 1, A[(st + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          if (decltype(rescale)::value && hh == 0) {
#pragma unroll
            for (int i = 0; i < 2; i++) {
              floatx16 t = O[2 * fp + i] * f;
              // back into accumulation registers, so that the multiplies
              // (and so both copies of the loop) keep O in the same registers
              asm volatile("" : "+a"(t));
              O[2 * fp + i] = t;
            }
          }
#pragma unroll
          for (int c = 0; c < 4; c++)
            O[2 * fp + (c & 1)] =
                mfma32x32x16(A[st & 1][c], as_bf16x8(P[hh][c >> 1]), O[2 * fp + (c & 1)]);
        }
      };
      if (rescaled)
        mix(std::true_type{});
      else
        mix(std::false_type{});
    }
  }

  // the prefetched values are never needed; this keeps the loads (a sink
  // of all ones bits would need a cache of all-ones rows and a negative B)
  if (sink == 0xFFFFFFFFu && p.B < 0) p.lse[0] = 0.f;
  // ---- epilogue: normalise; the group's 64 partial rows are staged in LDS
  // (the tile buffers are free once every wave is past the barrier below),
  // so each store instruction writes whole 1 KB rows instead of 32 rows'
  // 32-byte pieces. Row r of the stage is the group's head r: 64 chunks of
  // 16 bytes, chunk c at position c ^ (r mod 64), which keeps the writes
  // (32 rows, one chunk each) and the reads (one row, all chunks) free of
  // bank conflicts. ----
  const float L = pair_sum(l);
  // a head with no visible row in this split: zero partial, lse -inf
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t BH = static_cast<int64_t>(p.B) * p.n_h;
  const int64_t bh = static_cast<int64_t>(b) * p.n_h + head;
  if (ph == 0 && g == 0 && head < p.n_h) {
    const float lse_v = (m + log2f(L)) * LN2;  // natural log of sum exp(z)
    if (p.num_splits == 1) {
      if (p.lse) p.lse[bh] = lse_v;
    } else {
      p.ws_lse[static_cast<int64_t>(s) * BH + bh] = lse_v;
    }
  }
  __syncthreads();  // every wave is done with the tile buffers
  {
    const int row = hb * 32 + n;
    char* const srow_p = tiles + row * (D_C * 2);
#pragma unroll
    for (int fb = 0; fb < NFB; fb++) {
      u32x4 v0, v1;
#pragma unroll
      for (int w2 = 0; w2 < 4; w2++) {
        v0[w2] = pack_bf16x2(O[fb][2 * w2] * inv, O[fb][2 * w2 + 1] * inv);
        v1[w2] = pack_bf16x2(O[fb][8 + 2 * w2] * inv, O[fb][8 + 2 * w2 + 1] * inv);
      }
      const int c0 = 32 * ph + 4 * fb + 2 * g;  // chunk of features 256 ph + 32 fb + 16 g
      *reinterpret_cast<u32x4*>(srow_p + ((c0 ^ (row & 63)) << 4)) = v0;
      *reinterpret_cast<u32x4*>(srow_p + (((c0 + 1) ^ (row & 63)) << 4)) = v1;
    }
  }
  __syncthreads();
  uint16_t* out_base = p.num_splits == 1
                           ? static_cast<uint16_t*>(p.out_lat)
                           : static_cast<uint16_t*>(p.ws_o) + static_cast<int64_t>(s) * BH * D_C;
#pragma unroll
  for (int i = 0; i < A4_HEADS / A4_WAVES; i++) {
    const int r = (A4_HEADS / A4_WAVES) * wave + i;  // stage row of this instruction
    const int hr = hg * A4_HEADS + r;
    if (hr < p.n_h) {
      const u32x4 v = ld_lds16(tiles + r * (D_C * 2) + ((lane ^ (r & 63)) << 4));
      // whole rows, non-temporal (the merge reads them from L2 or HBM either
      // way; measured ~0.45 us per B=8 top-2048 step)
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(out_base + (static_cast<int64_t>(b) * p.n_h + hr) * D_C +
                                      8 * lane));
    }
  }
}

// ---------------------------------------------------------------------------
// merge of split partials: one 64-lane block per (b, h), 8 features per lane
template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
__device__ __forceinline__ void st_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_elem(uint16_t* p, int64_t i, float v) {
  p[i] = float_to_bf16_bits(v);
}

template <typename T>
__global__ __launch_bounds__(64) void merge_splits_f32_kernel(const T* __restrict__ ws_o,
                                                          const float* __restrict__ ws_lse,
                                                          int S, int64_t BH, T* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  float mx = -INFINITY;
  for (int s = 0; s < S; s++) mx = fmaxf(mx, ws_lse[s * BH + bh]);
  float wsum = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int c0 = threadIdx.x * 8;
  for (int s = 0; s < S; s++) {
    // no split saw a position (every index outside [0, T)): the empty sum
    const float w = mx != -INFINITY ? __expf(ws_lse[s * BH + bh] - mx) : 0.f;
    wsum += w;
    const T* src = ws_o + (s * BH + bh) * D_C + c0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = fmaf(w, ld_elem<T>(src, i), acc[i]);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) st_elem(out, bh * D_C + c0 + i, acc[i] * inv);
  if (threadIdx.x == 0 && lse) lse[bh] = mx + logf(wsum);
}

// bf16 partials: 64 lanes per (b, h) row, 8 latent features (16 bytes) per
// lane, four rows per workgroup (the per-row arithmetic is merge_rows8).
// Rows of more than MERGE_SPLIT_PARTS_ABOVE splits: two rows per workgroup,
// wave (part, row) folds one of the row's two parts and the part-1 state
// meets part 0 in LDS (the arithmetic of merge_rows8 for such rows, so the
// same bits, with half the memory round trips per wave).
__global__ __launch_bounds__(256) void merge_splits_bf16_kernel(const uint16_t* __restrict__ ws_o,
                                                                const float* __restrict__ ws_lse,
                                                                int S, int64_t BH,
                                                                uint16_t* __restrict__ out,
                                                                float* __restrict__ lse) {
  __shared__ float xs[2][10][64];  // part-1 states (max, sum, 8 accumulators) of two rows
  const int lane = threadIdx.x & 63;
  const int c0 = lane * 8;
  if (S > MERGE_SPLIT_PARTS_ABOVE) {
    const int wave = threadIdx.x >> 6;
    const int part = wave >> 1, r = wave & 1;
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * 2 + r;
    const bool ok = bh < BH;
    float mx = -INFINITY, wsum = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
    if (ok)
      merge_chunks<true>(ws_o, ws_lse, S, BH, bh, c0, merge_part_begin(S, part),
                         merge_part_end(S, part), mx, wsum, acc);
    if (part == 1) {
      xs[r][0][lane] = mx;
      xs[r][1][lane] = wsum;
#pragma unroll
      for (int i = 0; i < 8; i++) xs[r][2 + i][lane] = acc[i];
    }
    __syncthreads();
    if (part == 0 && ok) {
      float a1[8], o8[8];
#pragma unroll
      for (int i = 0; i < 8; i++) a1[i] = xs[r][2 + i][lane];
      merge_combine2(mx, wsum, acc, xs[r][0][lane], xs[r][1][lane], a1);
      const float l = merge_finish(mx, wsum, acc, o8);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = pack_bf16x2(o8[2 * i], o8[2 * i + 1]);
      st16(out + bh * D_C + c0, o);
      if (lane == 0 && lse) lse[bh] = l;
    }
    return;
  }
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;
  float o8[1][8], l;
  merge_rows8<1, true>(ws_o, ws_lse, S, BH, &bh, c0, o8, &l);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) o[i] = pack_bf16x2(o8[0][2 * i], o8[0][2 * i + 1]);
  st16(out + bh * D_C + c0, o);
  if (lane == 0 && lse) lse[bh] = l;
}

// ---------------------------------------------------------------------------
// fp32 decode: one block of 256 threads per (b, h, split)
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeParams p) {
  __shared__ float qs[D_QK];
  __shared__ float ps[256];
  __shared__ int ts[256];
  __shared__ float red[8];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * p.n_h + h;
  const float* ql = static_cast<const float*>(p.q_lat) + bh * D_C;
  const float* qp = static_cast<const float*>(p.q_pe) + bh * D_R;
  for (int c = tid; c < D_QK; c += 256) qs[c] = c < D_C ? ql[c] : qp[c - D_C];
  const float* lat = static_cast<const float*>(p.latent) + static_cast<int64_t>(b) * p.lat_bs;
  const float* rp = static_cast<const float*>(p.rope) + static_cast<int64_t>(b) * p.rope_bs;
  const int row_begin = s * p.tiles_per_split * TILE;
  const int row_end_split = min(p.rows, row_begin + p.tiles_per_split * TILE);
  // head h = token * n_h_tok + head; causal: token j sees up to T - s_q + j
  const int row_end = (!p.idx && p.causal) ? min(row_end_split, p.T - p.s_q + h / p.n_h_tok + 1)
                                           : row_end_split;
  __syncthreads();

  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int r0 = row_begin; r0 < row_end; r0 += 256) {
    const int rr = r0 + tid;
    float t = -INFINITY;
    int tok = 0;
    // an index entry outside [0, T) addresses no position: weight zero,
    // and row 0 stands in for it in the mix
    bool live = rr < row_end;
    if (live && p.idx) {
      tok = p.idx[static_cast<int64_t>(b) * p.K + rr];
      live = tok >= 0 && tok < p.T;
      if (!live) tok = 0;
    } else if (live) {
      tok = rr;
    }
    if (live) {
      const float* lrow = lat + static_cast<int64_t>(tok) * p.lat_rs;
      const float* rrow = rp + static_cast<int64_t>(tok) * p.rope_rs;
      float content = 0.f, rotary = 0.f;
      for (int c = 0; c < D_C; c++) content = fmaf(qs[c], lrow[c], content);
      for (int c = 0; c < D_R; c++) rotary = fmaf(qs[D_C + c], rrow[c], rotary);
      t = p.scale * (content + rotary);
    }
    // block max
    float v = t;
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const float tmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m, tmax);
    const float f = m_new != -INFINITY ? expf(m - m_new) : 1.f;
    const float pv = live ? expf(t - m_new) : 0.f;
    ps[tid] = pv;
    ts[tid] = tok;
    float sv = pv;
    for (int o = 32; o > 0; o >>= 1) sv += __shfl_xor(sv, o);
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = sv;
    __syncthreads();
    l = l * f + (red[4] + red[5] + red[6] + red[7]);
    acc0 *= f;
    acc1 *= f;
    m = m_new;
    const int nr = min(256, row_end - r0);
    for (int j = 0; j < nr; j++) {
      const float* lrow = lat + static_cast<int64_t>(ts[j]) * p.lat_rs;
      acc0 = fmaf(ps[j], lrow[tid], acc0);
      acc1 = fmaf(ps[j], lrow[tid + 256], acc1);
    }
    __syncthreads();
  }
  float* dst;
  float* lse_dst;
  if (p.num_splits == 1) {
    dst = static_cast<float*>(p.out_lat) + bh * D_C;
    lse_dst = p.lse ? p.lse + bh : nullptr;
  } else {
    const int64_t sbh = static_cast<int64_t>(s) * p.B * p.n_h + bh;
    dst = static_cast<float*>(p.ws_o) + sbh * D_C;
    lse_dst = p.ws_lse + sbh;
  }
  // no visible row in this split (causal limit): zero partial, lse -inf
  const float linv = l > 0.f ? 1.f / l : 0.f;
  dst[tid] = acc0 * linv;
  dst[tid + 256] = acc1 * linv;
  if (tid == 0 && lse_dst) *lse_dst = m + logf(l);
}

hipError_t launch_decode(const DecodeParams& p, bool is_bf16, hipStream_t stream,
                         bool merge_splits) {
  if (is_bf16) {
    if (p.idx) {
      // top-k rows: 64-head workgroups (fewer query and partial bytes per
      // gathered row; see attend64_bf16_kernel)
      dim3 grid(p.num_splits, (p.n_h + A4_HEADS - 1) / A4_HEADS, p.B);
      hipLaunchKernelGGL(attend64_bf16_kernel, grid, dim3(A4_WAVES * 64), 0, stream, p);
    } else {
      dim3 grid(p.num_splits, (p.n_h + 127) / 128, p.B);
      const bool full = p.n_h % 128 == 0;
      auto kern = p.causal ? (full ? decode_bf16_kernel<true, true> : decode_bf16_kernel<false, true>)
                           : (full ? decode_bf16_kernel<true, false> : decode_bf16_kernel<false, false>);
      hipLaunchKernelGGL(kern, grid, dim3(NWAVES * 64), 0, stream, p);
    }
  } else {
    hipLaunchKernelGGL(decode_f32_kernel, dim3(p.num_splits, p.n_h, p.B), dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1 || !merge_splits) return e;
  const int64_t BH = static_cast<int64_t>(p.B) * p.n_h;
  if (is_bf16)
    hipLaunchKernelGGL(merge_splits_bf16_kernel,
                       dim3(static_cast<unsigned>(p.num_splits > MERGE_SPLIT_PARTS_ABOVE
                                                      ? (BH + 1) / 2 : (BH + 3) / 4)),
                       dim3(256), 0, stream, static_cast<const uint16_t*>(p.ws_o), p.ws_lse,
                       p.num_splits, BH, static_cast<uint16_t*>(p.out_lat), p.lse);
  else
    hipLaunchKernelGGL(merge_splits_f32_kernel<float>, dim3(static_cast<unsigned>(BH)), dim3(64), 0,
                       stream, static_cast<const float*>(p.ws_o), p.ws_lse, p.num_splits, BH,
                       static_cast<float*>(p.out_lat), p.lse);
  return hipGetLastError();
}

}  // namespace mla
