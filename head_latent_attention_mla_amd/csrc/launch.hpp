// launch.hpp — internal kernel launchers of libmla (arguments already checked).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

hipError_t launch_dequant_fp8_block(const uint8_t* w, const float* scale, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t stream);

// is_bf16: element type of q_nope / wkv_b / q_lat (else float32)
hipError_t launch_absorb_q(const void* q_nope, const void* wkv_b, void* q_lat, int B, int n_h,
                           bool is_bf16, hipStream_t stream);

// bf16: q_lat written in the decode's operand order (DecodeParams::q_swz = 1)
// for B / s_q sequences of s_q * n_h query rows each; requires
// (s_q * n_h) % 128 == 0
hipError_t launch_absorb_q_swizzled(const void* q_nope, const void* wkv_b, void* q_lat, int B,
                                    int n_h, int s_q, hipStream_t stream);

hipError_t launch_out_up(const void* o_lat, const void* wkv_b, void* out, int B, int n_h,
                         bool is_bf16, hipStream_t stream);

hipError_t launch_kv_reconstruct(const void* c, const void* k_rope, const void* wkv_b, void* K,
                                 void* V, int64_t N, int n_h, bool is_bf16, hipStream_t stream);

struct DecodeParams {
  const void* q_lat;
  const void* q_pe;
  const void* latent;
  const void* rope;
  int64_t lat_bs, lat_rs, rope_bs, rope_rs;  // element strides
  int B, n_h, T;        // n_h counts every query row of a sequence: s_q * n_h_tok
  int s_q, n_h_tok;     // query tokens per sequence, heads per token
  int causal;           // token j sees positions < T - s_q + j + 1 (dense only)
  const int32_t* idx;  // nullptr = dense
  int K;
  int rows;            // attended positions per sequence (T or K)
  int num_splits;
  int tiles_per_split; // 32-row tiles per split
  float scale;
  void* out_lat;
  float* lse;
  void* ws_o;          // [num_splits, B, n_h, 512] partial outputs (split > 1)
  float* ws_lse;       // [num_splits, B, n_h]
  // q_lat layout: 0 = [B, n_h, 512] rows; 1 = operand order (full 128-row
  // groups only): 16-byte slot ((((b * n_h/128 + hg) * 4 + hq) * 32 + ks) * 64
  // + lane) holds row hg*128 + hq*32 + (lane & 31), features 16ks + 8*(lane >> 5)
  int q_swz;
};

// merge_splits = false leaves the split partials in the workspace (for
// launch_merge_out_up)
hipError_t launch_decode(const DecodeParams& p, bool is_bf16, hipStream_t stream,
                         bool merge_splits = true);

// bf16 only: merge of S split partials ([S][B*n_h][512] + [S][B*n_h] lse)
// fused with W^UV; out [B, n_h, 128], lse [B*n_h] or nullptr
hipError_t launch_merge_out_up(const void* ws_o, const float* ws_lse, int S, const void* wkv_b,
                               void* out, float* lse, int B, int n_h, hipStream_t stream);

struct AppendParams {
  const void* kv_a;      // [N, in_rstride]: 512 latent then 64 rotary features
  int64_t in_rstride;    // elements
  const float* gamma;    // [512]
  float eps;
  const float* freqs;    // [n_pos, 32, 2] (cos, sin)
  int n_pos;
  const int32_t* seq_idx;  // [N] or nullptr (row n -> sequence n)
  const int32_t* pos;      // [N]
  int64_t N;
  void* latent;
  void* rope;
  int64_t lat_bs, lat_rs, rope_bs, rope_rs;  // element strides
  int B_cache, T_cache;
};

hipError_t launch_cache_append(const AppendParams& p, bool is_bf16, hipStream_t stream);

struct AttnParams {
  const void* q;     // [B, S, n_h, 192]
  const void* k;     // [B, T, n_h, 192]
  const void* v;     // [B, T, n_h, 128]
  void* out;         // [B, S, n_h, 128]
  float* lse;        // [B, S, n_h] or nullptr
  uint32_t* mask;    // [B, mask_words, s_pad] bits (index sets) or nullptr
  int B, S, T, n_h;
  int nqb;           // query blocks per (sequence, head)
  int mask_words;    // key words per sequence (a multiple of 2)
  int s_pad;         // nqb * query block
  float scale;
  int causal;
};

// queries per workgroup and keys per tile of the bf16 attention kernel
int attention_query_block();
int attention_key_tile();
hipError_t launch_attention(AttnParams p, const int32_t* idx, int K, bool is_bf16,
                            hipStream_t stream);

}  // namespace mla
