/*
 * mla.h — C ABI of libmla.so: multi-head latent attention (MLA) decode over a
 * compressed KV cache, and the literal wkv_b key/value reconstruction, on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for the operations (web pages, cited by title and section):
 *   [KVR]  "KV Reconstruction" (DeepSeek-V3 study note): "How it works"
 *          (up-projection equations, absorb identities, scale 1/sqrt(192)),
 *          "Official code", "Watch-outs".
 *   [ABS]  "DeepSeek-V3.2-Exp · Absorb key weights": the absorb equation,
 *          "Explanation", and its MQA-decode code excerpt.
 *   [KVL]  "DeepSeek-V3.2-Exp · Key–value latent": the mla-init, mla-kv,
 *          linear (FP8 block scales) and rmsnorm code excerpts.
 *   [VUP]  "Value up-projection" (DeepSeek-V3.2-Exp atlas): in/out shapes,
 *          parameter table, "Explanation", prefill code excerpt.
 *   [DS3]  "DeepSeek V3" (inference notes): "Multi-Head Latent Attention"
 *          equations, "Decoupled RoPE" (cache size), inference data flow.
 *
 * Fixed dimensions (see [KVR] "How it works", [KVL] mla-init excerpt):
 *   d_c = 512 latent features (kv_lora_rank), d_R = 64 rotary features,
 *   d_h = 128 content ("nope") features per head = 128 value features.
 * wkv_b is always the [n_h*256, 512] matrix stored [out, in] ([VUP]
 * "Parameters"), viewed as [n_h][256][512]: rows 0..127 of each head are
 * W^UK and rows 128..255 are W^UV ([KVR] "Official code", [ABS] excerpt).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to caller-owned memory,
 *     row-major and densely packed unless a stride argument says otherwise.
 *     The library never allocates, frees or synchronises.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream). Inputs must stay valid until the work completes.
 *   - mla_dtype selects the element type of the floating-point tensors of a
 *     call: MLA_F32 (float) or MLA_BF16 (bfloat16 bits in uint16_t). All
 *     sums accumulate in fp32; bf16 results are rounded to nearest-even.
 *   - Arguments are checked on the host before anything is enqueued. A bad
 *     argument returns MLA_ERR_INVALID_ARG and a dimension or layout this
 *     build does not implement returns MLA_ERR_UNSUPPORTED; in both cases no
 *     HIP call is made. A failed launch returns MLA_ERR_HIP. The detail of
 *     the last failure on the calling thread is in mla_last_error().
 *   - A call whose batch/row count is zero is a no-op returning MLA_OK.
 *   - Pointers must be 16-byte aligned; element strides must keep every row
 *     16-byte aligned (multiples of 8 bf16 or 4 f32 elements).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad index count  */
  MLA_ERR_UNSUPPORTED = 2, /* dimension/stride/alignment not implemented    */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  MLA_ERR_HIP = 4          /* the HIP runtime reported an error at launch   */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Static, human-readable name of a status code. */
const char* mla_status_str(mla_status status);

/* Detail message of the last non-OK status returned on this thread
 * (static thread-local storage; "" if none). */
const char* mla_last_error(void);

/*
 * One-time FP8 block dequantisation of a weight ([KVL] linear excerpt: one
 * fp32 scale per 128x128 block of a 1-byte weight; [ABS] excerpt: wkv_b is
 * dequantised once and reused for decoding).
 *   w_fp8  [rows, cols] uint8, OCP E4M3 ("e4m3fn": bias 7, no infinities,
 *          S.1111.111 is NaN, max 448).
 *   scale  [ceil(rows/128), ceil(cols/128)] float32.
 *   w_bf16 [rows, cols] out: bf16( f32( decode(w[i,j]) * scale[i/128, j/128] ) )
 *          with the product rounded to fp32 and then to bf16, each to
 *          nearest-even. NaN codes produce a NaN (payload unspecified).
 * Requirements: cols % 16 == 0. rows == 0 or cols == 0 is a no-op.
 */
mla_status mla_dequant_fp8_block(const uint8_t* w_fp8, const float* scale,
                                 int64_t rows, int64_t cols, uint16_t* w_bf16,
                                 hipStream_t stream);

/*
 * Absorb W^UK into the content query ([ABS] equation and excerpt;
 * [KVR] "How it works", first absorb identity):
 *   q_lat[b,h,c] = sum_{d<128} q_nope[b,h,d] * wkv_b[h*256 + d, c]
 *   q_nope [B, n_h, 128], wkv_b [n_h*256, 512], q_lat [B, n_h, 512] (out);
 *   all of element type dt.
 */
mla_status mla_absorb_q(const void* q_nope, const void* wkv_b, void* q_lat,
                        int B, int n_h, mla_dtype dt, hipStream_t stream);

/*
 * Bytes of workspace mla_decode_latent_attn needs for these arguments
 * (K = 0 for dense attention over all T positions; num_splits as passed to
 * the decode call, 0 = automatic). Returns 0 when no workspace is needed,
 * and (size_t)-1 for arguments the decode call would reject.
 */
size_t mla_decode_workspace_bytes(int B, int n_h, int T, int K, int num_splits,
                                  mla_dtype dt);

/* The split count the decode call uses for num_splits == 0 (>= 1), or -1
 * for arguments the decode call would reject. */
int mla_decode_num_splits(int B, int n_h, int T, int K);

/*
 * Latent attention of the absorbed decode path, one query token per
 * sequence ([ABS] excerpt: scores against the latent and rotary caches,
 * index mask, softmax, probability-weighted latent; [KVR] "How it works":
 * rotary scores are added to the content scores; the scale is applied to
 * their sum):
 *   z[b,h,t]     = scale * ( sum_c q_lat[b,h,c] * latent[b,t,c]
 *                          + sum_r q_pe[b,h,r]  * rope[b,t,r] ),  t < T
 *   z[b,h,t]     = -inf for every h when topk_idx is given and t is not in
 *                  topk_idx[b, 0..K-1]
 *   p[b,h,:]     = softmax_t z[b,h,:]
 *   out_lat[b,h,c] = sum_t p[b,h,t] * latent[b,t,c]
 *   lse[b,h]     = log sum_t exp z[b,h,t]   (natural log; optional)
 *
 *   q_lat  [B, n_h, 512], q_pe [B, n_h, 64]            (dt)
 *   latent element (b,t,c) at latent[b*lat_bstride + t*lat_rstride + c]
 *   rope   element (b,t,r) at rope  [b*rope_bstride + t*rope_rstride + r]
 *          (dt; strides in elements). Two layouts are typical: separate
 *          latent [B_max,T_max,512] and rope [B_max,T_max,64] caches read as
 *          [:B, :T], or one packed [B,T,576] cache with latent = p,
 *          rope = p + 512 and both row strides 576.
 *   topk_idx  NULL for dense attention over all T positions (K ignored), or
 *          int32 [B, K], 1 <= K <= T, in any order: the positions the index
 *          mask leaves visible ([ABS] excerpt: 0 scattered into a -inf row).
 *          An entry outside [0, T) addresses no position and is ignored
 *          (e.g. -1 padding; no memory outside the cache is read); a
 *          sequence whose entries are all outside [0, T) gets the empty sum:
 *          out_lat = 0 and lse = -inf. The in-range entries of a row must be
 *          DISTINCT (as a top-k selection produces): each is gathered once,
 *          so a repeated position would be counted once per repeat. The
 *          naive path's mla_attention_naive, which stages the set as a bit
 *          mask, also accepts repeats.
 *   out_lat [B, n_h, 512] (dt, out), lse [B, n_h] float32 (out, or NULL).
 *   num_splits  number of partitions of the attended positions (0 = let the
 *          library choose; otherwise lo <= num_splits <= ceil(rows/32), where
 *          rows = T, or K with topk_idx, and lo = 1 dense, ceil(K/1024) with
 *          topk_idx). Results differ between split counts only by
 *          floating-point rounding.
 *   workspace  device memory of at least
 *          mla_decode_workspace_bytes(B, n_h, T, K, num_splits, dt) bytes
 *          (may be NULL when that is 0).
 * Requirements: n_h >= 1, T >= 1; lat_rstride >= 512, rope_rstride >= 64,
 *   row strides multiples of 8 (bf16) or 4 (f32) elements, batch strides
 *   >= 0 (0 shares one cache among all sequences).
 */
mla_status mla_decode_latent_attn(const void* q_lat, const void* q_pe,
                                  const void* latent, const void* rope,
                                  int64_t lat_bstride, int64_t lat_rstride,
                                  int64_t rope_bstride, int64_t rope_rstride,
                                  int B, int n_h, int T,
                                  const int32_t* topk_idx, int K, float scale,
                                  int num_splits, void* out_lat, float* lse,
                                  void* workspace, size_t ws_bytes,
                                  mla_dtype dt, hipStream_t stream);

/*
 * Latent attention with S_q query tokens per sequence: the token axis s of
 * the decode einsums ([ABS] excerpt: q [b,s,h,c] against the cache [b,t,c],
 * scores [b,s,h,t]). T counts the cached positions including the S_q new
 * tokens, which sit at positions T-S_q .. T-1 (append them first, e.g. with
 * mla_cache_append). For sequence b, token j < S_q, head h < n_h:
 *   z[b,j,h,t] = scale * (q_lat[b,j,h,:] . latent[b,t,:] + q_pe[b,j,h,:] . rope[b,t,:])
 * over t < T, with
 *   - topk_idx (int32 [B, K] or NULL): one index set per sequence shared by
 *     all tokens and heads ([ABS] excerpt: the mask has a singleton token
 *     axis); same contract as mla_decode_latent_attn;
 *   - causal != 0: token j sees only t <= T - S_q + j (the causal mask of
 *     the [VUP] prefill excerpt, for queries at the end of the cache);
 *     requires T >= S_q and dense attention (topk_idx NULL; otherwise
 *     MLA_ERR_UNSUPPORTED).
 *   p = softmax_t z, out_lat[b,j,h,:] = sum_t p * latent[b,t,:],
 *   lse[b,j,h] = log sum_t exp z (optional).
 * q_lat [B, S_q, n_h, 512], q_pe [B, S_q, n_h, 64], out_lat [B, S_q, n_h, 512]
 * (dt), lse [B, S_q, n_h] float32. Cache arguments, num_splits and the
 * workspace are those of mla_decode_latent_attn for n_h' = S_q * n_h query
 * rows: size the workspace with mla_decode_workspace_bytes(B, S_q * n_h, T,
 * K, num_splits, dt). S_q * n_h <= 65535. S_q == 1 with causal == 0 is
 * mla_decode_latent_attn. The S_q tokens of a sequence share one read of
 * each cache tile when S_q * n_h <= 128 (e.g. a tensor-parallel share of
 * the heads).
 */
mla_status mla_decode_latent_attn_multi(const void* q_lat, const void* q_pe, const void* latent,
                                        const void* rope, int64_t lat_bstride,
                                        int64_t lat_rstride, int64_t rope_bstride,
                                        int64_t rope_rstride, int B, int S_q, int n_h, int T,
                                        const int32_t* topk_idx, int K, int causal, float scale,
                                        int num_splits, void* out_lat, float* lse,
                                        void* workspace, size_t ws_bytes, mla_dtype dt,
                                        hipStream_t stream);

/*
 * Packed queries: q_lat in the attention kernel's operand order, which lets
 * each wave load the queries of one k-step as one contiguous KiB (with the
 * row layout every 64-lane query load touches 32 separate rows). bf16 only,
 * for S_q * n_h a multiple of 128. With R = S_q * n_h query rows per
 * sequence (row v = j * n_h + h for token j, head h) and G = R / 128, the
 * 16-byte slot
 *   ((((b * G + v / 128) * 4 + (v / 32) % 4) * 32 + k) * 64 + 32 * e + v % 32)
 * holds latent features 16k + 8e .. 16k + 8e + 7 of row v of sequence b
 * (k < 32, e < 2): the same B * R * 512 elements as the row layout.
 *   mla_absorb_q_packed: as mla_absorb_q for q_nope [B, S_q, n_h, 128],
 *     writing q_packed ([KVR] first absorb identity; [ABS] excerpt).
 *   mla_decode_latent_attn_packed: as mla_decode_latent_attn_multi with
 *     q_lat given packed (same workspace size).
 * Other dtypes or shapes return MLA_ERR_UNSUPPORTED.
 */
mla_status mla_absorb_q_packed(const void* q_nope, const void* wkv_b, void* q_packed, int B,
                               int S_q, int n_h, mla_dtype dt, hipStream_t stream);
mla_status mla_decode_latent_attn_packed(const void* q_packed, const void* q_pe,
                                         const void* latent, const void* rope,
                                         int64_t lat_bstride, int64_t lat_rstride,
                                         int64_t rope_bstride, int64_t rope_rstride, int B,
                                         int S_q, int n_h, int T, const int32_t* topk_idx, int K,
                                         int causal, float scale, int num_splits, void* out_lat,
                                         float* lse, void* workspace, size_t ws_bytes,
                                         mla_dtype dt, hipStream_t stream);

/*
 * The whole absorbed decode step in one call ([ABS] excerpt: absorb W^UK,
 * latent attention, W^UV): enqueues mla_absorb_q on B*S_q rows,
 * mla_decode_latent_attn_multi and mla_out_up on B*S_q rows, with q_lat and
 * out_lat kept in the workspace.
 *   q_nope [B, S_q, n_h, 128], q_pe [B, S_q, n_h, 64], wkv_b [n_h*256, 512],
 *   out [B, S_q, n_h, 128] (dt), lse [B, S_q, n_h] float32 or NULL; cache,
 *   topk_idx, causal, scale and num_splits as in mla_decode_latent_attn_multi.
 *   workspace: at least mla_decode_step_workspace_bytes(B, S_q, n_h, T, K,
 *   num_splits, dt) bytes ((size_t)-1 for arguments the call would reject).
 * Every argument is checked before the first kernel is enqueued.
 */
size_t mla_decode_step_workspace_bytes(int B, int S_q, int n_h, int T, int K, int num_splits,
                                       mla_dtype dt);
mla_status mla_decode_step(const void* q_nope, const void* q_pe, const void* wkv_b,
                           const void* latent, const void* rope, int64_t lat_bstride,
                           int64_t lat_rstride, int64_t rope_bstride, int64_t rope_rstride, int B,
                           int S_q, int n_h, int T, const int32_t* topk_idx, int K, int causal,
                           float scale, int num_splits, void* out, float* lse, void* workspace,
                           size_t ws_bytes, mla_dtype dt, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_decode_step with its workspace in a fixed device array of the library
 * instead of a caller buffer. Arguments and results are those of
 * mla_decode_step without workspace/ws_bytes; the kernels, and so the
 * results bit for bit, are the same.
 *   - The array holds 64 MiB (67108864 bytes) on each GPU the call runs on,
 *     reserved when the library's code is loaded there and held until the
 *     process ends. A call whose mla_decode_step_workspace_bytes exceeds it
 *     returns MLA_ERR_WORKSPACE before anything is enqueued (B = 32, n_h =
 *     128, T = 4096 needs about 40 MiB).
 *   - The call allocates and frees nothing. Its first call on a device
 *     looks up the array's address there (hipGetSymbolAddress, with the
 *     device current); make that first call outside graph capture.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or concurrent graph replays) race
 *     and give wrong results. Nothing in the array needs to start at zero:
 *     each call writes what it reads.
 */
mla_status mla_decode_step_noalloc(const void* q_nope, const void* q_pe, const void* wkv_b,
                                   const void* latent, const void* rope, int64_t lat_bstride,
                                   int64_t lat_rstride, int64_t rope_bstride,
                                   int64_t rope_rstride, int B, int S_q, int n_h, int T,
                                   const int32_t* topk_idx, int K, int causal, float scale,
                                   int num_splits, void* out, float* lse, mla_dtype dt,
                                   hipStream_t stream);

/*
 * W^UV after the probability-weighted sum ([KVR] "How it works", second
 * absorb identity, and "Watch-outs": attend on the latent, then W^UV;
 * [ABS] excerpt, last einsum; [VUP] "Explanation": value rows are 128..255
 * of each head's 256):
 *   out[b,h,d] = sum_c out_lat[b,h,c] * wkv_b[h*256 + 128 + d, c]
 *   out_lat [B, n_h, 512], wkv_b [n_h*256, 512], out [B, n_h, 128] (dt).
 */
mla_status mla_out_up(const void* out_lat, const void* wkv_b, void* out,
                      int B, int n_h, mla_dtype dt, hipStream_t stream);

/*
 * Literal ("naive") key/value reconstruction ([KVR] "How it works": k^C =
 * W^UK c, v^C = W^UV c, key = [k^C ; k^R]; [VUP] prefill excerpt: wkv_b,
 * view per head, split into k_nope and v, concatenate the broadcast k^R):
 *   kv[n,h,e] = sum_c wkv_b[h*256 + e, c] * c[n,c],   e < 256
 *   K[n,h,0:128]   = kv[n,h,0:128]
 *   K[n,h,128:192] = k_rope[n,0:64]   (an exact copy, shared by all heads)
 *   V[n,h,0:128]   = kv[n,h,128:256]
 *   c [N, 512], k_rope [N, 64], wkv_b [n_h*256, 512],
 *   K [N, n_h, 192] (out), V [N, n_h, 128] (out); all of element type dt.
 */
mla_status mla_kv_reconstruct(const void* c, const void* k_rope,
                              const void* wkv_b, void* K, void* V, int64_t N,
                              int n_h, mla_dtype dt, hipStream_t stream);

/*
 * Ordinary attention over reconstructed keys and values, the second half of
 * the naive path ([VUP] prefill excerpt: q = [q_nope ; q_pe] per head,
 * scores times the scale, plus the index mask of each query token and the
 * causal mask, softmax over keys, probability-weighted values; [KVR] "How it
 * works": the keys and values come from the reconstruction). Queries sit at
 * the end of the keys: query s is position T - S + s (T == S for a prefill
 * from an empty cache). For sequence b, query s < S, head h < n_h:
 *   z[t] = scale * q[b,s,h,:] . k[b,t,h,:],  t < T
 *   z[t] = -inf when topk_idx is given and t is not in topk_idx[b,s,0..K-1]
 *          (one set per query token; entries outside [0, T) are ignored and
 *          repeats count once: the set of the scatter), and when causal != 0
 *          and t > T - S + s
 *   out[b,s,h,:] = sum_t softmax_t(z) v[b,t,h,:];  lse[b,s,h] = log sum_t exp z
 *   A query with no visible key gets out = 0 and lse = -inf.
 *   q [B, S, n_h, 192], k [B, T, n_h, 192], v [B, T, n_h, 128] (the layouts
 *   mla_kv_reconstruct writes for N = B*T tokens), out [B, S, n_h, 128] (dt),
 *   lse [B, S, n_h] float32 or NULL, topk_idx int32 [B, S, K] or NULL.
 *   workspace: mla_attention_naive_workspace_bytes(B, S, T, K) bytes (0, and
 *   NULL allowed, without index sets): one bit per (query, key).
 * Requirements: T >= 1, 1 <= K <= T with index sets, T >= S when causal.
 */
size_t mla_attention_naive_workspace_bytes(int B, int S, int T, int K);
mla_status mla_attention_naive(const void* q, const void* k, const void* v, int B, int S, int T,
                               int n_h, const int32_t* topk_idx, int K, int causal, float scale,
                               void* out, float* lse, void* workspace, size_t ws_bytes,
                               mla_dtype dt, hipStream_t stream);

/*
 * Cache append: the new tokens' entries of the compressed cache ([KVL]
 * "Key–value down-projection": the down-projection output is split into the
 * latent and the rotary key, the latent is normalised and the key rotated;
 * [KVL] "Key–value latent RMSNorm": float32 arithmetic, mean of squares,
 * per-feature gain, one cast back; [DS3] "Decoupled RoPE": the rotated key is
 * cached once per token and shared by all heads). For row n, with
 * x = kv_a[n, 0:512], k = kv_a[n, 512:576], s = seq_idx[n] (or n when
 * seq_idx is NULL), t = pos[n] and (cos_i, sin_i) = freqs[t, i, 0:2]:
 *   latent(s,t,c)    = gamma[c] * (x[c] * rsqrt(mean_c x[c]^2 + eps))
 *   rope(s,t,2i)     = k[2i] cos_i - k[2i+1] sin_i
 *   rope(s,t,2i+1)   = k[2i] sin_i + k[2i+1] cos_i,     i < 32
 * computed in fp32 and rounded once to dt. The rotation of consecutive
 * feature pairs by a caller-supplied per-position angle table is this
 * library's reading of the rotary step, whose body the pages do not show.
 *   kv_a    [N, in_rstride] (dt): 576 used features per row.
 *   gamma   [512] float32, freqs [n_pos, 32, 2] float32 (cos, sin).
 *   seq_idx [N] int32 or NULL; pos [N] int32.
 *   latent element (s,t,c) at latent[s*lat_bstride + t*lat_rstride + c],
 *   rope   element (s,t,r) at rope  [s*rope_bstride + t*rope_rstride + r]
 *          (dt; the layouts mla_decode_latent_attn reads, packed [.,576]
 *          included).
 * Rows whose (s, t) lies outside [0, B_cache) x [0, min(T_cache, n_pos))
 * are skipped on the device (nothing is written for them). Two rows with
 * the same (s, t) in one call race. Other cache rows are not touched.
 * Requirements: in_rstride >= 576, lat_rstride >= 512, rope_rstride >= 64,
 *   strides multiples of 8 (bf16) or 4 (f32) elements, eps >= 0;
 *   N <= B_cache when seq_idx is NULL.
 */
mla_status mla_cache_append(const void* kv_a, int64_t in_rstride, const float* gamma, float eps,
                            const float* freqs, int n_pos, const int32_t* seq_idx,
                            const int32_t* pos, int64_t N, void* latent, void* rope,
                            int64_t lat_bstride, int64_t lat_rstride, int64_t rope_bstride,
                            int64_t rope_rstride, int B_cache, int T_cache, mla_dtype dt,
                            hipStream_t stream);

/*
 * mla_softmax_scale — the attention scale to pass as `scale` to
 * mla_decode_latent_attn ([KVL] mla-init excerpt): qk_head_dim^(-1/2)
 * (192 here: 128 content + 64 rotary features), and, when the model runs
 * past its original context (max_seq_len > original_seq_len), multiplied by
 * mscale_eff^2 with mscale_eff = 0.1 * mscale * ln(rope_factor) + 1 (the YaRN
 * extension). Pure host arithmetic in double, rounded to float; no GPU call.
 * Returns NaN if qk_head_dim <= 0, or if the extension applies and
 * rope_factor <= 0.
 */
float mla_softmax_scale(int qk_head_dim, int64_t max_seq_len, int64_t original_seq_len,
                        float mscale, float rope_factor);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
