// capi.hip — the C ABI of libmla (declared in include/mla.h): host-side
// argument checks, split planning for the decode call, and kernel dispatch.
// Every check happens before the first HIP call; the library never
// allocates, frees or synchronises.
#include <climits>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <mutex>

#include "mla.h"
#include "common.hpp"
#include "launch.hpp"

using namespace mla;

namespace {

thread_local char g_last_error[512] = "";

mla_status fail(mla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

mla_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(mla_dtype dt) { return dt == MLA_F32 || dt == MLA_BF16; }

// Split plan of the decode call: rows are cut into 32-row tiles, splits get
// equal tile counts. Automatic choice: aim at one workgroup (nearly all of
// the LDS) per compute unit (256 on MI355X) without making any split empty.
// Dense rows: workgroups of 128 heads. Top-k rows: workgroups of 64 heads and
// splits of whole 64-row iterations.
constexpr int kTargetWorkgroups = 256;
constexpr int kMaxSplits = 1024;
// The top-k kernel stages one split's indices in LDS: at most 1024 rows.
constexpr int kMaxSparseTilesPerSplit = 1024 / 32;

int group_heads(bool sparse) { return sparse ? 64 : 128; }

struct SplitPlan {
  int num_splits;
  int tiles_per_split;
};

// requested == 0: automatic. Returns false for a split count outside
// [minimum, tiles] (the minimum is 1 dense, ceil(tiles/32) with top-k).
bool plan_splits(int B, int n_h, int rows, bool sparse, int requested, SplitPlan* out) {
  const int ntiles = (rows + 31) / 32;
  const int min_s = sparse ? (ntiles + kMaxSparseTilesPerSplit - 1) / kMaxSparseTilesPerSplit : 1;
  int tps;
  if (requested == 0) {
    const int gh = group_heads(sparse);
    const long base = static_cast<long>(B) * ((n_h + gh - 1) / gh);
    const int unit = sparse ? 2 : 1;  // tiles per iteration of the kernel
    const int nunits = (ntiles + unit - 1) / unit;
    long want = (kTargetWorkgroups + base - 1) / base;
    if (want < 1) want = 1;
    int s = static_cast<int>(want < nunits ? want : nunits);
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < min_s) s = min_s;
    // whole iterations; at most 32 tiles per split when s >= min_s
    tps = unit * ((nunits + s - 1) / s);
  } else {
    if (requested < min_s || requested > ntiles) return false;
    tps = (ntiles + requested - 1) / requested;
  }
  out->tiles_per_split = tps;
  out->num_splits = (ntiles + tps - 1) / tps;  // no empty split
  return true;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t ws_bytes_for(int B, int n_h, const SplitPlan& sp, mla_dtype dt) {
  if (sp.num_splits == 1) return 0;
  const size_t bh = static_cast<size_t>(B) * n_h * sp.num_splits;
  const size_t esz = dt == MLA_BF16 ? 2 : 4;
  return align256(bh * D_C * esz) + align256(bh * sizeof(float));
}

// decode argument checks shared by the size query and the call
mla_status check_decode_dims(int B, int n_h, int T, int K, bool sparse, int* rows) {
  if (B < 0) return fail(MLA_ERR_INVALID_ARG, "B=%d < 0", B);
  if (n_h < 1) return fail(MLA_ERR_INVALID_ARG, "n_h=%d < 1", n_h);
  if (T < 1) return fail(MLA_ERR_INVALID_ARG, "T=%d < 1", T);
  if (sparse && (K < 1 || K > T))
    return fail(MLA_ERR_INVALID_ARG, "top-k count K=%d outside [1, T=%d]", K, T);
  *rows = sparse ? K : T;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status st) {
  switch (st) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error; }

mla_status mla_dequant_fp8_block(const uint8_t* w_fp8, const float* scale, int64_t rows,
                                 int64_t cols, uint16_t* w_bf16, hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(MLA_ERR_INVALID_ARG, "negative size %lld x %lld",
                                        (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return MLA_OK;
  if (!w_fp8 || !scale || !w_bf16) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (cols % 16) return fail(MLA_ERR_UNSUPPORTED, "cols=%lld not a multiple of 16", (long long)cols);
  if (!aligned16(w_fp8) || !aligned16(w_bf16) || (reinterpret_cast<uintptr_t>(scale) & 3))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  return from_hip(launch_dequant_fp8_block(w_fp8, scale, rows, cols, w_bf16, stream),
                  "dequant launch");
}

mla_status mla_absorb_q(const void* q_nope, const void* wkv_b, void* q_lat, int B, int n_h,
                        mla_dtype dt, hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 0 || n_h < 1) return fail(MLA_ERR_INVALID_ARG, "B=%d n_h=%d", B, n_h);
  if (B == 0) return MLA_OK;
  if (!q_nope || !wkv_b || !q_lat) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(q_lat))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  return from_hip(launch_absorb_q(q_nope, wkv_b, q_lat, B, n_h, dt == MLA_BF16, stream),
                  "absorb launch");
}

int mla_decode_num_splits(int B, int n_h, int T, int K) {
  int rows;
  if (check_decode_dims(B, n_h, T, K, K > 0, &rows) != MLA_OK) return -1;
  SplitPlan sp;
  if (!plan_splits(B > 0 ? B : 1, n_h, rows, K > 0, 0, &sp)) return -1;
  return sp.num_splits;
}

size_t mla_decode_workspace_bytes(int B, int n_h, int T, int K, int num_splits, mla_dtype dt) {
  int rows;
  if (!dtype_ok(dt) || num_splits < 0) return static_cast<size_t>(-1);
  if (check_decode_dims(B, n_h, T, K, K > 0, &rows) != MLA_OK) return static_cast<size_t>(-1);
  if (B == 0) return 0;
  SplitPlan sp;
  if (!plan_splits(B, n_h, rows, K > 0, num_splits, &sp)) return static_cast<size_t>(-1);
  return ws_bytes_for(B, n_h, sp, dt);
}

}  // extern "C"

namespace {

// Argument checks and launch parameters shared by the decode calls: S_q
// query tokens of n_h_tok heads per sequence, read as S_q * n_h_tok query
// rows. *empty is set when there is nothing to launch (B == 0).
mla_status decode_prepare(const void* q_lat, const void* q_pe, const void* latent,
                          const void* rope, int64_t lat_bstride, int64_t lat_rstride,
                          int64_t rope_bstride, int64_t rope_rstride, int B, int S_q,
                          int n_h_tok, int T, const int32_t* topk_idx, int K, int causal,
                          float scale, int num_splits, void* out_lat, float* lse,
                          void* workspace, size_t ws_bytes, mla_dtype dt, DecodeParams* pp,
                          bool* empty, bool q_packed = false) {
  *empty = false;
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (S_q < 1) return fail(MLA_ERR_INVALID_ARG, "S_q=%d < 1", S_q);
  const bool sparse = topk_idx != nullptr;
  int rows;
  mla_status st = check_decode_dims(B, n_h_tok, T, K, sparse, &rows);
  if (st != MLA_OK) return st;
  if (causal && T < S_q)
    return fail(MLA_ERR_INVALID_ARG, "causal with T=%d < S_q=%d query tokens", T, S_q);
  if (causal && sparse)
    return fail(MLA_ERR_UNSUPPORTED, "the causal limit is implemented for dense attention only");
  if (static_cast<int64_t>(S_q) * n_h_tok > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "S_q * n_h above 65535");
  const int n_h = S_q * n_h_tok;  // query rows per sequence
  if (q_packed && (dt != MLA_BF16 || n_h % 128 != 0))
    return fail(MLA_ERR_UNSUPPORTED, "packed queries need bf16 and S_q * n_h a multiple of 128");
  if (B == 0) {
    *empty = true;
    return MLA_OK;
  }
  if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "B above 65535");
  if (!q_lat || !q_pe || !latent || !rope || !out_lat)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (num_splits < 0) return fail(MLA_ERR_INVALID_ARG, "num_splits=%d < 0", num_splits);
  const int64_t ealign = dt == MLA_BF16 ? 8 : 4;
  if (lat_rstride < D_C || rope_rstride < D_R)
    return fail(MLA_ERR_INVALID_ARG, "row strides %lld/%lld below 512/64", (long long)lat_rstride,
                (long long)rope_rstride);
  if (lat_bstride < 0 || rope_bstride < 0)
    return fail(MLA_ERR_INVALID_ARG, "negative batch stride");
  if (lat_rstride % ealign || rope_rstride % ealign || lat_bstride % ealign ||
      rope_bstride % ealign)
    return fail(MLA_ERR_UNSUPPORTED, "strides must be multiples of %lld elements",
                (long long)ealign);
  if (!aligned16(q_lat) || !aligned16(q_pe) || !aligned16(latent) || !aligned16(rope) ||
      !aligned16(out_lat) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3)))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  // bf16 rows are fetched with 32-bit byte offsets from each sequence's base
  if (dt == MLA_BF16 && (static_cast<int64_t>(T) * lat_rstride * 2 > INT32_MAX ||
                         static_cast<int64_t>(T) * rope_rstride * 2 > INT32_MAX))
    return fail(MLA_ERR_UNSUPPORTED, "T * row stride above 2^31 bytes");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "scale must be finite and positive");
  SplitPlan sp;
  if (!plan_splits(B, n_h, rows, sparse, num_splits, &sp))
    return fail(MLA_ERR_INVALID_ARG, "num_splits=%d outside [%d, %d]", num_splits,
                sparse ? ((rows + 31) / 32 + kMaxSparseTilesPerSplit - 1) / kMaxSparseTilesPerSplit
                       : 1,
                (rows + 31) / 32);
  if (static_cast<int64_t>(sp.num_splits) * ((n_h + group_heads(sparse) - 1) / group_heads(sparse)) * B >
      INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 workgroups");
  if (sp.num_splits > 1 && static_cast<int64_t>(B) * n_h > (int64_t{1} << 26))
    return fail(MLA_ERR_UNSUPPORTED, "B * n_h above 2^26 with split rows");
  const size_t need = ws_bytes_for(B, n_h, sp, dt);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? ws_bytes : static_cast<size_t>(0));
  if (need > 0 && !aligned16(workspace)) return fail(MLA_ERR_UNSUPPORTED, "misaligned workspace");

  DecodeParams& p = *pp;
  p = DecodeParams{};
  p.q_lat = q_lat;
  p.q_pe = q_pe;
  p.latent = latent;
  p.rope = rope;
  p.lat_bs = lat_bstride;
  p.lat_rs = lat_rstride;
  p.rope_bs = rope_bstride;
  p.rope_rs = rope_rstride;
  p.B = B;
  p.n_h = n_h;
  p.T = T;
  p.s_q = S_q;
  p.n_h_tok = n_h_tok;
  p.causal = causal ? 1 : 0;
  p.idx = topk_idx;
  p.K = sparse ? K : 0;
  p.rows = rows;
  p.num_splits = sp.num_splits;
  p.tiles_per_split = sp.tiles_per_split;
  p.scale = scale;
  p.q_swz = q_packed ? 1 : 0;
  p.out_lat = out_lat;
  p.lse = lse;
  if (need > 0) {
    const size_t bh = static_cast<size_t>(B) * n_h * sp.num_splits;
    const size_t esz = dt == MLA_BF16 ? 2 : 4;
    p.ws_o = workspace;
    p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(bh * D_C * esz));
  }
  return MLA_OK;
}

mla_status decode_impl(const void* q_lat, const void* q_pe, const void* latent, const void* rope,
                       int64_t lat_bstride, int64_t lat_rstride, int64_t rope_bstride,
                       int64_t rope_rstride, int B, int S_q, int n_h_tok, int T,
                       const int32_t* topk_idx, int K, int causal, float scale, int num_splits,
                       void* out_lat, float* lse, void* workspace, size_t ws_bytes,
                       mla_dtype dt, hipStream_t stream, bool q_packed = false) {
  DecodeParams p;
  bool empty;
  mla_status st = decode_prepare(q_lat, q_pe, latent, rope, lat_bstride, lat_rstride,
                                 rope_bstride, rope_rstride, B, S_q, n_h_tok, T, topk_idx, K,
                                 causal, scale, num_splits, out_lat, lse, workspace, ws_bytes, dt,
                                 &p, &empty, q_packed);
  if (st != MLA_OK || empty) return st;
  return from_hip(launch_decode(p, dt == MLA_BF16, stream), "decode launch");
}


}  // namespace

extern "C" {

mla_status mla_decode_latent_attn(const void* q_lat, const void* q_pe, const void* latent,
                                  const void* rope, int64_t lat_bstride, int64_t lat_rstride,
                                  int64_t rope_bstride, int64_t rope_rstride, int B, int n_h,
                                  int T, const int32_t* topk_idx, int K, float scale,
                                  int num_splits, void* out_lat, float* lse, void* workspace,
                                  size_t ws_bytes, mla_dtype dt, hipStream_t stream) {
  return decode_impl(q_lat, q_pe, latent, rope, lat_bstride, lat_rstride, rope_bstride,
                     rope_rstride, B, 1, n_h, T, topk_idx, K, 0, scale, num_splits, out_lat, lse,
                     workspace, ws_bytes, dt, stream);
}

mla_status mla_decode_latent_attn_multi(const void* q_lat, const void* q_pe, const void* latent,
                                        const void* rope, int64_t lat_bstride,
                                        int64_t lat_rstride, int64_t rope_bstride,
                                        int64_t rope_rstride, int B, int S_q, int n_h, int T,
                                        const int32_t* topk_idx, int K, int causal, float scale,
                                        int num_splits, void* out_lat, float* lse,
                                        void* workspace, size_t ws_bytes, mla_dtype dt,
                                        hipStream_t stream) {
  return decode_impl(q_lat, q_pe, latent, rope, lat_bstride, lat_rstride, rope_bstride,
                     rope_rstride, B, S_q, n_h, T, topk_idx, K, causal, scale, num_splits,
                     out_lat, lse, workspace, ws_bytes, dt, stream);
}

mla_status mla_decode_latent_attn_packed(const void* q_packed, const void* q_pe,
                                         const void* latent, const void* rope,
                                         int64_t lat_bstride, int64_t lat_rstride,
                                         int64_t rope_bstride, int64_t rope_rstride, int B,
                                         int S_q, int n_h, int T, const int32_t* topk_idx, int K,
                                         int causal, float scale, int num_splits, void* out_lat,
                                         float* lse, void* workspace, size_t ws_bytes,
                                         mla_dtype dt, hipStream_t stream) {
  return decode_impl(q_packed, q_pe, latent, rope, lat_bstride, lat_rstride, rope_bstride,
                     rope_rstride, B, S_q, n_h, T, topk_idx, K, causal, scale, num_splits,
                     out_lat, lse, workspace, ws_bytes, dt, stream, true);
}

mla_status mla_absorb_q_packed(const void* q_nope, const void* wkv_b, void* q_packed, int B,
                               int S_q, int n_h, mla_dtype dt, hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 0 || S_q < 1 || n_h < 1)
    return fail(MLA_ERR_INVALID_ARG, "B=%d S_q=%d n_h=%d", B, S_q, n_h);
  if (dt != MLA_BF16 || (static_cast<int64_t>(S_q) * n_h) % 128 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "packed queries need bf16 and S_q * n_h a multiple of 128");
  if (static_cast<int64_t>(B) * S_q > INT32_MAX || static_cast<int64_t>(S_q) * n_h > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "B * S_q or S_q * n_h too large");
  if (B == 0) return MLA_OK;
  if (!q_nope || !wkv_b || !q_packed) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(q_packed))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  return from_hip(launch_absorb_q_swizzled(q_nope, wkv_b, q_packed, B * S_q, n_h, S_q, stream),
                  "absorb launch");
}

size_t mla_decode_step_workspace_bytes(int B, int S_q, int n_h, int T, int K, int num_splits,
                                       mla_dtype dt) {
  if (S_q < 1 || B < 0 || n_h < 1 || static_cast<int64_t>(S_q) * n_h > 65535)
    return static_cast<size_t>(-1);
  const size_t attn = mla_decode_workspace_bytes(B, S_q * n_h, T, K, num_splits, dt);
  if (attn == static_cast<size_t>(-1)) return attn;
  const size_t esz = dt == MLA_BF16 ? 2 : 4;
  const size_t lat = align256(static_cast<size_t>(B) * S_q * n_h * D_C * esz);
  return 2 * lat + attn;
}

}  // extern "C"

namespace {

// Workspace of mla_decode_step_noalloc: one fixed device array per GPU,
// reserved when the library's code object is loaded and held until the
// process ends. In host code `scratch` is only a stand-in for the symbol,
// never a device address: kernels get the per-device address that
// hipGetSymbolAddress reports.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
mla_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  mla_status st = from_hip(hipGetDevice(&dev), "hipGetDevice");
  if (st != MLA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d devices with scratch", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = from_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != MLA_OK) return st;
    if (!p) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

// The decode step. With from_scratch, workspace/ws_bytes are ignored and the
// library's fixed scratch array is used: every argument is checked first
// (against a stand-in workspace address), then the array's address on the
// current device is looked up, and only then is anything enqueued.
mla_status decode_step_impl(const void* q_nope, const void* q_pe, const void* wkv_b,
                            const void* latent, const void* rope, int64_t lat_bstride,
                            int64_t lat_rstride, int64_t rope_bstride, int64_t rope_rstride, int B,
                            int S_q, int n_h, int T, const int32_t* topk_idx, int K, int causal,
                            float scale, int num_splits, void* out, float* lse, void* workspace,
                            size_t ws_bytes, mla_dtype dt, hipStream_t stream, bool from_scratch) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (S_q < 1 || B < 0 || n_h < 1)
    return fail(MLA_ERR_INVALID_ARG, "B=%d S_q=%d n_h=%d", B, S_q, n_h);
  if (static_cast<int64_t>(B) * S_q > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "B * S_q above 2^31 - 1");
  if (B == 0) return MLA_OK;
  if (!q_nope || !wkv_b || !out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(out))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  const size_t need = mla_decode_step_workspace_bytes(B, S_q, n_h, T, topk_idx ? K : 0,
                                                      num_splits, dt);
  if (need == static_cast<size_t>(-1)) {
    // let the attention checks name the problem
    int rows;
    mla_status st = check_decode_dims(B, n_h, T, K, topk_idx != nullptr, &rows);
    if (st != MLA_OK) return st;
    return fail(MLA_ERR_INVALID_ARG, "arguments rejected (S_q * n_h above 65535 or num_splits=%d)",
                num_splits);
  }
  if (from_scratch) {
    if (need > kNoAllocScratchBytes)
      return fail(MLA_ERR_WORKSPACE,
                  "the step needs %zu bytes of workspace; the fixed scratch holds %zu", need,
                  kNoAllocScratchBytes);
    workspace = reinterpret_cast<void*>(uintptr_t{256});  // stand-in for the checks
    ws_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? ws_bytes : static_cast<size_t>(0));
  if (!aligned16(workspace)) return fail(MLA_ERR_UNSUPPORTED, "misaligned workspace");
  const size_t esz = dt == MLA_BF16 ? 2 : 4;
  const size_t lat = align256(static_cast<size_t>(B) * S_q * n_h * D_C * esz);
  char* ws = static_cast<char*>(workspace);
  void* q_lat = ws;
  void* o_lat = ws + lat;
  const int BS = B * S_q;  // absorb and W^UV see every (sequence, token) as a batch row
  // every check happens before the first launch
  DecodeParams p;
  bool empty;
  mla_status st = decode_prepare(q_lat, q_pe, latent, rope, lat_bstride, lat_rstride,
                                 rope_bstride, rope_rstride, B, S_q, n_h, T, topk_idx, K, causal,
                                 scale, num_splits, o_lat, lse, ws + 2 * lat, ws_bytes - 2 * lat,
                                 dt, &p, &empty, dt == MLA_BF16 && (S_q * n_h) % 128 == 0);
  if (st != MLA_OK) return st;
  if (from_scratch) {
    // every check has passed: the real workspace, then the same plan on it
    void* sp = nullptr;
    st = scratch_of_current_device(&sp);
    if (st != MLA_OK) return st;
    ws = static_cast<char*>(sp);
    q_lat = ws;
    o_lat = ws + lat;
    st = decode_prepare(q_lat, q_pe, latent, rope, lat_bstride, lat_rstride, rope_bstride,
                        rope_rstride, B, S_q, n_h, T, topk_idx, K, causal, scale, num_splits,
                        o_lat, lse, ws + 2 * lat, ws_bytes - 2 * lat, dt, &p, &empty,
                        dt == MLA_BF16 && (S_q * n_h) % 128 == 0);
    if (st != MLA_OK) return st;
  }
  // full 128-row groups: q_lat goes to the workspace in the attention
  // kernel's operand order (each wave then loads one contiguous KiB per
  // k-step instead of 32 row pieces)
  if (p.q_swz) {
    st = from_hip(launch_absorb_q_swizzled(q_nope, wkv_b, q_lat, BS, n_h, S_q, stream),
                  "absorb launch");
  } else {
    st = from_hip(launch_absorb_q(q_nope, wkv_b, q_lat, BS, n_h, dt == MLA_BF16, stream),
                  "absorb launch");
  }
  if (st != MLA_OK) return st;
  if (dt == MLA_BF16 && p.num_splits > 1) {
    // the split merge is fused into W^UV: the merged rows stay on chip
    st = from_hip(launch_decode(p, true, stream, false), "decode launch");
    if (st != MLA_OK) return st;
    return from_hip(launch_merge_out_up(p.ws_o, p.ws_lse, p.num_splits, wkv_b, out, lse, BS, n_h,
                                        stream),
                    "merge_out_up launch");
  }
  st = from_hip(launch_decode(p, dt == MLA_BF16, stream), "decode launch");
  if (st != MLA_OK) return st;
  return from_hip(launch_out_up(o_lat, wkv_b, out, BS, n_h, dt == MLA_BF16, stream),
                  "out_up launch");
}

}  // namespace

extern "C" {

mla_status mla_decode_step(const void* q_nope, const void* q_pe, const void* wkv_b,
                           const void* latent, const void* rope, int64_t lat_bstride,
                           int64_t lat_rstride, int64_t rope_bstride, int64_t rope_rstride, int B,
                           int S_q, int n_h, int T, const int32_t* topk_idx, int K, int causal,
                           float scale, int num_splits, void* out, float* lse, void* workspace,
                           size_t ws_bytes, mla_dtype dt, hipStream_t stream) {
  return decode_step_impl(q_nope, q_pe, wkv_b, latent, rope, lat_bstride, lat_rstride,
                          rope_bstride, rope_rstride, B, S_q, n_h, T, topk_idx, K, causal, scale,
                          num_splits, out, lse, workspace, ws_bytes, dt, stream, false);
}

mla_status mla_decode_step_noalloc(const void* q_nope, const void* q_pe, const void* wkv_b,
                                   const void* latent, const void* rope, int64_t lat_bstride,
                                   int64_t lat_rstride, int64_t rope_bstride,
                                   int64_t rope_rstride, int B, int S_q, int n_h, int T,
                                   const int32_t* topk_idx, int K, int causal, float scale,
                                   int num_splits, void* out, float* lse, mla_dtype dt,
                                   hipStream_t stream) {
  return decode_step_impl(q_nope, q_pe, wkv_b, latent, rope, lat_bstride, lat_rstride,
                          rope_bstride, rope_rstride, B, S_q, n_h, T, topk_idx, K, causal, scale,
                          num_splits, out, lse, nullptr, 0, dt, stream, true);
}

mla_status mla_out_up(const void* out_lat, const void* wkv_b, void* out, int B, int n_h,
                      mla_dtype dt, hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 0 || n_h < 1) return fail(MLA_ERR_INVALID_ARG, "B=%d n_h=%d", B, n_h);
  if (B == 0) return MLA_OK;
  if (!out_lat || !wkv_b || !out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(out_lat) || !aligned16(wkv_b) || !aligned16(out))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  return from_hip(launch_out_up(out_lat, wkv_b, out, B, n_h, dt == MLA_BF16, stream),
                  "out_up launch");
}

mla_status mla_kv_reconstruct(const void* c, const void* k_rope, const void* wkv_b, void* K,
                              void* V, int64_t N, int n_h, mla_dtype dt, hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (N < 0 || n_h < 1) return fail(MLA_ERR_INVALID_ARG, "N=%lld n_h=%d", (long long)N, n_h);
  if (N == 0) return MLA_OK;
  if (!c || !k_rope || !wkv_b || !K || !V) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(c) || !aligned16(k_rope) || !aligned16(wkv_b) || !aligned16(K) || !aligned16(V))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  if (N * n_h >= (static_cast<int64_t>(1) << 31))
    return fail(MLA_ERR_UNSUPPORTED, "N * n_h too large for one launch");
  return from_hip(launch_kv_reconstruct(c, k_rope, wkv_b, K, V, N, n_h, dt == MLA_BF16, stream),
                  "kv_reconstruct launch");
}

size_t mla_attention_naive_workspace_bytes(int B, int S, int T, int K) {
  if (B < 0 || S < 0 || T < 1 || K < 0 || K > T) return static_cast<size_t>(-1);
  if (K == 0) return 0;
  const int64_t qb = attention_query_block(), kt = attention_key_tile();
  const int64_t words = (T + kt - 1) / kt * (kt / 32);
  const int64_t s_pad = (S + qb - 1) / qb * qb;
  return static_cast<size_t>(B) * static_cast<size_t>(words) * static_cast<size_t>(s_pad) * 4;
}

mla_status mla_attention_naive(const void* q, const void* k, const void* v, int B, int S, int T,
                               int n_h, const int32_t* topk_idx, int K, int causal, float scale,
                               void* out, float* lse, void* workspace, size_t ws_bytes,
                               mla_dtype dt, hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 0 || S < 0 || T < 1 || n_h < 1)
    return fail(MLA_ERR_INVALID_ARG, "B=%d S=%d T=%d n_h=%d", B, S, T, n_h);
  if (topk_idx && (K < 1 || K > T))
    return fail(MLA_ERR_INVALID_ARG, "index count K=%d outside [1, T=%d]", K, T);
  if (causal && T < S) return fail(MLA_ERR_INVALID_ARG, "causal with T=%d < S=%d", T, S);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "scale must be finite and positive");
  if (B == 0 || S == 0) return MLA_OK;
  if (!q || !k || !v || !out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3)))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  if (n_h > 65535 || B > 65535 || (dt == MLA_F32 && S > INT32_MAX))
    return fail(MLA_ERR_UNSUPPORTED, "B or n_h above 65535");
  const int qb = attention_query_block();
  const int64_t nqb = (static_cast<int64_t>(S) + qb - 1) / qb;
  if (nqb * n_h * B > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 workgroups");
  // key rows are fetched with 32-bit byte offsets within a 64-key tile
  if (static_cast<int64_t>(n_h) * 192 * (dt == MLA_BF16 ? 2 : 4) * 64 > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "n_h too large");
  const size_t need = mla_attention_naive_workspace_bytes(B, S, T, topk_idx ? K : 0);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? ws_bytes : static_cast<size_t>(0));
  if (need > 0 && !aligned16(workspace)) return fail(MLA_ERR_UNSUPPORTED, "misaligned workspace");
  AttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.mask = static_cast<uint32_t*>(workspace);
  p.B = B;
  p.S = S;
  p.T = T;
  p.n_h = n_h;
  p.nqb = static_cast<int>(nqb);
  const int kt = attention_key_tile();
  p.mask_words = (T + kt - 1) / kt * (kt / 32);
  p.s_pad = static_cast<int>(nqb * qb);
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  return from_hip(launch_attention(p, topk_idx, topk_idx ? K : 0, dt == MLA_BF16, stream),
                  "attention launch");
}

mla_status mla_cache_append(const void* kv_a, int64_t in_rstride, const float* gamma, float eps,
                            const float* freqs, int n_pos, const int32_t* seq_idx,
                            const int32_t* pos, int64_t N, void* latent, void* rope,
                            int64_t lat_bstride, int64_t lat_rstride, int64_t rope_bstride,
                            int64_t rope_rstride, int B_cache, int T_cache, mla_dtype dt,
                            hipStream_t stream) {
  if (!dtype_ok(dt)) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (N < 0 || n_pos < 0 || B_cache < 0 || T_cache < 0)
    return fail(MLA_ERR_INVALID_ARG, "N=%lld n_pos=%d B_cache=%d T_cache=%d", (long long)N,
                n_pos, B_cache, T_cache);
  if (!(eps >= 0.f)) return fail(MLA_ERR_INVALID_ARG, "eps=%g is negative or NaN", (double)eps);
  if (N == 0) return MLA_OK;
  if (!kv_a || !gamma || !freqs || !pos || !latent || !rope)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (!seq_idx && N > B_cache)
    return fail(MLA_ERR_INVALID_ARG, "N=%lld rows without seq_idx but only %d sequences",
                (long long)N, B_cache);
  if (in_rstride < D_QK || lat_rstride < D_C || rope_rstride < D_R || lat_bstride < 0 ||
      rope_bstride < 0)
    return fail(MLA_ERR_INVALID_ARG, "stride too small");
  const int64_t vec = dt == MLA_BF16 ? 8 : 4;
  if (!aligned16(kv_a) || !aligned16(gamma) || !aligned16(freqs) || !aligned16(latent) ||
      !aligned16(rope))
    return fail(MLA_ERR_UNSUPPORTED, "misaligned pointer");
  if (in_rstride % vec || lat_rstride % vec || rope_rstride % vec || lat_bstride % vec ||
      rope_bstride % vec)
    return fail(MLA_ERR_UNSUPPORTED, "strides must be multiples of %lld elements", (long long)vec);
  if ((N + 3) / 4 > INT_MAX) return fail(MLA_ERR_UNSUPPORTED, "N too large for one launch");
  AppendParams p{kv_a, in_rstride, gamma, eps, freqs, n_pos, seq_idx, pos, N, latent, rope,
                 lat_bstride, lat_rstride, rope_bstride, rope_rstride, B_cache, T_cache};
  return from_hip(launch_cache_append(p, dt == MLA_BF16, stream), "cache_append launch");
}

}  // extern "C"

extern "C" float mla_softmax_scale(int qk_head_dim, int64_t max_seq_len, int64_t original_seq_len,
                                   float mscale, float rope_factor) {
  if (qk_head_dim <= 0) return NAN;
  double scale = 1.0 / std::sqrt(static_cast<double>(qk_head_dim));
  if (max_seq_len > original_seq_len) {
    if (!(rope_factor > 0.f)) return NAN;
    const double ms = 0.1 * static_cast<double>(mscale) * std::log(static_cast<double>(rope_factor)) + 1.0;
    scale *= ms * ms;
  }
  return static_cast<float>(scale);
}
