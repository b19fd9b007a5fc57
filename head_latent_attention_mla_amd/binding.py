"""Python binding of libmla.so (the C ABI in include/mla.h).

Argument marshalling only: every function checks torch tensor metadata,
allocates outputs the caller did not pass (torch device memory), and calls
the C entry point of the same name on the current HIP stream. All compute
happens in the library's HIP kernels; there is no fallback of any kind, and
a missing library raises MLAError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
SCALE = 192 ** -0.5  # 1 / sqrt(d_h + d_h^R)

_STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
           3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, status)} {detail}".strip())


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libmla.so (raises MLAError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MLAError("load", -1, f"{LIB_PATH} is missing; build it with "
                           "`python -m head_latent_attention_mla_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, L, F, Z = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                         ctypes.c_size_t)
        lib.mla_status_str.argtypes = [I]
        lib.mla_status_str.restype = ctypes.c_char_p
        lib.mla_last_error.argtypes = []
        lib.mla_last_error.restype = ctypes.c_char_p
        lib.mla_dequant_fp8_block.argtypes = [P, P, L, L, P, P]
        lib.mla_absorb_q.argtypes = [P, P, P, I, I, I, P]
        lib.mla_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
        lib.mla_decode_workspace_bytes.restype = Z
        lib.mla_decode_num_splits.argtypes = [I, I, I, I]
        lib.mla_decode_num_splits.restype = I
        lib.mla_decode_latent_attn.argtypes = [P, P, P, P, L, L, L, L, I, I, I, P, I, F, I,
                                               P, P, P, Z, I, P]
        lib.mla_out_up.argtypes = [P, P, P, I, I, I, P]
        lib.mla_kv_reconstruct.argtypes = [P, P, P, P, P, L, I, I, P]
        lib.mla_softmax_scale.argtypes = [I, L, L, F, F]
        lib.mla_softmax_scale.restype = F
        lib.mla_decode_latent_attn_multi.argtypes = [P, P, P, P, L, L, L, L, I, I, I, I, P, I,
                                                     I, F, I, P, P, P, Z, I, P]
        lib.mla_absorb_q_packed.argtypes = [P, P, P, I, I, I, I, P]
        lib.mla_decode_latent_attn_packed.argtypes = [P, P, P, P, L, L, L, L, I, I, I, I, P, I,
                                                      I, F, I, P, P, P, Z, I, P]
        lib.mla_decode_step_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.mla_decode_step_workspace_bytes.restype = Z
        lib.mla_decode_step.argtypes = [P, P, P, P, P, L, L, L, L, I, I, I, I, P, I, I, F, I, P,
                                        P, P, Z, I, P]
        lib.mla_decode_step_noalloc.argtypes = [P, P, P, P, P, L, L, L, L, I, I, I, I, P, I, I,
                                                F, I, P, P, I, P]
        lib.mla_attention_naive_workspace_bytes.argtypes = [I, I, I, I]
        lib.mla_attention_naive_workspace_bytes.restype = Z
        lib.mla_attention_naive.argtypes = [P, P, P, I, I, I, I, P, I, I, F, P, P, P, Z, I, P]
        lib.mla_cache_append.argtypes = [P, L, P, F, P, I, P, P, L, P, P, L, L, L, L, I, I, I,
                                         P]
        for name in ("mla_dequant_fp8_block", "mla_absorb_q", "mla_decode_latent_attn",
                     "mla_out_up", "mla_kv_reconstruct", "mla_cache_append",
                     "mla_decode_latent_attn_multi", "mla_decode_step", "mla_decode_step_noalloc",
                     "mla_absorb_q_packed", "mla_decode_latent_attn_packed",
                     "mla_attention_naive"):
            getattr(lib, name).restype = I
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MLAError(fn, status, library().mla_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        if t is not None:
            _require(t.is_cuda, "tensors must be on the GPU")


def mla_dequant_fp8_block(w_fp8: torch.Tensor, scale: torch.Tensor, out: torch.Tensor = None,
                          stream=None) -> torch.Tensor:
    """bf16 [rows, cols] = e4m3 codes (uint8) x fp32 scale per 128x128 block."""
    _dev(w_fp8, scale, out)
    _require(w_fp8.dtype == torch.uint8 and w_fp8.dim() == 2 and w_fp8.is_contiguous(),
             "w_fp8 must be a contiguous 2-D uint8 tensor")
    rows, cols = w_fp8.shape
    _require(scale.dtype == torch.float32 and scale.is_contiguous() and
             tuple(scale.shape) == ((rows + 127) // 128, (cols + 127) // 128),
             "scale must be contiguous float32 [ceil(rows/128), ceil(cols/128)]")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=w_fp8.device)
    _require(out.dtype == torch.bfloat16 and out.is_contiguous() and out.shape == w_fp8.shape,
             "out must be contiguous bf16 of the same shape")
    _check("mla_dequant_fp8_block", library().mla_dequant_fp8_block(
        _ptr(w_fp8), _ptr(scale), rows, cols, _ptr(out), _stream(stream)))
    return out


def mla_absorb_q(q_nope: torch.Tensor, wkv_b: torch.Tensor, q_lat: torch.Tensor = None,
                 stream=None) -> torch.Tensor:
    """q_lat [B, n_h, 512] = q_nope [B, n_h, 128] absorbed with W^UK of wkv_b."""
    _dev(q_nope, wkv_b, q_lat)
    B, n_h, d = q_nope.shape
    _require(d == 128 and q_nope.is_contiguous(), "q_nope must be contiguous [B, n_h, 128]")
    _require(wkv_b.dtype == q_nope.dtype and wkv_b.is_contiguous() and
             tuple(wkv_b.shape) == (n_h * 256, 512), "wkv_b must be contiguous [n_h*256, 512]")
    if q_lat is None:
        q_lat = torch.empty((B, n_h, 512), dtype=q_nope.dtype, device=q_nope.device)
    _require(q_lat.dtype == q_nope.dtype and q_lat.is_contiguous() and
             tuple(q_lat.shape) == (B, n_h, 512), "q_lat must be contiguous [B, n_h, 512]")
    _check("mla_absorb_q", library().mla_absorb_q(
        _ptr(q_nope), _ptr(wkv_b), _ptr(q_lat), B, n_h, _dtype_code(q_nope), _stream(stream)))
    return q_lat


def mla_decode_workspace_bytes(B: int, n_h: int, T: int, K: int = 0, num_splits: int = 0,
                               dtype=torch.bfloat16) -> int:
    code = MLA_BF16 if dtype == torch.bfloat16 else MLA_F32
    v = library().mla_decode_workspace_bytes(B, n_h, T, K, num_splits, code)
    if v == ctypes.c_size_t(-1).value:
        raise MLAError("mla_decode_workspace_bytes", 1, "arguments rejected")
    return v


def mla_decode_num_splits(B: int, n_h: int, T: int, K: int = 0) -> int:
    v = library().mla_decode_num_splits(B, n_h, T, K)
    if v < 0:
        raise MLAError("mla_decode_num_splits", 1, "arguments rejected")
    return v


def _cache_strides(t: torch.Tensor, width: int, name: str):
    _require(t.dim() == 3 and t.stride(2) == 1 and t.shape[2] == width,
             f"{name} must be [B, T_alloc, {width}] with unit stride in the last dim")
    return t.stride(0), t.stride(1)


def mla_decode_latent_attn(q_lat: torch.Tensor, q_pe: torch.Tensor, latent: torch.Tensor,
                           rope: torch.Tensor, T: int = None, topk_idx: torch.Tensor = None,
                           scale: float = SCALE, num_splits: int = 0,
                           out_lat: torch.Tensor = None, lse: torch.Tensor = None,
                           workspace: torch.Tensor = None, want_lse: bool = False,
                           stream=None):
    """Latent attention of the absorbed decode step.

    latent [B, T_alloc, 512] and rope [B, T_alloc, 64] may be views of one
    packed [B, T_alloc, 576] cache (cache[..., :512], cache[..., 512:]).
    Returns out_lat [B, n_h, 512] (and lse [B, n_h] fp32 if requested).
    """
    _dev(q_lat, q_pe, latent, rope, topk_idx, out_lat, lse, workspace)
    B, n_h, d = q_lat.shape
    _require(d == 512 and q_lat.is_contiguous(), "q_lat must be contiguous [B, n_h, 512]")
    _require(q_pe.dtype == q_lat.dtype and q_pe.is_contiguous() and
             tuple(q_pe.shape) == (B, n_h, 64), "q_pe must be contiguous [B, n_h, 64]")
    _require(latent.dtype == q_lat.dtype and rope.dtype == q_lat.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    _require(latent.shape[0] >= B and rope.shape[0] >= B, "cache batch too small")
    if T is None:
        T = latent.shape[1]
    _require(T <= latent.shape[1] and T <= rope.shape[1], "T exceeds the cache length")
    K = 0
    if topk_idx is not None:
        _require(topk_idx.dtype == torch.int32 and topk_idx.is_contiguous() and
                 topk_idx.dim() == 2 and topk_idx.shape[0] == B,
                 "topk_idx must be contiguous int32 [B, K]")
        K = topk_idx.shape[1]
    if out_lat is None:
        out_lat = torch.empty((B, n_h, 512), dtype=q_lat.dtype, device=q_lat.device)
    _require(out_lat.dtype == q_lat.dtype and out_lat.is_contiguous() and
             tuple(out_lat.shape) == (B, n_h, 512), "out_lat must be contiguous [B, n_h, 512]")
    if lse is None and want_lse:
        lse = torch.empty((B, n_h), dtype=torch.float32, device=q_lat.device)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and
                 tuple(lse.shape) == (B, n_h), "lse must be contiguous float32 [B, n_h]")
    need = mla_decode_workspace_bytes(B, n_h, T, K, num_splits, q_lat.dtype) if B > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_latent_attn", library().mla_decode_latent_attn(
        _ptr(q_lat), _ptr(q_pe), _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B, n_h, T,
        _ptr(topk_idx), K, float(scale), num_splits, _ptr(out_lat), _ptr(lse),
        _ptr(workspace), ws_bytes, _dtype_code(q_lat), _stream(stream)))
    return (out_lat, lse) if (want_lse or lse is not None) else out_lat


def _topk_arg(topk_idx, B):
    if topk_idx is None:
        return 0
    _require(topk_idx.dtype == torch.int32 and topk_idx.is_contiguous() and
             topk_idx.dim() == 2 and topk_idx.shape[0] == B,
             "topk_idx must be contiguous int32 [B, K]")
    return topk_idx.shape[1]


def mla_decode_latent_attn_multi(q_lat: torch.Tensor, q_pe: torch.Tensor, latent: torch.Tensor,
                                 rope: torch.Tensor, T: int = None, topk_idx: torch.Tensor = None,
                                 causal: bool = False, scale: float = SCALE, num_splits: int = 0,
                                 out_lat: torch.Tensor = None, lse: torch.Tensor = None,
                                 workspace: torch.Tensor = None, want_lse: bool = False,
                                 stream=None):
    """Latent attention of S_q query tokens per sequence: q_lat [B, S_q, n_h,
    512], q_pe [B, S_q, n_h, 64]; T counts the cached positions including the
    S_q new ones (default: the cache length). causal: token j sees positions
    up to T - S_q + j. Returns out_lat [B, S_q, n_h, 512] (and lse
    [B, S_q, n_h] fp32 if requested)."""
    _dev(q_lat, q_pe, latent, rope, topk_idx, out_lat, lse, workspace)
    _require(q_lat.dim() == 4 and q_lat.shape[3] == 512 and q_lat.is_contiguous(),
             "q_lat must be contiguous [B, S_q, n_h, 512]")
    B, S_q, n_h, _ = q_lat.shape
    _require(q_pe.dtype == q_lat.dtype and q_pe.is_contiguous() and
             tuple(q_pe.shape) == (B, S_q, n_h, 64), "q_pe must be contiguous [B, S_q, n_h, 64]")
    _require(latent.dtype == q_lat.dtype and rope.dtype == q_lat.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    _require(latent.shape[0] >= B and rope.shape[0] >= B, "cache batch too small")
    if T is None:
        T = latent.shape[1]
    _require(T <= latent.shape[1] and T <= rope.shape[1], "T exceeds the cache length")
    K = _topk_arg(topk_idx, B)
    if out_lat is None:
        out_lat = torch.empty((B, S_q, n_h, 512), dtype=q_lat.dtype, device=q_lat.device)
    _require(out_lat.dtype == q_lat.dtype and out_lat.is_contiguous() and
             tuple(out_lat.shape) == (B, S_q, n_h, 512),
             "out_lat must be contiguous [B, S_q, n_h, 512]")
    if lse is None and want_lse:
        lse = torch.empty((B, S_q, n_h), dtype=torch.float32, device=q_lat.device)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and
                 tuple(lse.shape) == (B, S_q, n_h), "lse must be contiguous float32 [B, S_q, n_h]")
    need = (mla_decode_workspace_bytes(B, S_q * n_h, T, K, num_splits, q_lat.dtype)
            if B > 0 else 0)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_latent_attn_multi", library().mla_decode_latent_attn_multi(
        _ptr(q_lat), _ptr(q_pe), _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B, S_q, n_h, T,
        _ptr(topk_idx), K, int(bool(causal)), float(scale), num_splits, _ptr(out_lat), _ptr(lse),
        _ptr(workspace), ws_bytes, _dtype_code(q_lat), _stream(stream)))
    return (out_lat, lse) if (want_lse or lse is not None) else out_lat


def mla_absorb_q_packed(q_nope: torch.Tensor, wkv_b: torch.Tensor, q_packed: torch.Tensor = None,
                        stream=None) -> torch.Tensor:
    """Absorbed queries in the attention kernel's operand order (see
    include/mla.h): q_nope [B, S_q, n_h, 128] (or [B, n_h, 128]) bf16 with
    S_q * n_h a multiple of 128. Returns q_packed [B, S_q * n_h * 512]."""
    _dev(q_nope, wkv_b, q_packed)
    if q_nope.dim() == 3:
        q_nope = q_nope.unsqueeze(1)
    _require(q_nope.dim() == 4 and q_nope.shape[3] == 128 and q_nope.is_contiguous(),
             "q_nope must be contiguous [B, S_q, n_h, 128]")
    B, S_q, n_h, _ = q_nope.shape
    _require(wkv_b.dtype == q_nope.dtype and wkv_b.is_contiguous() and
             tuple(wkv_b.shape) == (n_h * 256, 512), "wkv_b must be contiguous [n_h*256, 512]")
    if q_packed is None:
        q_packed = torch.empty((B, S_q * n_h * 512), dtype=q_nope.dtype, device=q_nope.device)
    _require(q_packed.dtype == q_nope.dtype and q_packed.is_contiguous() and
             q_packed.numel() == B * S_q * n_h * 512, "q_packed must hold B*S_q*n_h*512 elements")
    _check("mla_absorb_q_packed", library().mla_absorb_q_packed(
        _ptr(q_nope), _ptr(wkv_b), _ptr(q_packed), B, S_q, n_h, _dtype_code(q_nope),
        _stream(stream)))
    return q_packed


def mla_decode_latent_attn_packed(q_packed: torch.Tensor, q_pe: torch.Tensor,
                                  latent: torch.Tensor, rope: torch.Tensor, T: int = None,
                                  topk_idx: torch.Tensor = None, causal: bool = False,
                                  scale: float = SCALE, num_splits: int = 0,
                                  out_lat: torch.Tensor = None, lse: torch.Tensor = None,
                                  workspace: torch.Tensor = None, want_lse: bool = False,
                                  stream=None):
    """mla_decode_latent_attn_multi with packed queries (mla_absorb_q_packed);
    S_q and n_h are taken from q_pe [B, S_q, n_h, 64] (or [B, n_h, 64]).
    Returns out_lat [B, S_q, n_h, 512] (and lse [B, S_q, n_h])."""
    _dev(q_packed, q_pe, latent, rope, topk_idx, out_lat, lse, workspace)
    if q_pe.dim() == 3:
        q_pe = q_pe.unsqueeze(1)
    _require(q_pe.dim() == 4 and q_pe.shape[3] == 64 and q_pe.is_contiguous(),
             "q_pe must be contiguous [B, S_q, n_h, 64]")
    B, S_q, n_h, _ = q_pe.shape
    _require(q_packed.dtype == q_pe.dtype and q_packed.is_contiguous() and
             q_packed.numel() == B * S_q * n_h * 512, "q_packed must hold B*S_q*n_h*512 elements")
    _require(latent.dtype == q_pe.dtype and rope.dtype == q_pe.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    _require(latent.shape[0] >= B and rope.shape[0] >= B, "cache batch too small")
    if T is None:
        T = latent.shape[1]
    _require(T <= latent.shape[1] and T <= rope.shape[1], "T exceeds the cache length")
    K = _topk_arg(topk_idx, B)
    if out_lat is None:
        out_lat = torch.empty((B, S_q, n_h, 512), dtype=q_pe.dtype, device=q_pe.device)
    _require(out_lat.dtype == q_pe.dtype and out_lat.is_contiguous() and
             out_lat.numel() == B * S_q * n_h * 512, "out_lat must hold B*S_q*n_h*512 elements")
    if lse is None and want_lse:
        lse = torch.empty((B, S_q, n_h), dtype=torch.float32, device=q_pe.device)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and
                 lse.numel() == B * S_q * n_h, "lse must be contiguous float32 [B, S_q, n_h]")
    need = (mla_decode_workspace_bytes(B, S_q * n_h, T, K, num_splits, q_pe.dtype)
            if B > 0 else 0)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_pe.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_latent_attn_packed", library().mla_decode_latent_attn_packed(
        _ptr(q_packed), _ptr(q_pe), _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B, S_q, n_h, T,
        _ptr(topk_idx), K, int(bool(causal)), float(scale), num_splits, _ptr(out_lat), _ptr(lse),
        _ptr(workspace), ws_bytes, _dtype_code(q_pe), _stream(stream)))
    return (out_lat, lse) if (want_lse or lse is not None) else out_lat


def mla_decode_step_workspace_bytes(B: int, S_q: int, n_h: int, T: int, K: int = 0,
                                    num_splits: int = 0, dtype=torch.bfloat16) -> int:
    code = MLA_BF16 if dtype == torch.bfloat16 else MLA_F32
    v = library().mla_decode_step_workspace_bytes(B, S_q, n_h, T, K, num_splits, code)
    if v == ctypes.c_size_t(-1).value:
        raise MLAError("mla_decode_step_workspace_bytes", 1, "arguments rejected")
    return v


def mla_decode_step(q_nope: torch.Tensor, q_pe: torch.Tensor, wkv_b: torch.Tensor,
                    latent: torch.Tensor, rope: torch.Tensor, T: int = None,
                    topk_idx: torch.Tensor = None, causal: bool = False, scale: float = SCALE,
                    num_splits: int = 0, out: torch.Tensor = None, lse: torch.Tensor = None,
                    workspace: torch.Tensor = None, want_lse: bool = False, stream=None):
    """The whole absorbed decode step in one call: q_nope [B, S_q, n_h, 128]
    (or [B, n_h, 128] for one token), q_pe likewise with 64 features, wkv_b
    [n_h*256, 512]. Returns out [B, S_q, n_h, 128] (the input's rank) and lse
    if requested."""
    _dev(q_nope, q_pe, wkv_b, latent, rope, topk_idx, out, lse, workspace)
    squeeze = q_nope.dim() == 3
    if squeeze:
        q_nope, q_pe = q_nope.unsqueeze(1), q_pe.unsqueeze(1)
    _require(q_nope.dim() == 4 and q_nope.shape[3] == 128 and q_nope.is_contiguous(),
             "q_nope must be contiguous [B, S_q, n_h, 128]")
    B, S_q, n_h, _ = q_nope.shape
    _require(q_pe.dtype == q_nope.dtype and q_pe.is_contiguous() and
             tuple(q_pe.shape) == (B, S_q, n_h, 64), "q_pe must be contiguous [B, S_q, n_h, 64]")
    _require(wkv_b.dtype == q_nope.dtype and wkv_b.is_contiguous() and
             tuple(wkv_b.shape) == (n_h * 256, 512), "wkv_b must be contiguous [n_h*256, 512]")
    _require(latent.dtype == q_nope.dtype and rope.dtype == q_nope.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    _require(latent.shape[0] >= B and rope.shape[0] >= B, "cache batch too small")
    if T is None:
        T = latent.shape[1]
    _require(T <= latent.shape[1] and T <= rope.shape[1], "T exceeds the cache length")
    K = _topk_arg(topk_idx, B)
    shape = (B, n_h, 128) if squeeze else (B, S_q, n_h, 128)
    if out is None:
        out = torch.empty(shape, dtype=q_nope.dtype, device=q_nope.device)
    _require(out.dtype == q_nope.dtype and out.is_contiguous() and tuple(out.shape) == shape,
             f"out must be contiguous {list(shape)}")
    if lse is None and want_lse:
        lse = torch.empty(shape[:-1], dtype=torch.float32, device=q_nope.device)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * S_q * n_h,
                 "lse must be contiguous float32 with B * S_q * n_h elements")
    if workspace is None and B > 0:
        need = mla_decode_step_workspace_bytes(B, S_q, n_h, T, K, num_splits, q_nope.dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_nope.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_step", library().mla_decode_step(
        _ptr(q_nope), _ptr(q_pe), _ptr(wkv_b), _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B,
        S_q, n_h, T, _ptr(topk_idx), K, int(bool(causal)), float(scale), num_splits, _ptr(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _dtype_code(q_nope), _stream(stream)))
    return (out, lse) if (want_lse or lse is not None) else out


def mla_decode_step_noalloc(q_nope: torch.Tensor, q_pe: torch.Tensor, wkv_b: torch.Tensor,
                            latent: torch.Tensor, rope: torch.Tensor, out: torch.Tensor,
                            T: int = None, topk_idx: torch.Tensor = None, causal: bool = False,
                            scale: float = SCALE, num_splits: int = 0, lse: torch.Tensor = None,
                            stream=None) -> torch.Tensor:
    """mla_decode_step with its workspace in the library's fixed per-GPU
    scratch array (64 MiB): the caller passes inputs and outputs only (out is
    required; nothing is allocated here or in the library). Calls that
    overlap on one GPU share the scratch and race."""
    _dev(q_nope, q_pe, wkv_b, latent, rope, topk_idx, out, lse)
    squeeze = q_nope.dim() == 3
    if squeeze:
        q_nope, q_pe = q_nope.unsqueeze(1), q_pe.unsqueeze(1)
    _require(q_nope.dim() == 4 and q_nope.shape[3] == 128 and q_nope.is_contiguous(),
             "q_nope must be contiguous [B, S_q, n_h, 128]")
    B, S_q, n_h, _ = q_nope.shape
    _require(q_pe.dtype == q_nope.dtype and q_pe.is_contiguous() and
             tuple(q_pe.shape) == (B, S_q, n_h, 64), "q_pe must be contiguous [B, S_q, n_h, 64]")
    _require(wkv_b.dtype == q_nope.dtype and wkv_b.is_contiguous() and
             tuple(wkv_b.shape) == (n_h * 256, 512), "wkv_b must be contiguous [n_h*256, 512]")
    _require(latent.dtype == q_nope.dtype and rope.dtype == q_nope.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    _require(latent.shape[0] >= B and rope.shape[0] >= B, "cache batch too small")
    if T is None:
        T = latent.shape[1]
    _require(T <= latent.shape[1] and T <= rope.shape[1], "T exceeds the cache length")
    K = _topk_arg(topk_idx, B)
    shape = (B, n_h, 128) if squeeze else (B, S_q, n_h, 128)
    _require(out is not None and out.dtype == q_nope.dtype and out.is_contiguous() and
             tuple(out.shape) == shape, f"out must be given, contiguous {list(shape)}")
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * S_q * n_h,
                 "lse must be contiguous float32 with B * S_q * n_h elements")
    _check("mla_decode_step_noalloc", library().mla_decode_step_noalloc(
        _ptr(q_nope), _ptr(q_pe), _ptr(wkv_b), _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B,
        S_q, n_h, T, _ptr(topk_idx), K, int(bool(causal)), float(scale), num_splits, _ptr(out),
        _ptr(lse), _dtype_code(q_nope), _stream(stream)))
    return out


def mla_out_up(out_lat: torch.Tensor, wkv_b: torch.Tensor, out: torch.Tensor = None,
               stream=None) -> torch.Tensor:
    """out [B, n_h, 128] = W^UV of wkv_b applied to out_lat [B, n_h, 512]."""
    _dev(out_lat, wkv_b, out)
    B, n_h, d = out_lat.shape
    _require(d == 512 and out_lat.is_contiguous(), "out_lat must be contiguous [B, n_h, 512]")
    _require(wkv_b.dtype == out_lat.dtype and wkv_b.is_contiguous() and
             tuple(wkv_b.shape) == (n_h * 256, 512), "wkv_b must be contiguous [n_h*256, 512]")
    if out is None:
        out = torch.empty((B, n_h, 128), dtype=out_lat.dtype, device=out_lat.device)
    _require(out.dtype == out_lat.dtype and out.is_contiguous() and
             tuple(out.shape) == (B, n_h, 128), "out must be contiguous [B, n_h, 128]")
    _check("mla_out_up", library().mla_out_up(
        _ptr(out_lat), _ptr(wkv_b), _ptr(out), B, n_h, _dtype_code(out_lat), _stream(stream)))
    return out


def mla_kv_reconstruct(c: torch.Tensor, k_rope: torch.Tensor, wkv_b: torch.Tensor,
                       K: torch.Tensor = None, V: torch.Tensor = None, stream=None):
    """(K [N, n_h, 192], V [N, n_h, 128]) from c [N, 512], k_rope [N, 64]."""
    _dev(c, k_rope, wkv_b, K, V)
    N, d = c.shape
    _require(d == 512 and c.is_contiguous(), "c must be contiguous [N, 512]")
    _require(k_rope.dtype == c.dtype and k_rope.is_contiguous() and
             tuple(k_rope.shape) == (N, 64), "k_rope must be contiguous [N, 64]")
    _require(wkv_b.dtype == c.dtype and wkv_b.is_contiguous() and wkv_b.dim() == 2 and
             wkv_b.shape[1] == 512 and wkv_b.shape[0] % 256 == 0,
             "wkv_b must be contiguous [n_h*256, 512]")
    n_h = wkv_b.shape[0] // 256
    if K is None:
        K = torch.empty((N, n_h, 192), dtype=c.dtype, device=c.device)
    if V is None:
        V = torch.empty((N, n_h, 128), dtype=c.dtype, device=c.device)
    _require(K.dtype == c.dtype and K.is_contiguous() and tuple(K.shape) == (N, n_h, 192),
             "K must be contiguous [N, n_h, 192]")
    _require(V.dtype == c.dtype and V.is_contiguous() and tuple(V.shape) == (N, n_h, 128),
             "V must be contiguous [N, n_h, 128]")
    _check("mla_kv_reconstruct", library().mla_kv_reconstruct(
        _ptr(c), _ptr(k_rope), _ptr(wkv_b), _ptr(K), _ptr(V), N, n_h, _dtype_code(c),
        _stream(stream)))
    return K, V


def mla_softmax_scale(qk_head_dim: int = 192, max_seq_len: int = 0, original_seq_len: int = 0,
                      mscale: float = 1.0, rope_factor: float = 1.0) -> float:
    """The attention scale (with the YaRN factor when max_seq_len exceeds
    original_seq_len); see include/mla.h."""
    return library().mla_softmax_scale(qk_head_dim, max_seq_len, original_seq_len, mscale,
                                       rope_factor)


def mla_cache_append(kv_a: torch.Tensor, gamma: torch.Tensor, freqs: torch.Tensor,
                     pos: torch.Tensor, latent: torch.Tensor, rope: torch.Tensor,
                     seq_idx: torch.Tensor = None, eps: float = 1e-6, stream=None):
    """Write RMSNorm(kv_a[n, :512]) * gamma and the rotated kv_a[n, 512:576]
    into latent[s, pos[n]] and rope[s, pos[n]] (s = seq_idx[n], or n).

    kv_a [N, >=576] with unit stride in the last dim (the down-projection
    output, latent features first); gamma [512] float32; freqs [n_pos, 32, 2]
    float32 (cos, sin) per position and rotary pair; latent [B, T, 512] and
    rope [B, T, 64] caches (views of a packed [B, T, 576] cache allowed).
    Rows addressed outside the caches or the table are skipped. Returns
    (latent, rope).
    """
    _dev(kv_a, gamma, freqs, pos, latent, rope, seq_idx)
    _require(kv_a.dim() == 2 and kv_a.stride(1) == 1 and kv_a.shape[1] >= 576,
             "kv_a must be [N, >=576] with unit stride in the last dim")
    N = kv_a.shape[0]
    _require(gamma.dtype == torch.float32 and gamma.is_contiguous() and
             tuple(gamma.shape) == (512,), "gamma must be contiguous float32 [512]")
    _require(freqs.dtype == torch.float32 and freqs.is_contiguous() and freqs.dim() == 3 and
             tuple(freqs.shape[1:]) == (32, 2), "freqs must be contiguous float32 [n_pos, 32, 2]")
    _require(pos.dtype == torch.int32 and pos.is_contiguous() and tuple(pos.shape) == (N,),
             "pos must be contiguous int32 [N]")
    if seq_idx is not None:
        _require(seq_idx.dtype == torch.int32 and seq_idx.is_contiguous() and
                 tuple(seq_idx.shape) == (N,), "seq_idx must be contiguous int32 [N]")
    _require(latent.dtype == kv_a.dtype and rope.dtype == kv_a.dtype, "dtype mismatch")
    lbs, lrs = _cache_strides(latent, 512, "latent")
    rbs, rrs = _cache_strides(rope, 64, "rope")
    B_cache = min(latent.shape[0], rope.shape[0])
    T_cache = min(latent.shape[1], rope.shape[1])
    _check("mla_cache_append", library().mla_cache_append(
        _ptr(kv_a), kv_a.stride(0), _ptr(gamma), float(eps), _ptr(freqs), freqs.shape[0],
        _ptr(seq_idx), _ptr(pos), N, _ptr(latent), _ptr(rope), lbs, lrs, rbs, rrs, B_cache,
        T_cache, _dtype_code(kv_a), _stream(stream)))
    return latent, rope


def mla_attention_naive_workspace_bytes(B: int, S: int, T: int, K: int = 0) -> int:
    v = library().mla_attention_naive_workspace_bytes(B, S, T, K)
    if v == ctypes.c_size_t(-1).value:
        raise MLAError("mla_attention_naive_workspace_bytes", 1, "arguments rejected")
    return v


def mla_attention_naive(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        topk_idx: torch.Tensor = None, causal: bool = False,
                        scale: float = SCALE, out: torch.Tensor = None, lse: torch.Tensor = None,
                        workspace: torch.Tensor = None, want_lse: bool = False, stream=None):
    """Ordinary attention over reconstructed keys and values: q [B, S, n_h,
    192], k [B, T, n_h, 192], v [B, T, n_h, 128] (k, v as written by
    mla_kv_reconstruct for N = B*T tokens, viewed per sequence); topk_idx
    int32 [B, S, K] (one index set per query) or None; causal: query s sees
    keys up to T - S + s. Returns out [B, S, n_h, 128] (and lse [B, S, n_h])."""
    _dev(q, k, v, topk_idx, out, lse, workspace)
    _require(q.dim() == 4 and q.shape[3] == 192 and q.is_contiguous(),
             "q must be contiguous [B, S, n_h, 192]")
    B, S, n_h, _ = q.shape
    _require(k.dtype == q.dtype and k.is_contiguous() and k.dim() == 4 and k.shape[0] == B and
             k.shape[2] == n_h and k.shape[3] == 192, "k must be contiguous [B, T, n_h, 192]")
    T = k.shape[1]
    _require(v.dtype == q.dtype and v.is_contiguous() and tuple(v.shape) == (B, T, n_h, 128),
             "v must be contiguous [B, T, n_h, 128]")
    K = 0
    if topk_idx is not None:
        _require(topk_idx.dtype == torch.int32 and topk_idx.is_contiguous() and
                 topk_idx.dim() == 3 and tuple(topk_idx.shape[:2]) == (B, S),
                 "topk_idx must be contiguous int32 [B, S, K]")
        K = topk_idx.shape[2]
    if out is None:
        out = torch.empty((B, S, n_h, 128), dtype=q.dtype, device=q.device)
    _require(out.dtype == q.dtype and out.is_contiguous() and tuple(out.shape) == (B, S, n_h, 128),
             "out must be contiguous [B, S, n_h, 128]")
    if lse is None and want_lse:
        lse = torch.empty((B, S, n_h), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and
                 tuple(lse.shape) == (B, S, n_h), "lse must be contiguous float32 [B, S, n_h]")
    need = mla_attention_naive_workspace_bytes(B, S, T, K) if B > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_attention_naive", library().mla_attention_naive(
        _ptr(q), _ptr(k), _ptr(v), B, S, T, n_h, _ptr(topk_idx), K, int(bool(causal)),
        float(scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _dtype_code(q),
        _stream(stream)))
    return (out, lse) if (want_lse or lse is not None) else out
