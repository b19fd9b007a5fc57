"""fp64 CPU oracle for multi-head latent attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never loads it, and it
imports nothing from the GPU package: the two share no code.

This module is argument marshalling over ``liboracle.so`` (plain C, double
precision, see ``mla_oracle.c`` for the formulas and the pages they follow).
Inputs are numpy arrays (float32, float64, uint16 holding bfloat16 bits,
uint8 holding e4m3 codes, int32 indices) or CPU torch tensors of those
types; outputs are float64 numpy arrays.

Parity status (all pinned by ``tests/test_oracle_*.py``):
  dequant_fp8_block   pinned: torch e4m3fn decode, torch fp32*scale->bf16
  absorb_q, out_up    pinned: naive/absorbed identity, closed forms
  latent_attention    pinned: naive/absorbed identity, closed forms,
                      permutation invariance, hand-computed tiny case
  decode_absorbed     pinned: equals decode_naive; closed forms
  decode_naive        pinned: torch scaled_dot_product_attention (double)
  kv_reconstruct      pinned: structured weights with a closed form
  latent_attention_multi  pinned: s_q = 1 case, per-token reduction to
                      latent_attention (causal prefix / full), hand corner
  attention_naive     pinned: torch SDPA (double) with the same mask, first
                      causal row, one-query reduction to decode_naive
  cache_append        pinned: RMSNorm closed forms (constant, scaled, unit
                      RMS), rotation by quarter turns, composition, pairing
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2

# dimensions of the model the pages describe (defaults of every call)
D_C, D_R, D_N, D_V = 512, 64, 128, 128

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = D
        lib.orc_f64_to_bf16.argtypes = [D]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_f64.restype = D
        lib.orc_dequant_fp8_block.argtypes = [P, P, L, L, P]
        lib.orc_absorb_q.argtypes = [P, I, P, I, I, I, I, I, I, P]
        lib.orc_latent_attention.argtypes = [P, I, P, I, P, P, I, L, L, L, L, I, I, I, I,
                                             I, P, I, D, P, P, P]
        lib.orc_out_up.argtypes = [P, I, P, I, I, I, I, I, I, P]
        lib.orc_decode_absorbed.argtypes = [P, P, I, P, P, I, L, L, L, L, P, I, I, I, I,
                                            I, I, I, I, P, I, D, P, P, P, P]
        lib.orc_kv_reconstruct.argtypes = [P, P, I, P, I, L, I, I, I, I, I, P, P]
        lib.orc_decode_naive.argtypes = [P, P, I, P, P, I, L, L, L, L, P, I, I, I, I,
                                         I, I, I, I, P, I, D, P, P]
        lib.orc_softmax_scale.argtypes = [I, L, L, D, D]
        lib.orc_softmax_scale.restype = D
        lib.orc_latent_attention_multi.argtypes = [P, I, P, I, P, P, I, L, L, L, L, I, I, I,
                                                   I, I, I, P, I, I, D, P, P]
        lib.orc_attention_naive.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, I, D, P, P]
        lib.orc_cache_append.argtypes = [P, P, I, P, P, P, L, L, I, I, D, P, P]
        for name in ("orc_dequant_fp8_block", "orc_absorb_q", "orc_latent_attention",
                     "orc_out_up", "orc_decode_absorbed", "orc_kv_reconstruct",
                     "orc_decode_naive", "orc_cache_append",
                     "orc_latent_attention_multi", "orc_attention_naive"):
            getattr(lib, name).restype = I
        _lib = lib
    return _lib


def _np(x):
    """numpy view of an array or CPU torch tensor (bf16 -> uint16 bits)."""
    if isinstance(x, np.ndarray):
        return x
    import torch  # only for tensor inputs
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return x.contiguous().view(torch.int16).numpy().view(np.uint16)
        return x.contiguous().numpy()
    return np.asarray(x)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported element type {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_f64(bits)


def f64_to_bf16(x: float) -> int:
    """bfloat16 bits nearest (ties to even) to x."""
    return _load().orc_f64_to_bf16(float(x))


def e4m3_to_f64(code: int) -> float:
    return _load().orc_e4m3_to_f64(code)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of an array of bfloat16 bits."""
    b = np.ascontiguousarray(_np(bits)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_fp8_block(w_fp8, scale) -> np.ndarray:
    """bf16 bits [rows, cols] of decode(w) * scale[i/128, j/128]."""
    w = np.ascontiguousarray(_np(w_fp8), dtype=np.uint8)
    s = np.ascontiguousarray(_np(scale), dtype=np.float32)
    rows, cols = w.shape
    assert s.shape == ((rows + 127) // 128, (cols + 127) // 128)
    out = np.empty((rows, cols), np.uint16)
    _check(_load().orc_dequant_fp8_block(_ptr(w), _ptr(s), rows, cols, _ptr(out)), "dequant")
    return out


def absorb_q(q_nope, w, d_n=D_N, d_v=D_V) -> np.ndarray:
    q = np.ascontiguousarray(_np(q_nope))
    W = np.ascontiguousarray(_np(w))
    B, n_h, dn = q.shape
    assert dn == d_n and W.shape[0] == n_h * (d_n + d_v)
    d_c = W.shape[1]
    out = np.empty((B, n_h, d_c), np.float64)
    _check(_load().orc_absorb_q(_ptr(q), _dt(q), _ptr(W), _dt(W), B, n_h, d_n, d_v, d_c,
                                _ptr(out)), "absorb_q")
    return out


def out_up(o_lat, w, d_n=D_N, d_v=D_V) -> np.ndarray:
    o = np.ascontiguousarray(_np(o_lat))
    W = np.ascontiguousarray(_np(w))
    B, n_h, d_c = o.shape
    assert W.shape == (n_h * (d_n + d_v), d_c)
    out = np.empty((B, n_h, d_v), np.float64)
    _check(_load().orc_out_up(_ptr(o), _dt(o), _ptr(W), _dt(W), B, n_h, d_n, d_v, d_c,
                              _ptr(out)), "out_up")
    return out


def _cache_args(latent, rope):
    """latent [B,Tmax,d_c] and rope [B,Tmax,d_r] arrays (any dense layout)."""
    lat = np.ascontiguousarray(_np(latent))
    rp = np.ascontiguousarray(_np(rope))
    assert lat.dtype == rp.dtype and lat.shape[:2] == rp.shape[:2]
    return lat, rp, lat.shape[1] * lat.shape[2], lat.shape[2], rp.shape[1] * rp.shape[2], rp.shape[2]


def _idx_args(topk_idx, B):
    if topk_idx is None:
        return None, 0
    idx = np.ascontiguousarray(_np(topk_idx), dtype=np.int32)
    assert idx.ndim == 2 and idx.shape[0] == B
    return idx, idx.shape[1]


def split_packed(cache, d_c=D_C):
    """Views of a packed [B, T, d_c + d_r] cache as (latent, rope) arrays."""
    c = _np(cache)
    return c[..., :d_c], c[..., d_c:]


def latent_attention(q_lat, q_pe, latent, rope, T=None, topk_idx=None, scale=192 ** -0.5,
                     want_lse=False, want_probs=False):
    """(out_lat [B,n_h,d_c], lse [B,n_h] | None, probs [B,n_h,T] | None)."""
    ql = np.ascontiguousarray(_np(q_lat))
    qp = np.ascontiguousarray(_np(q_pe))
    lat, rp, lbs, lrs, rbs, rrs = _cache_args(latent, rope)
    B, n_h, d_c = ql.shape
    d_r = qp.shape[2]
    T = lat.shape[1] if T is None else T
    idx, K = _idx_args(topk_idx, B)
    o = np.empty((B, n_h, d_c), np.float64)
    lse = np.empty((B, n_h), np.float64) if want_lse else None
    probs = np.empty((B, n_h, T), np.float64) if want_probs else None
    _check(_load().orc_latent_attention(_ptr(ql), _dt(ql), _ptr(qp), _dt(qp), _ptr(lat),
                                        _ptr(rp), _dt(lat), lbs, lrs, rbs, rrs, B, n_h, T,
                                        d_c, d_r, _ptr(idx), K, float(scale), _ptr(o),
                                        _ptr(lse), _ptr(probs)), "latent_attention")
    return o, lse, probs


def latent_attention_multi(q_lat, q_pe, latent, rope, T=None, topk_idx=None,
                           scale=192 ** -0.5, causal=False):
    """Several query tokens per sequence: q_lat [B,s_q,n_h,d_c], q_pe
    [B,s_q,n_h,d_r]; T counts the cached positions including the s_q new
    tokens. Returns (out_lat [B,s_q,n_h,d_c], lse [B,s_q,n_h])."""
    ql = np.ascontiguousarray(_np(q_lat))
    qp = np.ascontiguousarray(_np(q_pe))
    lat, rp, lbs, lrs, rbs, rrs = _cache_args(latent, rope)
    B, s_q, n_h, d_c = ql.shape
    d_r = qp.shape[3]
    T = lat.shape[1] if T is None else T
    idx, K = _idx_args(topk_idx, B)
    o = np.empty((B, s_q, n_h, d_c), np.float64)
    lse = np.empty((B, s_q, n_h), np.float64)
    _check(_load().orc_latent_attention_multi(_ptr(ql), _dt(ql), _ptr(qp), _dt(qp), _ptr(lat),
                                              _ptr(rp), _dt(lat), lbs, lrs, rbs, rrs, B, s_q,
                                              n_h, T, d_c, d_r, _ptr(idx), K, int(causal),
                                              float(scale), _ptr(o), _ptr(lse)),
           "latent_attention_multi")
    return o, lse


def decode_absorbed(q_nope, q_pe, latent, rope, w, T=None, topk_idx=None,
                    scale=192 ** -0.5, d_n=D_N, d_v=D_V, want_olat=False, want_lse=False,
                    want_probs=False):
    """Whole absorbed decode in double. Returns dict with 'out' and optionals."""
    qn = np.ascontiguousarray(_np(q_nope))
    qp = np.ascontiguousarray(_np(q_pe))
    assert qn.dtype == qp.dtype
    W = np.ascontiguousarray(_np(w))
    lat, rp, lbs, lrs, rbs, rrs = _cache_args(latent, rope)
    B, n_h, _ = qn.shape
    d_c, d_r = lat.shape[2], rp.shape[2]
    T = lat.shape[1] if T is None else T
    idx, K = _idx_args(topk_idx, B)
    out = np.empty((B, n_h, d_v), np.float64)
    o = np.empty((B, n_h, d_c), np.float64) if want_olat else None
    lse = np.empty((B, n_h), np.float64) if want_lse else None
    probs = np.empty((B, n_h, T), np.float64) if want_probs else None
    _check(_load().orc_decode_absorbed(_ptr(qn), _ptr(qp), _dt(qn), _ptr(lat), _ptr(rp),
                                       _dt(lat), lbs, lrs, rbs, rrs, _ptr(W), _dt(W), B,
                                       n_h, T, d_c, d_r, d_n, d_v, _ptr(idx), K,
                                       float(scale), _ptr(out), _ptr(o), _ptr(lse),
                                       _ptr(probs)), "decode_absorbed")
    return {"out": out, "o_lat": o, "lse": lse, "probs": probs}


def decode_naive(q_nope, q_pe, latent, rope, w, T=None, topk_idx=None, scale=192 ** -0.5,
                 d_n=D_N, d_v=D_V, want_probs=False):
    """Reconstruct-then-attend decode in double. Returns dict with 'out'."""
    qn = np.ascontiguousarray(_np(q_nope))
    qp = np.ascontiguousarray(_np(q_pe))
    assert qn.dtype == qp.dtype
    W = np.ascontiguousarray(_np(w))
    lat, rp, lbs, lrs, rbs, rrs = _cache_args(latent, rope)
    B, n_h, _ = qn.shape
    d_c, d_r = lat.shape[2], rp.shape[2]
    T = lat.shape[1] if T is None else T
    idx, K = _idx_args(topk_idx, B)
    out = np.empty((B, n_h, d_v), np.float64)
    probs = np.empty((B, n_h, T), np.float64) if want_probs else None
    _check(_load().orc_decode_naive(_ptr(qn), _ptr(qp), _dt(qn), _ptr(lat), _ptr(rp),
                                    _dt(lat), lbs, lrs, rbs, rrs, _ptr(W), _dt(W), B, n_h,
                                    T, d_c, d_r, d_n, d_v, _ptr(idx), K, float(scale),
                                    _ptr(out), _ptr(probs)), "decode_naive")
    return {"out": out, "probs": probs}


def kv_reconstruct(c, k_rope, w, n_h, d_n=D_N, d_v=D_V):
    """(K [N,n_h,d_n+d_r], V [N,n_h,d_v]) in double."""
    cc = np.ascontiguousarray(_np(c))
    kr = np.ascontiguousarray(_np(k_rope))
    assert cc.dtype == kr.dtype
    W = np.ascontiguousarray(_np(w))
    N, d_c = cc.shape
    d_r = kr.shape[1]
    assert W.shape == (n_h * (d_n + d_v), d_c)
    K = np.empty((N, n_h, d_n + d_r), np.float64)
    V = np.empty((N, n_h, d_v), np.float64)
    _check(_load().orc_kv_reconstruct(_ptr(cc), _ptr(kr), _dt(cc), _ptr(W), _dt(W), N, n_h,
                                      d_c, d_r, d_n, d_v, _ptr(K), _ptr(V)), "kv_reconstruct")
    return K, V


def softmax_scale(qk_head_dim=192, max_seq_len=0, original_seq_len=0, mscale=1.0,
                  rope_factor=1.0) -> float:
    """Attention scale of the mla-init excerpt (YaRN extension when
    max_seq_len > original_seq_len), in double."""
    return _load().orc_softmax_scale(qk_head_dim, max_seq_len, original_seq_len,
                                     float(mscale), float(rope_factor))


def cache_append(kv, k_pe, gamma, freqs, pos, eps=1e-6):
    """(latent rows [N,d_c], rotary rows [N,d_r]) in double: RMSNorm of the
    latent with gain gamma, and the rotary key rotated pairwise by the table
    row freqs[pos[n]] ((cos, sin) per pair)."""
    x = np.ascontiguousarray(_np(kv))
    r = np.ascontiguousarray(_np(k_pe))
    assert x.dtype == r.dtype and x.shape[0] == r.shape[0]
    g = np.ascontiguousarray(_np(gamma), dtype=np.float32)
    f = np.ascontiguousarray(_np(freqs), dtype=np.float32)
    p = np.ascontiguousarray(_np(pos), dtype=np.int32)
    N, d_c = x.shape
    d_r = r.shape[1]
    assert g.shape == (d_c,) and f.shape[1:] == (d_r // 2, 2) and p.shape == (N,)
    lat = np.empty((N, d_c), np.float64)
    rope = np.empty((N, d_r), np.float64)
    _check(_load().orc_cache_append(_ptr(x), _ptr(r), _dt(x), _ptr(g), _ptr(f), _ptr(p), N,
                                    f.shape[0], d_c, d_r, float(eps), _ptr(lat), _ptr(rope)),
           "cache_append")
    return lat, rope


def attention_naive(q, k, v, topk_idx=None, causal=False, scale=192 ** -0.5):
    """Ordinary attention over reconstructed keys and values: q [B,S,n_h,d_qk],
    k [B,T,n_h,d_qk], v [B,T,n_h,d_v]; topk_idx int32 [B,S,K] (one index set
    per query token) or None; causal: query s sees t <= T - S + s.
    Returns (out [B,S,n_h,d_v], lse [B,S,n_h]) in double."""
    qq = np.ascontiguousarray(_np(q))
    kk = np.ascontiguousarray(_np(k))
    vv = np.ascontiguousarray(_np(v))
    assert qq.dtype == kk.dtype == vv.dtype
    B, S, n_h, d_qk = qq.shape
    T = kk.shape[1]
    assert kk.shape == (B, T, n_h, d_qk) and vv.shape[:3] == (B, T, n_h)
    d_v = vv.shape[3]
    K = 0
    idx = None
    if topk_idx is not None:
        idx = np.ascontiguousarray(_np(topk_idx), dtype=np.int32)
        assert idx.shape[:2] == (B, S)
        K = idx.shape[2]
    out = np.empty((B, S, n_h, d_v), np.float64)
    lse = np.empty((B, S, n_h), np.float64)
    _check(_load().orc_attention_naive(_ptr(qq), _ptr(kk), _ptr(vv), _dt(qq), B, S, T, n_h,
                                       d_qk, d_v, _ptr(idx), K, int(causal), float(scale),
                                       _ptr(out), _ptr(lse)), "attention_naive")
    return out, lse
