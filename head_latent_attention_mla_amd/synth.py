"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic (no absorption, scores, softmax, mixing, up-projection
or dequantisation). Tensors are CPU torch tensors; callers copy them to the
device or hand them to the oracle.

Recipe (one numpy PCG64 stream per tensor, spawned from one SeedSequence,
in the fixed order latent, rope, q_nope, q_pe, wkv_b, scales, top-k, then
the stand-alone stage inputs q_lat and o_lat, then the cache-append inputs
kv_a, gain, angles, positions):
  latent   rows of 512 standard normals, each scaled (float64) to a root
           mean square of exactly 1: a uniformly random direction on the
           sphere of radius sqrt(512), which is how an RMS-normalised
           standard normal row with unit gain is distributed (the eps of the
           norm moves the RMS by ~1e-6). Drawing it this way is sampling,
           not the cache-append arithmetic (no gain, no eps).
  rope     ~ N(0,1)           (already-rotated shared key)
  q_nope   ~ N(0,1), q_pe ~ N(0,1)
  wkv_b    ~ N(0, 1/512)  [n_h*256, 512], stored [out, in]
  fp8      wkv_b / scale[block] cast to e4m3fn by torch (round to nearest),
           scales ~ U[0.5, 2] * 2^-4 per 128x128 block
  top-k    per sequence, K distinct positions drawn uniformly without
           replacement from [0, T), unsorted
  q_lat    ~ N(0, 1/4)  (the spread of q_nope @ W^UK for the above)
  o_lat    ~ N(0, 1)
  kv_a     down-projection output rows [N, 576] ~ N(0,1) times a per-row
           scale 2^U[-2, 3] (unnormalised activations of varied size)
  gain     RMSNorm gain [512] ~ U[0.5, 1.5]
  angles   rotation table [n_pos, 32]: angles ~ U[-pi, pi), stored as
           float32 (cos, sin) pairs
  pos      per row: the sequence's current length, ~ U[0, T) (decode), or
           consecutive positions (prefill)
  q, k, v  per-head queries [B,S,n_h,192], keys [B,T,n_h,192] and values
           [B,T,n_h,128] of the naive path ~ N(0,1) (the spread of the
           reconstructed k_nope / v for the weights above, and of k^R)
  sets     per query token, K distinct key positions: drawn uniformly from
           the keys the query may see (t <= T - S + s under the causal mask)
           and, when fewer than K are visible, topped up with hidden ones (as
           a top-k over masked scores would)
Values are rounded once to the storage type (bf16 round-to-nearest-even via
torch, or kept float32).
"""
from __future__ import annotations

import numpy as np
import torch

D_C, D_R, D_N, D_V = 512, 64, 128, 128
SCALE = 192 ** -0.5

_ORDER = ("latent", "rope", "q_nope", "q_pe", "wkv_b", "scales", "topk", "q_lat", "o_lat",
          "kv_a", "gain", "angles", "pos", "q", "k", "v", "sets")


def _streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(_ORDER))
    return {k: np.random.Generator(np.random.PCG64(s)) for k, s in zip(_ORDER, children)}


def _normal(g, shape, std=1.0):
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _unit_rms_rows(g, shape):
    x = g.standard_normal(size=shape, dtype=np.float32)
    ms = np.einsum("...i,...i->...", x, x, dtype=np.float64) / shape[-1]
    x *= (1.0 / np.sqrt(ms)).astype(np.float32)[..., None]
    return x


def _store(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t if dtype == torch.float32 else t.to(dtype)


def decode_inputs(B: int, n_h: int, T: int, dtype=torch.bfloat16, seed: int = 0,
                  topk: int | None = None, fp8_weights: bool = False,
                  stage_inputs: bool = False) -> dict:
    """Inputs of one absorbed decode step.

    Returns a dict with
      cache  [B, T, 576] packed (latent 0..511, rope 512..575), dtype
      q_nope [B, n_h, 128], q_pe [B, n_h, 64], dtype
      wkv_b  [n_h*256, 512] dtype (absent when fp8_weights)
      wkv_b_fp8 uint8 [n_h*256, 512] and wkv_b_scale float32 [n_h*2, 4]
             (when fp8_weights)
      topk_idx int32 [B, topk] (when topk)
      q_lat [B, n_h, 512], o_lat [B, n_h, 512] (when stage_inputs)
    """
    g = _streams(seed)
    cache = np.empty((B, T, D_C + D_R), np.float32)
    cache[..., :D_C] = _unit_rms_rows(g["latent"], (B, T, D_C))
    cache[..., D_C:] = _normal(g["rope"], (B, T, D_R))
    out = {
        "cache": _store(cache, dtype),
        "q_nope": _store(_normal(g["q_nope"], (B, n_h, D_N)), dtype),
        "q_pe": _store(_normal(g["q_pe"], (B, n_h, D_R)), dtype),
    }
    del cache
    w = _normal(g["wkv_b"], (n_h * (D_N + D_V), D_C), std=512 ** -0.5)
    if fp8_weights:
        rows, cols = w.shape
        sr, sc = (rows + 127) // 128, (cols + 127) // 128
        scales = ((g["scales"].uniform(0.5, 2.0, size=(sr, sc)) * 2.0 ** -4)
                  .astype(np.float32))
        full = np.repeat(np.repeat(scales, 128, axis=0), 128, axis=1)[:rows, :cols]
        q = torch.from_numpy(w / full).to(torch.float8_e4m3fn)
        out["wkv_b_fp8"] = q.view(torch.uint8).contiguous()
        out["wkv_b_scale"] = torch.from_numpy(scales)
    else:
        out["wkv_b"] = _store(w, dtype)
    if topk is not None:
        idx = np.stack([g["topk"].choice(T, size=topk, replace=False) for _ in range(B)])
        out["topk_idx"] = torch.from_numpy(idx.astype(np.int32))
    if stage_inputs:
        out["q_lat"] = _store(_normal(g["q_lat"], (B, n_h, D_C), std=0.5), dtype)
        out["o_lat"] = _store(_normal(g["o_lat"], (B, n_h, D_C)), dtype)
    return out


def reconstruct_inputs(N: int, n_h: int, dtype=torch.bfloat16, seed: int = 0) -> dict:
    """c [N, 512], k_rope [N, 64], wkv_b [n_h*256, 512]."""
    g = _streams(seed)
    return {
        "c": _store(_unit_rms_rows(g["latent"], (N, D_C)), dtype),
        "k_rope": _store(_normal(g["rope"], (N, D_R)), dtype),
        "wkv_b": _store(_normal(g["wkv_b"], (n_h * (D_N + D_V), D_C), std=512 ** -0.5), dtype),
    }


def append_inputs(N: int, B: int, T: int, dtype=torch.bfloat16, seed: int = 0,
                  prefill: bool = False, n_pos: int | None = None) -> dict:
    """Inputs of one cache append.

    Decode (prefill=False): N <= B rows, row n is the new token of sequence n
    at position pos[n] ~ U[0, T). Prefill: N = B * (N // B) rows, sequence
    n // (N // B), consecutive positions from a random start so that the
    block fits in [0, T). Returns kv_a [N, 576] (dtype), gamma [512] f32,
    freqs [n_pos, 32, 2] f32 (cos, sin), pos [N] int32 and, for prefill,
    seq_idx [N] int32.
    """
    g = _streams(seed)
    n_pos = T if n_pos is None else n_pos
    scale = np.exp2(g["kv_a"].uniform(-2.0, 3.0, size=(N, 1))).astype(np.float32)
    kv_a = _normal(g["kv_a"], (N, D_C + D_R)) * scale
    theta = g["angles"].uniform(-np.pi, np.pi, size=(n_pos, D_R // 2))
    freqs = np.stack([np.cos(theta), np.sin(theta)], -1).astype(np.float32)
    out = {
        "kv_a": _store(kv_a, dtype),
        "gamma": torch.from_numpy(g["gain"].uniform(0.5, 1.5, size=D_C).astype(np.float32)),
        "freqs": torch.from_numpy(np.ascontiguousarray(freqs)),
    }
    if prefill:
        per = N // B
        assert per * B == N and per <= T
        start = g["pos"].integers(0, T - per + 1, size=B)
        out["pos"] = torch.from_numpy((start[:, None] + np.arange(per)).reshape(-1).astype(np.int32))
        out["seq_idx"] = torch.from_numpy(np.repeat(np.arange(B), per).astype(np.int32))
    else:
        assert N <= B
        out["pos"] = torch.from_numpy(g["pos"].integers(0, T, size=N).astype(np.int32))
    return out


def attention_inputs(B: int, S: int, T: int, n_h: int, dtype=torch.bfloat16, seed: int = 0,
                     topk: int | None = None, causal: bool = True) -> dict:
    """q [B,S,n_h,192], k [B,T,n_h,192], v [B,T,n_h,128] and, with topk,
    topk_idx int32 [B,S,topk] (one set per query token)."""
    g = _streams(seed)
    out = {
        "q": _store(_normal(g["q"], (B, S, n_h, D_N + D_R)), dtype),
        "k": _store(_normal(g["k"], (B, T, n_h, D_N + D_R)), dtype),
        "v": _store(_normal(g["v"], (B, T, n_h, D_V)), dtype),
    }
    if topk is not None:
        assert 1 <= topk <= T
        idx = np.empty((B, S, topk), np.int32)
        for b in range(B):
            # random priorities; visible keys first, then hidden ones
            pri = g["sets"].random((S, T), dtype=np.float32)
            if causal:
                hidden = np.arange(T)[None, :] > (T - S + np.arange(S))[:, None]
                pri = pri + hidden.astype(np.float32) * 2.0
            idx[b] = np.argpartition(pri, topk - 1, axis=1)[:, :topk]
        out["topk_idx"] = torch.from_numpy(idx)
    return out


def fp8_codes(rows: int, cols: int, seed: int = 0, with_nan: bool = False) -> torch.Tensor:
    """Uniformly random e4m3 byte codes (NaN codes 0x7F/0xFF excluded unless
    with_nan): exercises every code, including subnormals and +-448."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    codes = g.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    if not with_nan:
        codes[(codes & 0x7F) == 0x7F] = 0x7E
    return torch.from_numpy(codes)


# The five workloads the hot path is specified and measured on.
CONFIGS = {
    1: dict(kind="decode", B=1, n_h=16, T=128, dtype=torch.float32, seed=1001,
            name="tiny fp32 decode B=1 n_h=16 T=128"),
    2: dict(kind="decode", B=32, n_h=128, T=4096, dtype=torch.bfloat16, seed=1002,
            name="absorbed decode bf16 B=32 n_h=128 T=4096"),
    3: dict(kind="decode", B=4, n_h=128, T=32768, dtype=torch.bfloat16, seed=1003,
            name="long-context absorbed decode bf16 B=4 n_h=128 T=32768"),
    4: dict(kind="decode", B=8, n_h=128, T=65536, dtype=torch.bfloat16, seed=1004,
            topk=2048, fp8_weights=True,
            name="sparse top-2048 decode, fp8 wkv_b, B=8 n_h=128 T=65536"),
    5: dict(kind="reconstruct", N=8192, n_h=128, dtype=torch.bfloat16, seed=1005,
            name="naive KV reconstruction bf16 N=8192 n_h=128"),
}


def config_inputs(cfg: int, **overrides) -> dict:
    c = dict(CONFIGS[cfg])
    c.update(overrides)
    if c["kind"] == "reconstruct":
        return reconstruct_inputs(c["N"], c["n_h"], c["dtype"], c["seed"])
    return decode_inputs(c["B"], c["n_h"], c["T"], c["dtype"], c["seed"],
                         topk=c.get("topk"), fp8_weights=c.get("fp8_weights", False))
