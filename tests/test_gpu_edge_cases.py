"""GPU parity on the degenerate shapes of every entry point, against the fp64
oracle: one head, a head group holding a single real head, one cached row,
one row past a tile boundary, index sets of one row and of every row, one
query against one key, and empty batches (a no-op that leaves the outputs
untouched).

Bar as in the other parity tests: max|err| <= 2e-2 * max|ref| (bf16) or
1e-5 * max|ref| (fp32), for outputs and log-sum-exp alike; the k^R copy
inside K is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_mla_amd import binding as mla
from head_latent_attention_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
DTYPES = [torch.bfloat16, torch.float32]


def f64(t):
    return t.detach().cpu().double().numpy()


def check(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    m = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    assert err <= tol * m, f"{what}: max|err| {err:.3e} > {tol} * {m:.3e}"


# --------------------------------------------------------------------------
# latent attention (one query token)
# --------------------------------------------------------------------------

DECODE_EDGE = [
    # B, n_h, T, topk K, splits
    (3, 1, 1, None, 0),      # one head, one cached row
    (2, 1, 100, 1, 0),       # one head, an index set of one row
    (2, 1, 700, None, 5),    # one head, five splits
    (2, 129, 65, None, 0),   # second 128-head group holds one head; one row past two tiles
    (1, 16, 33, None, 0),    # one row past a tile
    (1, 1, 50, 50, 0),       # index set of every row, in random order
    (4, 2, 2, 2, 1),
]


@pytest.mark.parametrize("B,n_h,T,K,splits", DECODE_EDGE)
@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_edge_shapes(B, n_h, T, K, splits, dtype):
    inp = synth.decode_inputs(B, n_h, T, dtype, seed=B * 997 + n_h * 31 + T, topk=K,
                              stage_inputs=True)
    idx = inp.get("topk_idx")
    cache = inp["cache"].to(DEV)
    out, lse = mla.mla_decode_latent_attn(inp["q_lat"].to(DEV), inp["q_pe"].to(DEV),
                                          cache[..., :512], cache[..., 512:],
                                          topk_idx=None if idx is None else idx.to(DEV),
                                          num_splits=splits, want_lse=True)
    ref, ref_lse, _ = oracle.latent_attention(inp["q_lat"], inp["q_pe"], inp["cache"][..., :512],
                                              inp["cache"][..., 512:], topk_idx=idx,
                                              want_lse=True)
    check(f64(out), ref, TOL[dtype], "out_lat")
    check(f64(lse), ref_lse, TOL[dtype], "lse")


def test_decode_single_row_returns_that_row():
    # one visible row: its weight is exactly 1, so the output is the row
    # itself (bf16 in, bf16 out: bit-exact)
    B, n_h = 2, 128
    inp = synth.decode_inputs(B, n_h, 1, torch.bfloat16, seed=17, stage_inputs=True)
    cache = inp["cache"].to(DEV)
    out = mla.mla_decode_latent_attn(inp["q_lat"].to(DEV), inp["q_pe"].to(DEV),
                                     cache[..., :512], cache[..., 512:])
    torch.cuda.synchronize()
    want = inp["cache"][:, 0, :512][:, None, :].expand(B, n_h, 512)
    assert torch.equal(out.cpu().view(torch.int16), want.contiguous().view(torch.int16))


# --------------------------------------------------------------------------
# absorb and W^UV with one head / one extra head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,n_h,dtype", [(1, 1, torch.bfloat16), (3, 1, torch.bfloat16),
                                         (2, 129, torch.bfloat16), (1, 1, torch.float32),
                                         (2, 3, torch.float32)])
def test_absorb_and_out_up_edge_heads(B, n_h, dtype):
    inp = synth.decode_inputs(B, n_h, 1, dtype, seed=B * 13 + n_h, stage_inputs=True)
    w = inp["wkv_b"].to(DEV)
    q_lat = mla.mla_absorb_q(inp["q_nope"].to(DEV), w)
    out = mla.mla_out_up(inp["o_lat"].to(DEV), w)
    check(f64(q_lat), oracle.absorb_q(inp["q_nope"], inp["wkv_b"]), TOL[dtype], "q_lat")
    check(f64(out), oracle.out_up(inp["o_lat"], inp["wkv_b"]), TOL[dtype], "out")


# --------------------------------------------------------------------------
# the one-call step: one head, one row, several tokens of one head
# --------------------------------------------------------------------------

def step_inputs(B, S_q, n_h, T, dtype, seed):
    base = synth.decode_inputs(B * S_q, n_h, 1, dtype, seed=seed, stage_inputs=True)
    cache = synth.decode_inputs(B, 1, T, dtype, seed=seed + 1)["cache"]
    return (base["q_nope"].reshape(B, S_q, n_h, 128).contiguous(),
            base["q_pe"].reshape(B, S_q, n_h, 64).contiguous(), base["wkv_b"], cache)


@pytest.mark.parametrize("B,S_q,n_h,T,causal", [(1, 1, 1, 1, False), (2, 1, 1, 1, True),
                                                (2, 3, 1, 3, True), (2, 1, 129, 70, False),
                                                (3, 2, 64, 2, True)])
@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_step_edge_shapes(B, S_q, n_h, T, causal, dtype):
    qn, qp, w, cache = step_inputs(B, S_q, n_h, T, dtype, seed=B * 71 + S_q * 7 + n_h + T)
    dc = cache.to(DEV)
    out, lse = mla.mla_decode_step(qn.to(DEV), qp.to(DEV), w.to(DEV), dc[..., :512], dc[..., 512:],
                                   causal=causal, want_lse=True)
    q_lat = oracle.absorb_q(qn.reshape(B * S_q, n_h, 128), w).reshape(B, S_q, n_h, 512)
    o, ref_lse = oracle.latent_attention_multi(q_lat, qp, cache[..., :512], cache[..., 512:],
                                               causal=causal)
    ref = oracle.out_up(o.reshape(B * S_q, n_h, 512), w).reshape(B, S_q, n_h, 128)
    check(f64(out), ref, TOL[dtype], "out")
    check(f64(lse), ref_lse, TOL[dtype], "lse")


# --------------------------------------------------------------------------
# naive-path attention: one query, one key, one head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,T,n_h,causal,topk", [
    (1, 1, 1, 1, True, None),    # one query against one key
    (2, 1, 1, 3, False, None),
    (1, 3, 1, 1, False, None),   # several queries, one key (no causal limit)
    (1, 1, 5, 1, True, 1),       # an index set of one key
    (1, 65, 65, 1, True, None),      # one key past a 64-key tile
    (1, 257, 257, 1, False, 257),    # every key in every set; one query past a 256-query block
])
@pytest.mark.parametrize("dtype", DTYPES)
def test_attention_naive_edge_shapes(B, S, T, n_h, causal, topk, dtype):
    inp = synth.attention_inputs(B, S, T, n_h, dtype, seed=S * 11 + T * 3 + n_h, topk=topk,
                                 causal=causal)
    idx = inp.get("topk_idx")
    out, lse = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                       topk_idx=None if idx is None else idx.to(DEV),
                                       causal=causal, want_lse=True)
    ref, ref_lse = oracle.attention_naive(inp["q"], inp["k"], inp["v"], topk_idx=idx,
                                          causal=causal)
    check(f64(out), ref, TOL[dtype], "out")
    check(f64(lse), ref_lse, TOL[dtype], "lse")


def test_attention_one_key_returns_its_value():
    # a single visible key carries weight 1: the output is its value row
    B, S, T, n_h = 1, 4, 1, 2
    inp = synth.attention_inputs(B, S, T, n_h, torch.bfloat16, seed=23, causal=False)
    out = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV))
    torch.cuda.synchronize()
    want = inp["v"][:, :1].expand(B, S, n_h, 128).contiguous()
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))


# --------------------------------------------------------------------------
# reconstruction with one head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,dtype", [(1, torch.bfloat16), (257, torch.bfloat16),
                                     (3, torch.float32)])
def test_kv_reconstruct_one_head(N, dtype):
    inp = synth.reconstruct_inputs(N, 1, dtype, seed=N + 5)
    K, V = mla.mla_kv_reconstruct(inp["c"].to(DEV), inp["k_rope"].to(DEV), inp["wkv_b"].to(DEV))
    Kr, Vr = oracle.kv_reconstruct(inp["c"], inp["k_rope"], inp["wkv_b"], 1)
    check(f64(K)[..., :128], Kr[..., :128], TOL[dtype], "k_nope")
    check(f64(V), Vr, TOL[dtype], "v")
    assert torch.equal(K.cpu()[..., 128:], inp["k_rope"][:, None, :])


# --------------------------------------------------------------------------
# empty batches: every entry point returns without touching its outputs
# --------------------------------------------------------------------------

def sentinel(shape, dtype=torch.bfloat16):
    return torch.full(shape, 7.0, dtype=dtype, device=DEV)


def test_empty_batches_are_noops():
    bf = torch.bfloat16
    w = torch.zeros((128 * 256, 512), dtype=bf, device=DEV)
    cache = torch.zeros((1, 4, 576), dtype=bf, device=DEV)
    q0 = torch.empty((0, 128, 128), dtype=bf, device=DEV)
    assert mla.mla_absorb_q(q0, w).shape == (0, 128, 512)
    assert mla.mla_out_up(torch.empty((0, 128, 512), dtype=bf, device=DEV), w).shape == (0, 128, 128)
    out = mla.mla_decode_step(q0, torch.empty((0, 128, 64), dtype=bf, device=DEV), w,
                              cache[..., :512], cache[..., 512:], T=4)
    assert out.shape == (0, 128, 128)
    multi = mla.mla_decode_latent_attn_multi(
        torch.empty((0, 2, 16, 512), dtype=bf, device=DEV),
        torch.empty((0, 2, 16, 64), dtype=bf, device=DEV), cache[..., :512], cache[..., 512:],
        causal=True)
    assert multi.shape == (0, 2, 16, 512)
    # attention with no queries: the output keeps its contents
    k = torch.zeros((1, 5, 2, 192), dtype=bf, device=DEV)
    v = torch.zeros((1, 5, 2, 128), dtype=bf, device=DEV)
    o = sentinel((1, 0, 2, 128))
    mla.mla_attention_naive(torch.empty((1, 0, 2, 192), dtype=bf, device=DEV), k, v, out=o)
    # append of no rows and reconstruction of no tokens leave the caches alone
    lat = sentinel((2, 4, 576))
    mla.mla_cache_append(torch.empty((0, 576), dtype=bf, device=DEV),
                         torch.ones(512, device=DEV), torch.zeros((4, 32, 2), device=DEV),
                         torch.empty(0, dtype=torch.int32, device=DEV), lat[..., :512],
                         lat[..., 512:])
    Kc, Vc = mla.mla_kv_reconstruct(torch.empty((0, 512), dtype=bf, device=DEV),
                                    torch.empty((0, 64), dtype=bf, device=DEV), w)
    torch.cuda.synchronize()
    assert Kc.shape == (0, 128, 192) and Vc.shape == (0, 128, 128)
    assert torch.all(lat == 7.0)
