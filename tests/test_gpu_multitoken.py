"""GPU parity of multi-token decode (S_q query tokens per sequence, optional
causal limit at the end of the cache, shared index set) and of the one-call
decode step, against the fp64 oracle.

Bar: max|err| <= 2e-2 * max|ref| for bf16, 1e-5 * max|ref| for fp32, for
out_lat / out and for the log-sum-exp. Cases cover full and partial 128-row
head groups, splits whose rows are all hidden from some tokens by the causal
limit, a query block that fills the whole cache (T == S_q), and the decode
workload's sizes (sampled sequences).
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


def f64(t):
    return t.detach().cpu().double().numpy()


def check(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    m = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    assert err <= tol * m, f"{what}: max|err| {err:.3e} > {tol} * {m:.3e}"


def multi_inputs(B, S_q, n_h, T, dtype, seed, topk=None):
    """Query rows [B, S_q, n_h, .] and a cache from the shared generators: the
    S_q tokens of sequence b are drawn as B*S_q single-token rows."""
    base = synth.decode_inputs(B * S_q, n_h, 1, dtype, seed=seed, stage_inputs=True)
    cache = synth.decode_inputs(B, 1, T, dtype, seed=seed + 1, topk=topk)
    out = {
        "q_lat": base["q_lat"].reshape(B, S_q, n_h, 512).contiguous(),
        "q_pe": base["q_pe"].reshape(B, S_q, n_h, 64).contiguous(),
        "q_nope": base["q_nope"].reshape(B, S_q, n_h, 128).contiguous(),
        "wkv_b": base["wkv_b"],
        "cache": cache["cache"],
    }
    if topk:
        out["topk_idx"] = cache["topk_idx"]
    return out


MULTI_CASES = [
    # B, S_q, n_h, T, dtype, causal, topk, num_splits
    (2, 2, 128, 700, torch.bfloat16, True, None, 0),     # two full head groups
    (3, 4, 16, 333, torch.bfloat16, True, None, 0),      # 64 rows: one partial group
    (2, 3, 16, 100, torch.bfloat16, False, None, 0),
    (2, 4, 16, 33, torch.bfloat16, True, None, 2),       # split 1 = row 32, hidden from 3 tokens
    (1, 5, 16, 5, torch.bfloat16, True, None, 0),        # T == S_q: token 0 sees one row
    (2, 2, 128, 1000, torch.bfloat16, False, 300, 0),    # shared index set
    (2, 3, 16, 65, torch.float32, True, None, 0),
    (2, 4, 16, 33, torch.float32, True, None, 2),
]


@pytest.mark.parametrize("B,S_q,n_h,T,dtype,causal,topk,splits", MULTI_CASES)
def test_multi_token_latent_attention(B, S_q, n_h, T, dtype, causal, topk, splits):
    inp = multi_inputs(B, S_q, n_h, T, dtype, seed=B * 1000 + S_q * 100 + T, topk=topk)
    cache = inp["cache"].to(DEV)
    idx = inp.get("topk_idx")
    out, lse = mla.mla_decode_latent_attn_multi(
        inp["q_lat"].to(DEV), inp["q_pe"].to(DEV), cache[..., :512], cache[..., 512:],
        topk_idx=None if idx is None else idx.to(DEV), causal=causal, num_splits=splits,
        want_lse=True)
    ref, ref_lse = oracle.latent_attention_multi(inp["q_lat"], inp["q_pe"],
                                                 inp["cache"][..., :512], inp["cache"][..., 512:],
                                                 topk_idx=idx, causal=causal)
    check(f64(out), ref, TOL[dtype], "out_lat")
    check(f64(lse), ref_lse, TOL[dtype], "lse")


def test_multi_token_with_one_token_matches_single_token_call():
    inp = multi_inputs(4, 1, 128, 300, torch.bfloat16, seed=7)
    cache = inp["cache"].to(DEV)
    a = mla.mla_decode_latent_attn_multi(inp["q_lat"].to(DEV), inp["q_pe"].to(DEV),
                                         cache[..., :512], cache[..., 512:])
    b = mla.mla_decode_latent_attn(inp["q_lat"][:, 0].contiguous().to(DEV),
                                   inp["q_pe"][:, 0].contiguous().to(DEV), cache[..., :512],
                                   cache[..., 512:])
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0].cpu().view(torch.int16), b.cpu().view(torch.int16))


def oracle_step(inp, causal, idx=None, sel=None):
    """absorb -> multi-token latent attention -> W^UV, all in double."""
    qn, qp, cache = inp["q_nope"], inp["q_pe"], inp["cache"]
    if sel is not None:
        qn, qp, cache = qn[sel], qp[sel], cache[sel]
        idx = None if idx is None else idx[sel]
    B, S_q, n_h, _ = qn.shape
    w = inp["wkv_b"]
    q_lat = oracle.absorb_q(qn.reshape(B * S_q, n_h, 128), w).reshape(B, S_q, n_h, 512)
    o, lse = oracle.latent_attention_multi(q_lat, qp, cache[..., :512], cache[..., 512:],
                                           topk_idx=idx, causal=causal)
    out = oracle.out_up(o.reshape(B * S_q, n_h, 512), w).reshape(B, S_q, n_h, 128)
    return out, lse


@pytest.mark.parametrize("B,S_q,n_h,T,dtype,causal,topk", [
    (2, 2, 128, 517, torch.bfloat16, True, None),
    (3, 1, 128, 300, torch.bfloat16, False, 100),
    (2, 4, 16, 90, torch.bfloat16, True, None),
    (2, 2, 16, 70, torch.float32, True, None),
])
def test_decode_step_one_call(B, S_q, n_h, T, dtype, causal, topk):
    inp = multi_inputs(B, S_q, n_h, T, dtype, seed=31 + T, topk=topk)
    cache = inp["cache"].to(DEV)
    idx = inp.get("topk_idx")
    out, lse = mla.mla_decode_step(inp["q_nope"].to(DEV), inp["q_pe"].to(DEV),
                                   inp["wkv_b"].to(DEV), cache[..., :512], cache[..., 512:],
                                   topk_idx=None if idx is None else idx.to(DEV), causal=causal,
                                   want_lse=True)
    ref, ref_lse = oracle_step(inp, causal, idx)
    check(f64(out), ref, TOL[dtype], "out")
    check(f64(lse), ref_lse, TOL[dtype], "lse")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_decode_step_single_token_equals_the_three_calls(cfg):
    # the benchmark's one-call step (packed queries, split merge fused into
    # W^UV) against the separate calls the parity tests check against the
    # oracle, at the full workload sizes: the same bits
    print(f"step vs three calls: config {cfg}", flush=True)
    inp = synth.config_inputs(cfg)
    d = {k: v.to(DEV) for k, v in inp.items()}
    if cfg == 4:
        d["wkv_b"] = mla.mla_dequant_fp8_block(d["wkv_b_fp8"], d["wkv_b_scale"])
    idx = d.get("topk_idx")
    cache = d["cache"]
    one = mla.mla_decode_step(d["q_nope"], d["q_pe"], d["wkv_b"], cache[..., :512],
                              cache[..., 512:], topk_idx=idx)
    q_lat = mla.mla_absorb_q(d["q_nope"], d["wkv_b"])
    o_lat = mla.mla_decode_latent_attn(q_lat, d["q_pe"], cache[..., :512], cache[..., 512:],
                                       topk_idx=idx)
    three = mla.mla_out_up(o_lat, d["wkv_b"])
    torch.cuda.synchronize()
    assert torch.equal(one.cpu().view(torch.int16), three.cpu().view(torch.int16))


def test_decode_step_causal_pair_at_decode_workload_size_sampled():
    # B=32 sequences of T=4096 cached positions, n_h=128, two query tokens
    # per sequence (the second one sees one more position); three sequences
    # are checked against the oracle
    B, S_q, n_h, T = 32, 2, 128, 4096
    inp = multi_inputs(B, S_q, n_h, T, torch.bfloat16, seed=1002)
    cache = inp["cache"].to(DEV)
    out = mla.mla_decode_step(inp["q_nope"].to(DEV), inp["q_pe"].to(DEV), inp["wkv_b"].to(DEV),
                              cache[..., :512], cache[..., 512:], causal=True)
    sel = [0, 17, 31]
    ref, _ = oracle_step(inp, True, sel=sel)
    check(f64(out.cpu()[sel]), ref, TOL[torch.bfloat16], "out")


@pytest.mark.parametrize("B,S_q,n_h,T", [(33, 1, 128, 700), (3, 2, 16, 900), (5, 1, 20, 2000),
                                         (17, 1, 96, 300)])
def test_decode_step_fused_merge_matches_the_separate_kernels(B, S_q, n_h, T):
    # with several splits the one-call step merges them inside W^UV; the
    # result must have exactly the bits of attention (with its merge) + W^UV
    inp = multi_inputs(B, S_q, n_h, T, torch.bfloat16, seed=B * 7 + n_h + T)
    assert mla.mla_decode_num_splits(B, S_q * n_h, T) > 1
    d = {k: v.to(DEV) for k, v in inp.items()}
    cache = d["cache"]
    one, lse1 = mla.mla_decode_step(d["q_nope"], d["q_pe"], d["wkv_b"], cache[..., :512],
                                    cache[..., 512:], causal=S_q > 1, want_lse=True)
    BS = B * S_q
    q_lat = mla.mla_absorb_q(d["q_nope"].reshape(BS, n_h, 128), d["wkv_b"])
    o_lat, lse3 = mla.mla_decode_latent_attn_multi(q_lat.reshape(B, S_q, n_h, 512), d["q_pe"],
                                                   cache[..., :512], cache[..., 512:],
                                                   causal=S_q > 1, want_lse=True)
    three = mla.mla_out_up(o_lat.reshape(BS, n_h, 512), d["wkv_b"]).reshape(B, S_q, n_h, 128)
    torch.cuda.synchronize()
    assert torch.equal(one.cpu().view(torch.int16), three.cpu().view(torch.int16))
    assert torch.equal(lse1.cpu(), lse3.cpu())


@pytest.mark.parametrize("B,n_h,T,splits", [
    (2, 128, 8000, 0),    # automatic plan: 125 splits of 2 tiles, 2 rows per tile (parts on two waves)
    (4, 64, 3000, 47),    # 47 splits, 4 rows: parts on two waves
    (5, 32, 4000, 52),    # 42 splits of 3 tiles, 5 rows: both parts in one wave
    (20, 16, 2500, 41),   # 40 splits; tile 0: two rows per wave, both parts in one wave;
                          # tile 1: 4 rows, parts on two waves
    (3, 128, 1050, 33),   # 33 splits of one tile: just past the two-part bound
    (2, 256, 4096, 0),    # 64 splits, 256 (head, tile) workgroups: the one-part-per-quarter
                          # W^UV layout with the parts on two waves
])
def test_merge_of_many_splits_fused_and_separate(B, n_h, T, splits):
    # rows of more than 32 splits are merged in two parts, by two waves or by
    # one; the fused merge + W^UV and the stand-alone merge must give the same
    # bits, and both must match the oracle
    print(f"many-split merge: B={B} n_h={n_h} T={T} splits={splits}", flush=True)
    inp = multi_inputs(B, 1, n_h, T, torch.bfloat16, seed=B * 11 + n_h + T)
    d = {k: v.to(DEV) for k, v in inp.items()}
    cache = d["cache"]
    ntiles = -(-T // 32)
    req = splits or mla.mla_decode_num_splits(B, n_h, T)
    S = -(-ntiles // -(-ntiles // req))  # no empty split: whole tiles per split
    assert S > 32
    one, lse1 = mla.mla_decode_step(d["q_nope"], d["q_pe"], d["wkv_b"], cache[..., :512],
                                    cache[..., 512:], num_splits=splits, want_lse=True)
    q_lat = mla.mla_absorb_q(d["q_nope"].reshape(B, n_h, 128), d["wkv_b"])
    o_lat, lse3 = mla.mla_decode_latent_attn_multi(q_lat.reshape(B, 1, n_h, 512), d["q_pe"],
                                                   cache[..., :512], cache[..., 512:],
                                                   num_splits=splits, want_lse=True)
    three = mla.mla_out_up(o_lat.reshape(B, n_h, 512), d["wkv_b"]).reshape(B, 1, n_h, 128)
    torch.cuda.synchronize()
    assert torch.equal(one.cpu().view(torch.int16), three.cpu().view(torch.int16))
    assert torch.equal(lse1.cpu(), lse3.cpu())
    ref, ref_lse = oracle_step(inp, False, None)
    check(f64(one), ref, TOL[torch.bfloat16], "out")
    check(f64(lse1), ref_lse, TOL[torch.bfloat16], "lse")


def unpack_queries(packed, B, S_q, n_h):
    """Row layout [B, S_q, n_h, 512] of packed queries, by the slot formula
    the header states (plain numpy indexing)."""
    R = S_q * n_h
    G = R // 128
    p = packed.reshape(B, G, 4, 32, 2, 32, 8)  # b, group, quarter, k-step, half, row%32, 8 features
    rows = p.transpose(0, 1, 2, 5, 3, 4, 6).reshape(B, R, 512)
    return rows.reshape(B, S_q, n_h, 512)


@pytest.mark.parametrize("B,S_q,n_h", [(3, 1, 128), (2, 2, 64), (33, 1, 256)])
def test_packed_queries_layout_and_attention(B, S_q, n_h):
    T = 300
    inp = multi_inputs(B, S_q, n_h, T, torch.bfloat16, seed=B + S_q + n_h)
    d = {k: v.to(DEV) for k, v in inp.items()}
    cache = d["cache"]
    rows = mla.mla_absorb_q(d["q_nope"].reshape(B * S_q, n_h, 128), d["wkv_b"])
    packed = mla.mla_absorb_q_packed(d["q_nope"], d["wkv_b"])
    torch.cuda.synchronize()
    un = unpack_queries(packed.cpu().view(torch.int16).numpy(), B, S_q, n_h)
    assert np.array_equal(un, rows.cpu().view(torch.int16).numpy().reshape(B, S_q, n_h, 512))
    causal = S_q > 1
    a, la = mla.mla_decode_latent_attn_packed(packed, d["q_pe"], cache[..., :512],
                                              cache[..., 512:], causal=causal, want_lse=True)
    b, lb = mla.mla_decode_latent_attn_multi(rows.reshape(B, S_q, n_h, 512), d["q_pe"],
                                             cache[..., :512], cache[..., 512:], causal=causal,
                                             want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu().view(torch.int16), b.cpu().view(torch.int16))
    assert torch.equal(la.cpu(), lb.cpu())
