"""GPU parity of the ordinary attention over reconstructed keys and values
(the naive path's second half: per-head scores over 192 features, per-token
index sets, causal mask, softmax, values) against the fp64 oracle.

Bar: max|err| <= 2e-2 * max|ref| (bf16) or 1e-5 * max|ref| (fp32) for the
outputs and the log-sum-exp. Cases span several 256-query blocks and 64-key
tiles with ragged tails, queries at the end of a longer key sequence, index
sets with hidden entries, and the full prefill size (S = T = 8192, 128 heads;
sampled queries).
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


def check(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite pattern differs"
    m = np.max(np.abs(ref[fin]))
    err = np.max(np.abs(got[fin] - ref[fin]))
    assert err <= tol * m, f"{what}: max|err| {err:.3e} > {tol} * {m:.3e}"
    assert np.array_equal(got[~fin], ref[~fin])


CASES = [
    # B, S, T, n_h, causal, topk, dtype
    (1, 300, 300, 2, True, None, torch.bfloat16),
    (2, 200, 333, 3, True, None, torch.bfloat16),
    (2, 100, 257, 2, False, None, torch.bfloat16),
    (1, 300, 300, 2, True, 64, torch.bfloat16),
    (2, 130, 190, 1, False, 50, torch.bfloat16),
    (1, 520, 520, 1, True, 3, torch.bfloat16),     # early sets partly hidden
    (1, 1, 1000, 4, True, None, torch.bfloat16),   # one query at the end
    (1, 40, 70, 2, True, None, torch.float32),
    (2, 33, 80, 2, True, 20, torch.float32),
]


@pytest.mark.parametrize("B,S,T,n_h,causal,topk,dtype", CASES)
def test_attention_naive(B, S, T, n_h, causal, topk, dtype):
    inp = synth.attention_inputs(B, S, T, n_h, dtype, seed=S * 7 + T, topk=topk, causal=causal)
    idx = inp.get("topk_idx")
    out, lse = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                       topk_idx=None if idx is None else idx.to(DEV),
                                       causal=causal, want_lse=True)
    ref, ref_lse = oracle.attention_naive(inp["q"], inp["k"], inp["v"], topk_idx=idx,
                                          causal=causal)
    check(out.cpu().double().numpy(), ref, TOL[dtype], "out")
    check(lse.cpu().double().numpy(), ref_lse, TOL[dtype], "lse")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_queries_whose_whole_set_is_hidden(dtype):
    # every set is the last key only: under the causal mask all queries but
    # the last see nothing (zero output, lse -inf); the last sees one key
    B, S, T, n_h = 1, 300, 300, 2
    inp = synth.attention_inputs(B, S, T, n_h, dtype, seed=5)
    idx = torch.full((B, S, 1), T - 1, dtype=torch.int32)
    out, lse = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                       topk_idx=idx.to(DEV), causal=True, want_lse=True)
    ref, ref_lse = oracle.attention_naive(inp["q"], inp["k"], inp["v"], topk_idx=idx,
                                          causal=True)
    check(out.cpu().double().numpy(), ref, TOL[dtype], "out")
    check(lse.cpu().double().numpy(), ref_lse, TOL[dtype], "lse")


def test_repeated_indices_count_once():
    B, S, T, n_h = 1, 64, 64, 2
    inp = synth.attention_inputs(B, S, T, n_h, seed=3, topk=8, causal=False)
    idx = inp["topk_idx"]
    dup = torch.cat([idx, idx[..., :3]], -1).contiguous()  # three repeats per set
    a = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                topk_idx=idx.to(DEV))
    b = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                topk_idx=dup.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a.cpu().view(torch.int16), b.cpu().view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_index_sets_with_repeats_and_out_of_range_entries(causal, dtype):
    # the mask is a scatter into a -inf row: repeats mark a position once and
    # entries outside [0, T) mark nothing; the oracle follows the same set
    # reading, independently of the GPU's bit mask
    B, S, T, n_h, K = 2, 130, 190, 2, 40
    inp = synth.attention_inputs(B, S, T, n_h, dtype, seed=11, topk=K - 12, causal=causal)
    g = np.random.default_rng(12)
    base = inp["topk_idx"].numpy()
    bad = np.array([-1, T, T + 64, -(2 ** 31), 2 ** 31 - 1], np.int64)
    idx = np.empty((B, S, K), np.int64)
    for b in range(B):
        for s in range(S):
            row = np.concatenate([base[b, s], base[b, s, :6], bad[g.integers(5, size=6)]])
            idx[b, s] = row[g.permutation(K)]
    idx = torch.from_numpy(idx.astype(np.int32))
    out, lse = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                       topk_idx=idx.to(DEV), causal=causal, want_lse=True)
    ref, ref_lse = oracle.attention_naive(inp["q"], inp["k"], inp["v"], topk_idx=idx,
                                          causal=causal)
    check(out.cpu().double().numpy(), ref, TOL[dtype], "out")
    check(lse.cpu().double().numpy(), ref_lse, TOL[dtype], "lse")


def test_prefill_full_size_sampled_queries():
    # S = T = 8192 tokens, 128 heads, causal: the launch the benchmark times;
    # eight queries (all heads) against the oracle over their visible keys
    B, S, T, n_h = 1, 8192, 8192, 128
    inp = synth.attention_inputs(B, S, T, n_h, seed=1007)
    out = mla.mla_attention_naive(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                  causal=True)
    got = out.cpu()
    for s in (0, 1, 255, 256, 4095, 5000, 8190, 8191):
        ref, _ = oracle.attention_naive(inp["q"][:, s:s + 1], inp["k"][:, :s + 1],
                                        inp["v"][:, :s + 1], causal=True)
        check(got[:, s:s + 1].double().numpy(), ref, TOL[torch.bfloat16], f"query {s}")
