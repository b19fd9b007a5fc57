"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a hand-computed example, a closed form,
an identity the pages state, or an independent library routine (torch's
e4m3fn decode, float32 multiply and bfloat16 cast; torch's scaled dot-product
attention in double). A plausible slip anywhere in the oracle -- a dropped
rotary term, a swapped W^UK/W^UV half, a transposed weight, a wrong head
offset, a missing scale, a mask applied per head -- fails at least one of
them. No GPU is used.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def tiny_problem(seed, B, n_h, T, d_c=16, d_r=4, d_n=8, d_v=6, T_alloc=None):
    g = rng(seed)
    Ta = T_alloc or T
    return dict(
        q_nope=g.standard_normal((B, n_h, d_n)),
        q_pe=g.standard_normal((B, n_h, d_r)),
        latent=g.standard_normal((B, Ta, d_c)),
        rope=g.standard_normal((B, Ta, d_r)),
        w=g.standard_normal((n_h * (d_n + d_v), d_c)) / math.sqrt(d_c),
        d_n=d_n, d_v=d_v,
    )


def run_both(p, T=None, topk_idx=None, scale=0.3, **kw):
    common = dict(T=T, topk_idx=topk_idx, scale=scale, d_n=p["d_n"], d_v=p["d_v"])
    a = oracle.decode_absorbed(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                               **common, **kw)
    n = oracle.decode_naive(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"], **common)
    return a, n


def rel_err(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


# --------------------------------------------------------------------------
# hand-computed example (tests/golden/tiny_hand_example.json)
# --------------------------------------------------------------------------

def _hand():
    with open(os.path.join(GOLD, "tiny_hand_example.json")) as f:
        g = json.load(f)
    i = g["inputs"]
    p = dict(
        q_nope=np.array([[i["q_nope"]]]),
        q_pe=np.array([[[math.log(3.0)]]]),
        latent=np.array([i["latent"]]),
        rope=np.array([i["rope"]]),
        w=np.array(i["wkv_b"]),
        d_n=1, d_v=1,
    )
    return g, p


def test_hand_example_absorbed_and_naive():
    g, p = _hand()
    e = g["expected"]
    a, n = run_both(p, scale=g["inputs"]["scale"], want_olat=True, want_lse=True,
                    want_probs=True)
    assert np.allclose(oracle.absorb_q(p["q_nope"], p["w"], d_n=1, d_v=1)[0, 0], e["q_lat"],
                       rtol=0, atol=1e-15)
    assert np.allclose(a["probs"][0, 0], e["probs"], rtol=0, atol=1e-15)
    assert np.allclose(a["o_lat"][0, 0], e["o_lat"], rtol=0, atol=1e-15)
    assert abs(a["out"][0, 0, 0] - e["out"]) < 1e-14
    assert abs(n["out"][0, 0, 0] - e["out"]) < 1e-14
    assert abs(a["lse"][0, 0] - (2.0 + math.log(4.0))) < 1e-14


def test_hand_example_masked():
    g, p = _hand()
    e = g["expected"]
    idx = np.array([e["masked_idx"]], np.int32)
    a, n = run_both(p, topk_idx=idx, scale=1.0, want_olat=True, want_lse=True,
                    want_probs=True)
    assert np.array_equal(a["probs"][0, 0], e["masked_probs"])
    assert np.allclose(a["o_lat"][0, 0], e["masked_o_lat"], rtol=0, atol=1e-15)
    assert a["out"][0, 0, 0] == e["masked_out"] and n["out"][0, 0, 0] == e["masked_out"]
    assert abs(a["lse"][0, 0] - (2.0 + math.log(3.0))) < 1e-14


# --------------------------------------------------------------------------
# the absorbed path equals the naive path ("KV Reconstruction", How it works)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,n_h,T", [(1, 1, 1), (2, 2, 5), (3, 16, 37), (1, 2, 300)])
def test_absorbed_equals_naive_small_dims(B, n_h, T):
    p = tiny_problem(10 + B * 100 + n_h * 10 + T, B, n_h, T)
    a, n = run_both(p)
    assert rel_err(a["out"], n["out"]) < 1e-12


def test_absorbed_equals_naive_model_dims_with_mask_and_strides():
    # real dims (512/64/128), cache allocated longer than T, top-k mask
    p = tiny_problem(7, 2, 3, 40, d_c=512, d_r=64, d_n=128, d_v=128, T_alloc=48)
    g = rng(8)
    idx = np.stack([g.choice(40, 11, replace=False) for _ in range(2)]).astype(np.int32)
    a, n = run_both(p, T=40, topk_idx=idx, scale=192 ** -0.5)
    assert rel_err(a["out"], n["out"]) < 1e-12


def test_naive_and_absorbed_differ_if_wuk_wuv_swapped():
    # "Watch-outs": the two halves of wkv_b are not interchangeable
    p = tiny_problem(11, 1, 2, 9, d_n=6, d_v=6)
    a, _ = run_both(p)
    w = p["w"].reshape(2, 12, -1)
    p2 = dict(p, w=np.concatenate([w[:, 6:], w[:, :6]], axis=1).reshape(24, -1))
    b, _ = run_both(p2)
    assert rel_err(a["out"], b["out"]) > 1e-3


# --------------------------------------------------------------------------
# naive path against torch's scaled dot-product attention (double, CPU)
# --------------------------------------------------------------------------

def _dirty_sets(g, rows, T, K, n_bad=4, n_rep=3):
    """Index rows of K entries: distinct in-range positions, then repeats of
    some of them and entries outside [0, T) (padding -1, T, beyond), in a
    shuffled order."""
    out = np.empty((rows, K), np.int32)
    for r in range(rows):
        good = g.choice(T, K - n_bad - n_rep, replace=False)
        bad = np.array([-1, T, T + 7, -(2 ** 31)], np.int64)[:n_bad]
        row = np.concatenate([good, good[:n_rep], bad]).astype(np.int32)
        out[r] = row[g.permutation(K)]
    return out


def _set_mask(idx, T):
    """Boolean [rows, T] mask of the in-range entries of each index row."""
    flat = idx.reshape(-1, idx.shape[-1])
    m = np.zeros((flat.shape[0], T), bool)
    for r, row in enumerate(flat):
        m[r, row[(row >= 0) & (row < T)]] = True
    return m.reshape(idx.shape[:-1] + (T,))


@pytest.mark.parametrize("masked", [False, True, "dirty"])
def test_naive_matches_torch_sdpa(masked):
    B, n_h, T = 2, 4, 50
    p = tiny_problem(21, B, n_h, T, d_c=512, d_r=64, d_n=128, d_v=128)
    scale = 192 ** -0.5
    idx = None
    allowed = np.ones((B, T), bool)
    if masked == "dirty":
        # repeats and out-of-range entries: the scatter marks a set
        idx = _dirty_sets(rng(23), B, T, 24)
        allowed = _set_mask(idx, T)
    elif masked:
        g = rng(22)
        idx = np.stack([g.choice(T, 17, replace=False) for _ in range(B)]).astype(np.int32)
        allowed[:] = False
        for b in range(B):
            allowed[b, idx[b]] = True
    n = oracle.decode_naive(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                            topk_idx=idx, scale=scale)["out"]
    for b in range(B):
        K, V = oracle.kv_reconstruct(p["latent"][b], p["rope"][b], p["w"], n_h)
        q = torch.from_numpy(np.concatenate([p["q_nope"][b], p["q_pe"][b]], -1))[:, None, :]
        k = torch.from_numpy(K).permute(1, 0, 2).contiguous()
        v = torch.from_numpy(V).permute(1, 0, 2).contiguous()
        m = torch.from_numpy(allowed[b])[None, None, :].expand(n_h, 1, T)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                               scale=scale)
        assert rel_err(n[b], ref[:, 0, :].numpy()) < 1e-12


# --------------------------------------------------------------------------
# reconstruction with structured weights (closed form)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d_c,d_r,d_n,d_v,n_h", [(16, 4, 5, 6, 3), (512, 64, 128, 128, 2)])
def test_reconstruct_structured_weights(d_c, d_r, d_n, d_v, n_h):
    # W^UK of head h picks latent feature e scaled by (h+1); W^UV of head h
    # picks feature (e + 3 + h) mod d_c scaled by -(h+2). Any transposition,
    # swapped half or head offset changes the result.
    N = 7
    g = rng(31)
    c = g.standard_normal((N, d_c))
    kr = g.standard_normal((N, d_r))
    w = np.zeros((n_h * (d_n + d_v), d_c))
    for h in range(n_h):
        for e in range(d_n):
            w[h * (d_n + d_v) + e, e % d_c] = h + 1
        for e in range(d_v):
            w[h * (d_n + d_v) + d_n + e, (e + 3 + h) % d_c] = -(h + 2)
    K, V = oracle.kv_reconstruct(c, kr, w, n_h, d_n=d_n, d_v=d_v)
    for h in range(n_h):
        for e in range(d_n):
            assert np.array_equal(K[:, h, e], (h + 1) * c[:, e % d_c])
        for e in range(d_v):
            assert np.array_equal(V[:, h, e], -(h + 2) * c[:, (e + 3 + h) % d_c])
        assert np.array_equal(K[:, h, d_n:], kr)  # rotary part is an exact copy


def test_reconstruct_copies_bf16_rope_bits_exactly():
    g = rng(33)
    c = torch.from_numpy(g.standard_normal((5, 16)).astype(np.float32)).bfloat16()
    kr = torch.from_numpy(g.standard_normal((5, 4)).astype(np.float32)).bfloat16()
    w = torch.from_numpy(g.standard_normal((2 * 12, 16)).astype(np.float32)).bfloat16()
    K, _ = oracle.kv_reconstruct(c, kr, w, 2, d_n=6, d_v=6)
    for h in range(2):
        assert np.array_equal(K[:, h, 6:], kr.double().numpy())


# --------------------------------------------------------------------------
# closed forms of the absorbed decode
# --------------------------------------------------------------------------

def _w_uv(w, n_h, d_n, d_v):
    return w.reshape(n_h, d_n + d_v, -1)[:, d_n:, :]  # [n_h, d_v, d_c]


def test_single_position_returns_w_uv_times_latent():
    p = tiny_problem(41, 2, 3, 1)
    a, _ = run_both(p, want_lse=True)
    wuv = _w_uv(p["w"], 3, p["d_n"], p["d_v"])
    for b in range(2):
        exp = wuv @ p["latent"][b, 0]  # [n_h, d_v]
        assert rel_err(a["out"][b], exp) < 1e-13
    # lse of one position is its score
    # lse of one position is its score; q_lat taken from the naive form
    # (q_nope . W^UK c) so the check does not reuse the oracle's absorb
    w = p["w"].reshape(3, p["d_n"] + p["d_v"], -1)
    for b in range(2):
        for h in range(3):
            k_c = w[h, :p["d_n"]] @ p["latent"][b, 0]
            zz = 0.3 * (p["q_nope"][b, h] @ k_c + p["q_pe"][b, h] @ p["rope"][b, 0])
            assert abs(a["lse"][b, h] - zz) < 1e-12


def test_zero_query_gives_uniform_weights():
    p = tiny_problem(42, 2, 2, 23)
    p["q_nope"][:] = 0
    p["q_pe"][:] = 0
    a, _ = run_both(p, want_lse=True, want_probs=True)
    assert np.allclose(a["probs"], 1.0 / 23, rtol=1e-14, atol=0)
    assert np.allclose(a["lse"], math.log(23), rtol=1e-14, atol=0)
    wuv = _w_uv(p["w"], 2, p["d_n"], p["d_v"])
    for b in range(2):
        assert rel_err(a["out"][b], wuv @ p["latent"][b].mean(0)) < 1e-13


def test_one_index_selects_that_row():
    p = tiny_problem(43, 3, 2, 19)
    idx = np.array([[4], [0], [18]], np.int32)
    a, _ = run_both(p, topk_idx=idx, want_probs=True)
    wuv = _w_uv(p["w"], 2, p["d_n"], p["d_v"])
    for b in range(3):
        assert rel_err(a["out"][b], wuv @ p["latent"][b, idx[b, 0]]) < 1e-13
        assert np.all(a["probs"][b, :, idx[b, 0]] == 1.0)


def test_constant_rope_key_makes_q_pe_irrelevant():
    p = tiny_problem(44, 2, 3, 31)
    p["rope"][:] = p["rope"][:, :1, :]  # same rotary key at every position
    a1, _ = run_both(p)
    p2 = dict(p, q_pe=rng(45).standard_normal(p["q_pe"].shape) * 10)
    a2, _ = run_both(p2)
    assert rel_err(a1["out"], a2["out"]) < 1e-12


def test_rope_scores_enter_with_the_scale():
    # Same content score everywhere (latent rows equal); only the rotary
    # score differs, so p_t must be softmax(scale * q_pe . k^R_t).
    p = tiny_problem(46, 1, 2, 6)
    p["latent"][:] = p["latent"][:, :1, :]
    a, _ = run_both(p, scale=0.7, want_probs=True)
    for h in range(2):
        z = 0.7 * (p["rope"][0] @ p["q_pe"][0, h])
        e = np.exp(z - z.max())
        assert np.allclose(a["probs"][0, h], e / e.sum(), rtol=1e-13, atol=0)


def test_mask_is_shared_by_all_heads_and_probs_sum_to_one():
    p = tiny_problem(47, 2, 5, 40)
    g = rng(48)
    idx = np.stack([g.choice(40, 9, replace=False) for _ in range(2)]).astype(np.int32)
    a, _ = run_both(p, topk_idx=idx, want_probs=True)
    pr = a["probs"]
    assert np.allclose(pr.sum(-1), 1.0, rtol=1e-14, atol=0)
    for b in range(2):
        outside = np.setdiff1d(np.arange(40), idx[b])
        assert np.all(pr[b][:, outside] == 0.0)  # exactly zero for every head
        assert np.all(pr[b][:, idx[b]] > 0.0)


def test_masked_rows_are_never_read():
    p = tiny_problem(49, 1, 2, 12)
    idx = np.array([[1, 5, 7]], np.int32)
    a, n = run_both(p, topk_idx=idx)
    poisoned = dict(p, latent=p["latent"].copy(), rope=p["rope"].copy())
    for t in set(range(12)) - {1, 5, 7}:
        poisoned["latent"][0, t] = np.nan
        poisoned["rope"][0, t] = 1e300
    a2, n2 = run_both(poisoned, topk_idx=idx)
    assert np.array_equal(a["out"], a2["out"]) and np.array_equal(n["out"], n2["out"])


def test_permutation_invariance():
    p = tiny_problem(50, 2, 3, 29)
    g = rng(51)
    idx = np.stack([g.choice(29, 10, replace=False) for _ in range(2)]).astype(np.int32)
    a, _ = run_both(p, topk_idx=idx)
    perm = g.permutation(29)
    inv = np.argsort(perm)
    p2 = dict(p, latent=p["latent"][:, perm], rope=p["rope"][:, perm])
    a2, _ = run_both(p2, topk_idx=inv[idx].astype(np.int32))
    assert rel_err(a2["out"], a["out"]) < 1e-13
    # index order is irrelevant
    a3, _ = run_both(p, topk_idx=idx[:, ::-1].copy())
    assert rel_err(a3["out"], a["out"]) < 1e-13


def test_index_sets_are_sets():
    # the mask is a scatter into a -inf row: repeats mark a position once,
    # entries outside [0, T) mark nothing
    p = tiny_problem(52, 2, 3, 8)
    a, n = run_both(p, topk_idx=np.array([[1, 5, 1, -1], [8, 0, 0, 3]], np.int32))
    c, _ = run_both(p, topk_idx=np.array([[1, 5], [0, 3]], np.int32))
    assert rel_err(a["out"], c["out"]) < 1e-14 and rel_err(n["out"], c["out"]) < 1e-14
    # a set that marks no position: the empty sum (zero output, lse -inf)
    e = oracle.decode_absorbed(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                               topk_idx=np.array([[-1, 8], [1, 1]], np.int32), scale=0.3,
                               d_n=p["d_n"], d_v=p["d_v"], want_lse=True, want_probs=True)
    assert np.all(e["out"][0] == 0.0) and np.all(np.isneginf(e["lse"][0]))
    assert np.all(e["probs"][0] == 0.0)
    np.testing.assert_allclose(e["probs"][1, :, 1], 1.0, rtol=1e-15)
    nn = oracle.decode_naive(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                             topk_idx=np.array([[-1, 8], [1, 1]], np.int32), scale=0.3,
                             d_n=p["d_n"], d_v=p["d_v"])
    assert np.all(nn["out"][0] == 0.0)
    assert rel_err(nn["out"][1], e["out"][1]) < 1e-13


def test_stage_functions_compose_to_the_whole_path():
    p = tiny_problem(53, 2, 3, 17, d_c=512, d_r=64, d_n=128, d_v=128)
    a = oracle.decode_absorbed(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                               scale=0.2, want_olat=True, want_lse=True)
    ql = oracle.absorb_q(p["q_nope"], p["w"])
    o, lse, _ = oracle.latent_attention(ql, p["q_pe"], p["latent"], p["rope"], scale=0.2,
                                        want_lse=True)
    out = oracle.out_up(o, p["w"])
    assert np.array_equal(o, a["o_lat"]) and np.array_equal(lse, a["lse"])
    assert np.array_equal(out, a["out"])


# --------------------------------------------------------------------------
# FP8 (OCP E4M3) decode and block dequantisation
# --------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = oracle.e4m3_to_f64(c)
        if (c & 0x7F) == 0x7F:
            assert math.isnan(v) and math.isnan(ref[c])
        else:
            assert v == ref[c], (c, v, ref[c])


def test_e4m3_definition_values():
    # OCP 8-bit FP spec, E4M3: bias 7, max normal 448, min subnormal 2^-9
    assert oracle.e4m3_to_f64(0x7E) == 448.0 and oracle.e4m3_to_f64(0xFE) == -448.0
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_f64(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x38) == 1.0 and oracle.e4m3_to_f64(0xB8) == -1.0
    assert oracle.e4m3_to_f64(0x3C) == 1.5
    assert oracle.e4m3_to_f64(0x00) == 0.0 and math.copysign(1, oracle.e4m3_to_f64(0x80)) < 0


def test_bf16_rounding_matches_torch_on_float32_values():
    g = rng(61)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32),
                        (g.standard_normal(2000) * 1e-38).astype(np.float32),
                        (g.standard_normal(2000) * 1e37).astype(np.float32)])
    ref = torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_ties_and_single_rounding():
    one = 0x3F80
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == one            # tie -> even (down)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == one + 2    # tie -> even (up)
    # just above the tie: a double rounds up in one step (float32 first would
    # drop the 2^-40 and then tie down to 1.0)
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == one + 1
    assert oracle.f64_to_bf16(3.4e38) == 0x7F80                  # overflow -> inf
    assert oracle.f64_to_bf16(-0.0) == 0x8000


@pytest.mark.parametrize("rows,cols", [(300, 272), (128, 128), (1, 16)])
def test_dequant_matches_torch_fp32_multiply_then_bf16(rows, cols):
    from head_latent_attention_mla_amd import synth
    codes = synth.fp8_codes(rows, cols, seed=rows + cols)
    g = rng(62)
    scales = (g.uniform(0.5, 2.0, ((rows + 127) // 128, (cols + 127) // 128)) * 2.0 ** -4
              ).astype(np.float32)
    got = oracle.dequant_fp8_block(codes.numpy(), scales)
    full = np.repeat(np.repeat(scales, 128, 0), 128, 1)[:rows, :cols]
    ref = (codes.view(torch.float8_e4m3fn).float() * torch.from_numpy(full)).bfloat16()
    assert np.array_equal(got, ref.view(torch.int16).numpy().view(np.uint16))


def test_dequant_uses_block_of_row_and_column():
    # distinct power-of-two scales per block: every element must carry its own
    codes = np.full((256, 384), 0x38, np.uint8)  # 1.0
    scales = np.array([[1, 2, 4], [8, 16, 32]], np.float32)
    got = oracle.bf16_bits_to_f64(oracle.dequant_fp8_block(codes, scales))
    for i in range(2):
        for j in range(3):
            assert np.all(got[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] == scales[i, j])


# --------------------------------------------------------------------------
# sizes and counts the pages print (tests/golden/page_counts.json)
# --------------------------------------------------------------------------

def test_page_counts():
    from head_latent_attention_mla_amd import synth
    with open(os.path.join(GOLD, "page_counts.json")) as f:
        g = json.load(f)
    n_h = 128
    w = synth.reconstruct_inputs(1, n_h)["wkv_b"]
    assert list(w.shape) == g["wkv_b_shape"]["value"]
    w_uv = w.view(n_h, 256, 512)[:, 128:, :]
    assert w_uv.numel() == g["w_uv_params_per_instance"]["value"]
    assert w_uv.numel() * 58 == g["w_uv_params_58_blocks"]["value"]
    assert [n_h * 128, 512] == g["up_projection_shape"]["value"]
    d = g["dims"]
    assert (d["d_c"], d["d_R"], d["d_h"]) == (synth.D_C, synth.D_R, synth.D_N)
    assert d["qk_head_dim"] == synth.D_N + synth.D_R and synth.SCALE == d["qk_head_dim"] ** -0.5
    # cache size B*N*(d_c+d_R)*s of a generated cache
    inp = synth.decode_inputs(2, 2, 33)
    cache = inp["cache"]
    assert cache.numel() * cache.element_size() == 2 * 33 * (512 + 64) * 2
    # the B=32, T=4096 decode workload: 32 x 4096 x 576 x 2 bytes
    assert 32 * 4096 * (512 + 64) * 2 == 150_994_944


# --------------------------------------------------------------------------
# attention scale ("Key–value latent", mla-init excerpt): closed forms
# --------------------------------------------------------------------------

def test_softmax_scale_closed_forms():
    def near(a, b):  # the oracle takes 1/sqrt, Python's ** takes pow: within 2 ulp
        return abs(a - b) <= 4.5e-16 * abs(b)
    base = 192 ** -0.5
    # no context extension: qk_head_dim^-1/2 with the 128 + 64 features
    assert near(oracle.softmax_scale(192), base)
    assert near(oracle.softmax_scale(192, max_seq_len=4096, original_seq_len=4096,
                                     mscale=1.0, rope_factor=40.0), base)
    # extension: factor (0.1 * m * ln(rope_factor) + 1)^2; ln(e^10) = 10 gives 2^2
    assert near(oracle.softmax_scale(192, 163840, 4096, mscale=1.0, rope_factor=math.exp(10.0)),
                4.0 * base)
    # m = 0 switches the factor off; m = 0.5, ln = 10 gives 1.5^2
    assert near(oracle.softmax_scale(192, 163840, 4096, 0.0, 40.0), base)
    assert near(oracle.softmax_scale(192, 163840, 4096, 0.5, math.exp(10.0)), 2.25 * base)
    assert math.isnan(oracle.softmax_scale(0))
    assert math.isnan(oracle.softmax_scale(192, 2, 1, 1.0, 0.0))


# --------------------------------------------------------------------------
# cache append: RMSNorm of the latent and rotation of the rotary key
# ("Key–value down-projection" and "Key–value latent RMSNorm" sections)
# --------------------------------------------------------------------------

def _angles_table(theta):
    th = np.asarray(theta, np.float64)
    return np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)


def test_rmsnorm_constant_row_closed_form():
    # x = c * ones: mean of squares is c^2, so y = gamma * c / sqrt(c^2 + eps)
    d_c, d_r = 512, 64
    for c, eps in ((0.75, 1e-6), (-3.0, 0.0), (1e-3, 1e-6), (2.0, 0.5)):
        x = np.full((1, d_c), c, np.float32)
        g = np.linspace(-2, 2, d_c).astype(np.float32)
        lat, _ = oracle.cache_append(x, np.zeros((1, d_r), np.float32), g,
                                     _angles_table(np.zeros((1, 32))), [0], eps=eps)
        want = g.astype(np.float64) * (np.float64(np.float32(c)) /
                                       math.sqrt(np.float64(np.float32(c)) ** 2 + eps))
        np.testing.assert_allclose(lat[0], want, rtol=1e-14, atol=0)


def test_rmsnorm_unit_rms_scale_invariance_and_zero_row():
    g = rng(41)
    x = g.standard_normal((4, 512)).astype(np.float32)
    x[1] *= 1024.0  # scaling by a power of two is exact in float32
    ones = np.ones(512, np.float32)
    z = np.zeros((4, 64), np.float32)
    tab = _angles_table(np.zeros((1, 32)))
    lat, _ = oracle.cache_append(x, z, ones, tab, [0] * 4, eps=0.0)
    np.testing.assert_allclose(np.sqrt((lat ** 2).mean(1)), 1.0, rtol=1e-14)
    lat1, _ = oracle.cache_append(x[1:2] / 1024.0, z[:1], ones, tab, [0], eps=0.0)
    np.testing.assert_allclose(lat[1], lat1[0], rtol=1e-14)
    # the mean runs over all 512 features, not a sum and not 511 of them:
    # a single nonzero feature v gives sqrt(512) * sign(v)
    e = np.zeros((1, 512), np.float32)
    e[0, 77] = -5.0
    le, _ = oracle.cache_append(e, z[:1], ones, tab, [0], eps=0.0)
    assert le[0, 77] == pytest.approx(-math.sqrt(512), rel=1e-15)
    assert np.count_nonzero(le[0]) == 1
    # eps keeps an all-zero row finite
    l0, _ = oracle.cache_append(np.zeros((1, 512), np.float32), z[:1], ones, tab, [0])
    assert np.all(l0 == 0.0)


def test_rotation_pairing_quarter_turns_and_identity():
    d_r = 64
    tab = _angles_table(np.array([np.zeros(32), np.full(32, math.pi / 2),
                                  np.full(32, math.pi)]))
    # quarter-turn entries of the table, as float32, are not exactly (0, 1);
    # the pins below use the table's own values
    c1, s1 = np.float64(tab[1, 0, 0]), np.float64(tab[1, 0, 1])
    ones = np.ones(512, np.float32)
    lat0 = np.ones((1, 512), np.float32)
    for k in (0, 5, 31):
        x = np.zeros((1, d_r), np.float32)
        x[0, 2 * k] = 1.0  # first feature of pair k only
        _, r0 = oracle.cache_append(lat0, x, ones, tab, [0])
        _, r1 = oracle.cache_append(lat0, x, ones, tab, [1])
        assert np.array_equal(r0[0], x[0].astype(np.float64))  # angle 0: identity
        want = np.zeros(d_r)
        want[2 * k], want[2 * k + 1] = c1, s1  # (1, 0) turns to (cos, sin)
        assert np.array_equal(r1[0], want)
        y = np.zeros((1, d_r), np.float32)
        y[0, 2 * k + 1] = 1.0  # (0, 1) turns to (-sin, cos)
        _, r2 = oracle.cache_append(lat0, y, ones, tab, [1])
        want = np.zeros(d_r)
        want[2 * k], want[2 * k + 1] = -s1, c1
        assert np.array_equal(r2[0], want)


def test_rotation_preserves_pair_norms_and_composes():
    g = rng(43)
    N, d_r = 6, 64
    x = g.standard_normal((N, d_r)).astype(np.float32)
    a = g.uniform(-math.pi, math.pi, (N, 32))
    b = g.uniform(-math.pi, math.pi, (N, 32))
    lat = np.ones((N, 512), np.float32)
    ones = np.ones(512, np.float32)
    pos = np.arange(N, dtype=np.int32)
    ta, tb, tab = _angles_table(a), _angles_table(b), _angles_table(a + b)
    _, ra = oracle.cache_append(lat, x, ones, ta, pos)
    n_in = np.hypot(x[:, 0::2].astype(np.float64), x[:, 1::2])
    n_out = np.hypot(ra[:, 0::2], ra[:, 1::2])
    # float32 cos/sin are within 2^-24 of a unit vector
    np.testing.assert_allclose(n_out, n_in, rtol=2e-7)
    # rotating by a, then by b, equals rotating by a + b (up to the float32
    # rounding of the tables and of the intermediate result)
    _, rab = oracle.cache_append(lat, ra.astype(np.float32), ones, tb, pos)
    _, rs = oracle.cache_append(lat, x, ones, tab, pos)
    np.testing.assert_allclose(rab, rs, atol=2e-6 * np.abs(x).max())
    # and the table row is chosen by position, not by row number
    _, rrev = oracle.cache_append(lat[::-1].copy(), x[::-1].copy(), ones, ta, pos[::-1].copy())
    np.testing.assert_array_equal(rrev[::-1], ra)


def test_cache_append_rejects_positions_outside_the_table():
    lat = np.ones((2, 512), np.float32)
    kp = np.ones((2, 64), np.float32)
    tab = _angles_table(np.zeros((3, 32)))
    with pytest.raises(ValueError):
        oracle.cache_append(lat, kp, np.ones(512, np.float32), tab, [0, 3])
    with pytest.raises(ValueError):
        oracle.cache_append(lat, kp, np.ones(512, np.float32), tab, [-1, 0])


# --------------------------------------------------------------------------
# several query tokens per sequence (the token axis of the decode einsums)
# --------------------------------------------------------------------------

def _multi_problem(seed, B, s_q, n_h, T, d_c=16, d_r=4):
    g = rng(seed)
    return dict(q_lat=g.standard_normal((B, s_q, n_h, d_c)),
                q_pe=g.standard_normal((B, s_q, n_h, d_r)),
                latent=g.standard_normal((B, T, d_c)), rope=g.standard_normal((B, T, d_r)))


def test_multi_token_with_one_token_is_the_single_token_function():
    p = _multi_problem(51, 3, 1, 4, 37)
    idx = np.stack([rng(52 + b).choice(37, 9, replace=False) for b in range(3)]).astype(np.int32)
    for topk in (None, idx):
        for causal in (False, True):
            o, lse = oracle.latent_attention_multi(p["q_lat"], p["q_pe"], p["latent"], p["rope"],
                                                   topk_idx=topk, scale=0.4, causal=causal)
            o1, l1, _ = oracle.latent_attention(p["q_lat"][:, 0], p["q_pe"][:, 0], p["latent"],
                                                p["rope"], topk_idx=topk, scale=0.4,
                                                want_lse=True)
            np.testing.assert_allclose(o[:, 0], o1, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[:, 0], l1, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_multi_token_reduces_to_single_token_over_its_visible_prefix(causal):
    B, s_q, n_h, T = 2, 5, 3, 23
    p = _multi_problem(53, B, s_q, n_h, T)
    o, lse = oracle.latent_attention_multi(p["q_lat"], p["q_pe"], p["latent"], p["rope"],
                                           scale=0.3, causal=causal)
    for j in range(s_q):
        Tj = T - s_q + j + 1 if causal else T
        oj, lj, _ = oracle.latent_attention(p["q_lat"][:, j], p["q_pe"][:, j], p["latent"],
                                            p["rope"], T=Tj, scale=0.3, want_lse=True)
        np.testing.assert_allclose(o[:, j], oj, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, j], lj, rtol=1e-12)
    if causal:  # the last token sees everything, the first one does not
        full, _, _ = oracle.latent_attention(p["q_lat"][:, 0], p["q_pe"][:, 0], p["latent"],
                                             p["rope"], scale=0.3)
        assert np.max(np.abs(o[:, 0] - full)) > 1e-6


def test_causal_corner_first_token_of_a_full_block_sees_one_position():
    # T == s_q: token 0 sits at position 0 and may only see it, so its output
    # is that latent row and its lse is its own score
    B, s_q, n_h, T = 2, 4, 3, 4
    p = _multi_problem(55, B, s_q, n_h, T)
    o, lse = oracle.latent_attention_multi(p["q_lat"], p["q_pe"], p["latent"], p["rope"],
                                           scale=0.7, causal=True)
    for b in range(B):
        for h in range(n_h):
            np.testing.assert_allclose(o[b, 0, h], p["latent"][b, 0], rtol=1e-14)
            z = 0.7 * (p["q_lat"][b, 0, h] @ p["latent"][b, 0] + p["q_pe"][b, 0, h] @ p["rope"][b, 0])
            assert lse[b, 0, h] == pytest.approx(z, rel=1e-13, abs=1e-13)


def test_causal_with_an_index_set_that_hides_every_visible_row():
    # the index set holds only the last position: the first token sees none of
    # it (empty sum: zero output, lse -inf), the last token sees only it
    B, s_q, n_h, T = 1, 3, 2, 10
    p = _multi_problem(57, B, s_q, n_h, T)
    idx = np.array([[T - 1]], np.int32)
    o, lse = oracle.latent_attention_multi(p["q_lat"], p["q_pe"], p["latent"], p["rope"],
                                           topk_idx=idx, causal=True)
    assert np.all(o[0, 0] == 0.0) and np.all(np.isneginf(lse[0, 0]))
    np.testing.assert_allclose(o[0, 2], np.broadcast_to(p["latent"][0, T - 1], (n_h, 16)),
                               rtol=1e-14)


# --------------------------------------------------------------------------
# ordinary attention over reconstructed keys and values (prefill excerpt)
# --------------------------------------------------------------------------

def _naive_problem(seed, B, S, T, n_h, d_qk=12, d_v=5):
    g = rng(seed)
    return (g.standard_normal((B, S, n_h, d_qk)), g.standard_normal((B, T, n_h, d_qk)),
            g.standard_normal((B, T, n_h, d_v)))


@pytest.mark.parametrize("S,T,causal,K", [(7, 7, True, None), (5, 11, True, 4),
                                          (6, 9, False, 3), (4, 4, False, None),
                                          (6, 13, False, "dirty"), (9, 12, True, "dirty")])
def test_attention_naive_matches_torch_sdpa(S, T, causal, K):
    B, n_h = 2, 3
    q, k, v = _naive_problem(61 + S + T, B, S, T, n_h)
    allowed = np.ones((B, S, T), bool)
    idx = None
    if K == "dirty":
        # repeats and entries outside [0, T) (the reading of the scatter as a
        # set); each query's own position is listed so none is left empty
        g = rng(64)
        idx = _dirty_sets(g, B * S, T, 10, n_bad=3, n_rep=2).reshape(B, S, 10)
        for b in range(B):
            for s in range(S):
                idx[b, s, g.integers(10)] = T - S + s
        allowed = _set_mask(idx, T)
    elif K:
        g = rng(62)
        # every query keeps at least one visible key: the last row of the set
        # is its own position
        idx = np.empty((B, S, K), np.int32)
        for b in range(B):
            for s in range(S):
                own = T - S + s
                others = g.choice(np.delete(np.arange(T), own), K - 1, replace=False)
                idx[b, s] = np.concatenate([others, [own]])
        allowed[:] = False
        for b in range(B):
            for s in range(S):
                allowed[b, s, idx[b, s]] = True
    if causal:
        allowed &= np.arange(T)[None, None, :] <= (T - S + np.arange(S))[None, :, None]
    out, lse = oracle.attention_naive(q, k, v, topk_idx=idx, causal=causal, scale=0.35)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    mask = torch.from_numpy(allowed)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=0.35)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)
    z = 0.35 * torch.einsum("bhsd,bhtd->bhst", tq, tk).masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).permute(0, 2, 1).numpy(), rtol=1e-12)


def test_attention_naive_first_causal_row_and_hidden_queries():
    B, S, T, n_h = 1, 4, 4, 2
    q, k, v = _naive_problem(63, B, S, T, n_h)
    out, lse = oracle.attention_naive(q, k, v, causal=True, scale=0.5)
    np.testing.assert_allclose(out[0, 0], v[0, 0], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 0.5 * np.sum(q[0, 0] * k[0, 0], -1), rtol=1e-13)
    # an index set that lies wholly after a query hides every key from it
    idx = np.full((B, S, 1), T - 1, np.int32)
    out, lse = oracle.attention_naive(q, k, v, topk_idx=idx, causal=True)
    assert np.all(out[0, :3] == 0.0) and np.all(np.isneginf(lse[0, :3]))
    np.testing.assert_allclose(out[0, 3], v[0, 3], rtol=1e-14)


def test_attention_naive_one_query_equals_the_naive_decode():
    # reconstruct K and V with the reconstruction function, attend with one
    # query at the end: the naive decode does both steps itself
    p = tiny_problem(65, 2, 3, 9)
    idx = np.stack([rng(66 + b).choice(9, 4, replace=False) for b in range(2)]).astype(np.int32)
    ref = oracle.decode_naive(p["q_nope"], p["q_pe"], p["latent"], p["rope"], p["w"],
                              topk_idx=idx, scale=0.3, d_n=p["d_n"], d_v=p["d_v"])["out"]
    B, T = 2, 9
    K, V = oracle.kv_reconstruct(p["latent"].reshape(B * T, -1), p["rope"].reshape(B * T, -1),
                                 p["w"], 3, d_n=p["d_n"], d_v=p["d_v"])
    q = np.concatenate([p["q_nope"], p["q_pe"]], -1)[:, None]
    out, _ = oracle.attention_naive(q, K.reshape(B, T, 3, -1), V.reshape(B, T, 3, -1),
                                    topk_idx=idx[:, None], causal=True, scale=0.3)
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-12, atol=1e-13)
