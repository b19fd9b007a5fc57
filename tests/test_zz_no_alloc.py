"""The allocation-free decode step (mla_decode_step_noalloc) against the
workspace step (mla_decode_step): same kernels, so the same bits. Two calls
in a row on the library's fixed scratch, the second with a smaller input;
a step too large for the scratch is rejected on the host."""
import pytest
import torch

from head_latent_attention_mla_amd import binding as mla
from head_latent_attention_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, n_h, T, K, seed):
    inp = synth.decode_inputs(B, n_h, T, torch.bfloat16, seed=seed, topk=K)
    x = {k: v.to(DEV) for k, v in inp.items()}
    return x


def _both(x, topk=None):
    cache = x["cache"]
    args = (x["q_nope"], x["q_pe"], x["wkv_b"], cache[..., :512], cache[..., 512:])
    ref, ref_lse = mla.mla_decode_step(*args, topk_idx=topk, want_lse=True)
    out = torch.empty_like(ref)
    lse = torch.empty_like(ref_lse)
    mla.mla_decode_step_noalloc(*args, out=out, topk_idx=topk, lse=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def test_noalloc_step_gives_the_bits_of_the_workspace_step_twice():
    print("noalloc call 1: B=32 n_h=128 T=4096 dense", flush=True)
    x = _inputs(32, 128, 4096, None, seed=301)
    ref, ref_lse, out, lse = _both(x)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse, ref_lse)
    del x
    print("noalloc call 2: B=3 n_h=128 T=700 top-300", flush=True)
    y = _inputs(3, 128, 700, 300, seed=302)
    ref, ref_lse, out, lse = _both(y, topk=y["topk_idx"])
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse, ref_lse)


def test_noalloc_step_rejects_a_step_beyond_the_scratch():
    # B=512, n_h=128: q_lat and out_lat alone are 2 x 64 MiB
    B, n_h, T = 512, 128, 64
    q = torch.zeros((B, n_h, 128), dtype=torch.bfloat16, device=DEV)
    qp = torch.zeros((B, n_h, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((n_h * 256, 512), dtype=torch.bfloat16, device=DEV)
    cache = torch.zeros((B, T, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, n_h, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_step_noalloc(q, qp, w, cache[..., :512], cache[..., 512:], out=out)
    assert "scratch" in str(e.value)
