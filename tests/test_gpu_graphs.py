"""The library's calls inside a captured HIP graph: every replay gives the
bits of the eager calls (workspace clears and index-set scatters are
kernels, never memset nodes). Eager work and synchronisations run between
the replays."""
import pytest
import torch

from head_latent_attention_mla_amd import binding as mla
from head_latent_attention_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.dtype == torch.bfloat16
                                              else torch.int32).clone()


def test_decode_step_append_and_attention_replay_like_eager():
    B, n_h, T = 8, 128, 1000
    inp = synth.decode_inputs(B, n_h, T, torch.bfloat16, seed=21, topk=300)
    d = {k: v.to(DEV) for k, v in inp.items()}
    app = synth.append_inputs(B, B, T, torch.bfloat16, seed=22)
    a = {k: v.to(DEV) for k, v in app.items()}
    att = synth.attention_inputs(1, 300, 300, 2, torch.bfloat16, seed=23, topk=40)
    t = {k: v.to(DEV) for k, v in att.items()}

    cache = d["cache"].clone()
    out = torch.empty((B, n_h, 128), dtype=torch.bfloat16, device=DEV)
    out_sparse = torch.empty_like(out)
    att_out = torch.empty((1, 300, 2, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(mla.mla_decode_step_workspace_bytes(B, 1, n_h, T, 0), dtype=torch.uint8,
                     device=DEV)
    ws_sp = torch.empty(mla.mla_decode_step_workspace_bytes(B, 1, n_h, T, 300),
                        dtype=torch.uint8, device=DEV)
    ws_att = torch.empty(mla.mla_attention_naive_workspace_bytes(1, 300, 300, 40),
                         dtype=torch.uint8, device=DEV)

    def work():
        cache.copy_(d["cache"])
        mla.mla_cache_append(a["kv_a"], a["gamma"], a["freqs"], a["pos"], cache[..., :512],
                             cache[..., 512:])
        mla.mla_decode_step(d["q_nope"], d["q_pe"], d["wkv_b"], cache[..., :512],
                            cache[..., 512:], out=out, workspace=ws)
        mla.mla_decode_step(d["q_nope"], d["q_pe"], d["wkv_b"], cache[..., :512],
                            cache[..., 512:], topk_idx=d["topk_idx"], out=out_sparse,
                            workspace=ws_sp)
        mla.mla_attention_naive(t["q"], t["k"], t["v"], topk_idx=t["topk_idx"], causal=True,
                                out=att_out, workspace=ws_att)

    work()
    torch.cuda.synchronize()
    ref = [bits(cache), bits(out), bits(out_sparse), bits(att_out)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        # scribble over every output and workspace between replays
        for x in (cache, out, out_sparse, att_out, ws, ws_sp, ws_att):
            x.view(torch.uint8).fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits(cache), bits(out), bits(out_sparse), bits(att_out)]
        for i, (x, y) in enumerate(zip(got, ref)):
            assert torch.equal(x, y), f"replay {rep}: output {i} differs from the eager call"
