"""The generated assembly of every HIP source is free of MFMA result-read
hazards (see tests/isa_hazards.py). Needs hipcc, no GPU."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from head_latent_attention_mla_amd import _build

from isa_hazards import check_assembly

KERNEL_SOURCES = [s for s in _build.SOURCES if s != "capi.hip"]


def _asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [_build.HIPCC, *[f for f in _build.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.skipif(not os.path.exists(_build.HIPCC) and not shutil.which("hipcc"),
                    reason="hipcc is not installed")
def test_no_mfma_result_read_hazards(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, str(tmp_path)), KERNEL_SOURCES))
    found = []
    for t in texts:
        found += check_assembly(t)
    assert not found, "\n".join(found[:20])


def test_the_check_sees_a_read_across_a_branch():
    # a jump that skips the padding between an MFMA and the read of its result
    asm = "\n".join([
        "_Zdemo:",
        "  v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
        "  s_cbranch_scc1 .LBB0_2",
        "  s_nop 7",
        "  s_nop 7",
        ".LBB0_2:",
        "  v_accvgpr_read_b32 v8, a15",
        "  s_endpgm",
    ])
    assert len(check_assembly(asm)) == 1
    padded = asm.replace("  s_cbranch_scc1 .LBB0_2\n", "")
    assert check_assembly(padded) == []
