"""Code-generation checks on the library's own kernels, compiled here for gfx950 (CPU only).

Parity tests see the bytes a kernel writes, not how it moves them. These checks read the
assembly that the library's sources and flags produce and pin what the bytes cannot show:
  * no packed-FP32 VALU instruction anywhere (the build turns the target feature off, and no
    source writes one by hand);
  * the store forms the launch policies choose: the BF16 kernels instantiated for streaming
    stores emit non-temporal stores and the others ordinary ones (a run-time choice between two
    stores of the same value once compiled into a single ordinary store); the MXFP8 kernels
    carry both forms; the streaming probe streams every store.
"""
import os
import re
import shutil
from concurrent.futures import ThreadPoolExecutor

import pytest

from glu_activation_microscaling_amd import build

SOURCES = ["glu_bf16.hip", "glu_mxfp8.hip", "glu_nvfp4.hip", "glu_gemm.hip", "glu_stream.hip"]
PACKED_FP32 = re.compile(r"^\s+v_pk_(fma|mul|add)_f32\b", re.M)

pytestmark = pytest.mark.skipif(
    shutil.which(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")) is None,
    reason="hipcc not available")


@pytest.fixture(scope="module")
def asm():
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(build.device_asm, SOURCES)))


def kernels(text, stem):
    """{mangled name: body} of the kernels in `text` whose mangled name contains `stem`."""
    out = {}
    for m in re.finditer(r"^(_Z\S*" + re.escape(stem) + r"\S*):", text, re.M):
        end = text.index("s_endpgm", m.end())
        out[m.group(1)] = text[m.end():end]
    return out


def stores(body, op):
    """(non-temporal, ordinary) counts of the store instruction `op` in a kernel body."""
    lines = re.findall(r"^\s+" + op + r"\b.*$", body, re.M)
    nt = sum(1 for l in lines if re.search(r"\bnt\b", l))
    return nt, len(lines) - nt


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32_instructions(asm, src):
    found = PACKED_FP32.findall(asm[src])
    assert not found, f"{src}: {len(found)} packed-FP32 instructions"


def test_bf16_store_form_follows_the_template_flag(asm):
    ks = {**kernels(asm["glu_bf16.hip"], "k_glu_fwd_bf16"), **kernels(asm["glu_bf16.hip"], "k_glu_bwd_bf16")}
    streamed = {n: b for n, b in ks.items() if n.split("EEEv")[0].endswith("Lb1")}
    ordinary = {n: b for n, b in ks.items() if n.split("EEEv")[0].endswith("Lb0")}
    assert streamed and ordinary and len(streamed) + len(ordinary) == len(ks)
    for n, b in streamed.items():
        nt, plain = stores(b, "global_store_dwordx4")
        assert nt > 0 and plain == 0, (n, nt, plain)
    for n, b in ordinary.items():
        nt, plain = stores(b, "global_store_dwordx4")
        assert nt == 0 and plain > 0, (n, nt, plain)


def test_mxfp8_carries_both_store_forms(asm):
    nt, plain = stores(asm["glu_mxfp8.hip"], "buffer_store_dwordx4")
    assert nt > 0 and plain > 0, (nt, plain)


def test_stream_probe_streams_every_store(asm):
    for op in ("global_store_dwordx4", "global_store_dwordx2", "global_store_dword"):
        nt, plain = stores(asm["glu_stream.hip"], op)
        assert nt > 0 and plain == 0, (op, nt, plain)
