"""Host-side logic of bench.py (CPU only): the algorithmic byte models that the roofline
divides by, the lookup of measured HBM traffic, the CPU oracle baseline and the one-GPU
refusal.  Nothing here launches a kernel."""
import os
import subprocess
import sys

import pytest
import torch

import bench
import glu_activation_microscaling_amd as glu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _numel(ts):
    return sum(t.numel() * t.element_size() for t in ts)


@pytest.mark.parametrize("M,N", [(32, 64), (96, 160), (16384, 7168)])
def test_mxfp8_byte_model_is_inputs_plus_output_buffers(M, N):
    """Forward: gate and up read once, codes and scales of each direction written once;
    backward: gate, up and dh read, [dGate | dUp] ([M, 2N]) written.  The output sizes are
    those of the buffers the binding allocates (row-major scales, meta tensors: no memory)."""
    for rowwise, colwise, ndir in ((True, False, 1), (False, True, 1), (True, True, 2)):
        fwd = glu._mx_buffers(M, N, rowwise, colwise, "meta", None)
        bwd = glu._mx_buffers(M, 2 * N, rowwise, colwise, "meta", None)
        assert bench.mx_bytes(M, N, False, ndir) == 2 * (2 * M * N) + _numel(fwd)
        assert bench.mx_bytes(M, N, True, ndir) == 3 * (2 * M * N) + _numel(bwd)


@pytest.mark.parametrize("M,H", [(1, 16), (968, 16384), (16384, 7168)])
def test_nvfp4_and_bf16_byte_models(M, H):
    q, sf = glu._nv_buffers(M, H, "rowmajor", "meta", None)
    assert bench.nv_bytes(M, H) == 2 * (2 * M * H) + _numel([q, sf])
    q, sf = glu._nv_buffers(M, 2 * H, "rowmajor", "meta", None)
    assert bench.nv_bwd_bytes(M, H) == 3 * (2 * M * H) + _numel([q, sf])
    assert bench.bf16_bytes(M, H, False) == (2 + 1) * 2 * M * H
    assert bench.bf16_bytes(M, H, True) == (3 + 2) * 2 * M * H


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.h"
    a.write_text("int f() {\n  return 1;  // one\n}\n")
    b.write_text("// header\nint g;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a), str(b)])
    h0 = bench.kernel_source_sha256()
    a.write_text("// a new comment\nint f() {\n\n  return 1;  // uno\n}\n")
    assert bench.kernel_source_sha256() == h0
    a.write_text("int f() {\n  return 2;  // one\n}\n")
    assert bench.kernel_source_sha256() != h0


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha256()
    prof = tmp_path / "p.md"
    prof.write_text(f"traffic_record: kernel=k<1> source_sha256={sha} read_bytes=10 write_bytes=5\n"
                    f"traffic_record: kernel=k<2> source_sha256={'0' * 64} read_bytes=1 write_bytes=1\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.traffic_bytes("k<1>") == 15
    assert bench.traffic_bytes("k<2>") is None
    assert bench.traffic_bytes("k<3>") is None


def test_committed_counter_profile_matches_the_kernel_sources():
    """The roofline kernel's HBM traffic in profiles/ was taken on the current sources, so the
    bench line carries it (it would be null after a kernel change until the counters are
    taken again)."""
    t = bench.traffic_bytes("k_mxfp8<0,0,3,1>")
    assert t is not None
    alg = bench.mx_bytes(16384, 7168, True, 2)
    assert 0.99 * alg <= t <= 1.05 * alg


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    import synthetic_inputs as si
    r = bench.cpu_baseline(si, 0.01)  # one 512-row slab
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1
    assert r["value"] > 0 and r["sample"].startswith("512 rows")


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr and not p.stdout.strip()


def test_no_visible_gpu_fails_loudly():
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 1 and "no GPU visible" in p.stderr and not p.stdout.strip()
