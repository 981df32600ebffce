"""Host logic of bench.py (no GPU): the algorithmic FLOP count behind
`value`, the traffic lookup keyed to the GEMM source, the per-family
roofline arithmetic and the refusal of more than one GPU."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _linear_flops(d, B, S_img, S_txt):
    """2 * tokens * out * in for every weight matrix of the model, each
    applied to the tokens it sees (from the tensor shape tables), plus the
    two products of joint attention per block."""
    tok = {"img": B * S_img, "txt": B * S_txt}
    per_stream = 0
    for st in synth.STREAMS:
        for name, (o, i) in ((n, s) for n, s in synth.stream_tensor_shapes(d).items() if n.endswith("_w")):
            t = B if name == "mod_w" else tok[st]      # AdaLN sees one temb per sample
            per_stream += 2 * t * o * i
    S = S_img + S_txt
    attn = 2 * 2 * B * S * S * d.head_dim * d.heads    # Q K^T and P V
    top = 0
    for name, (o, i) in ((n, s) for n, s in synth.top_tensor_shapes(d).items() if n.endswith("_w")):
        t = {"img_in_w": tok["img"], "txt_in_w": tok["txt"], "proj_out_w": tok["img"]}.get(name, B)
        top += 2 * t * o * i
    return d.n_blocks * (per_stream + attn) + top


def test_step_flops_match_the_model_shapes():
    d = synth.LENS
    for (si, st, b) in ((4096, 512, 2), (4096, 512, 1), (8100, 512, 1), (4050, 512, 8)):
        assert bench.step_flops(d, si, st, b)["total"] == _linear_flops(d, b, si, st)


def test_step_flops_of_the_benchmarked_step():
    # 1024^2 CFG step: 48 blocks, 4096 image + 512 text tokens, batch 2
    assert bench.step_flops(synth.LENS, 4096, 512, 2)["total"] == 37620520845312


def test_measured_traffic_follows_the_gemm_source(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_bytes(b"// some kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    prof.write_text(f"table\n\ntraffic_bytes_per_launch: 123456789\ngemm_source_sha256: {sha}\n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    assert bench.measured_traffic() == 123456789.0
    src.write_bytes(b"// the kernel changed\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


class _L:
    KERNEL_NAMES = ("gemm", "attention", "norm", "qknorm_rope", "adaln")


def test_family_roofline_arithmetic():
    steps = 4
    ms = [40.0, 20.0, 4.0, 0.0, 1.0]          # over all steps
    n = [400, 80, 200, 0, 8]
    flops = {"gemm": 1.0e13, "attention": 4.0e12}
    kernels, roof = bench.family_roofline(_L, ms, n, steps, flops)
    assert set(kernels) == {"gemm", "attention", "norm", "adaln"}
    assert roof["kernel"] == "gemm"
    per_launch = 1.0e13 / (400 / steps)
    avg_s = 40.0 / 400 * 1e-3
    assert roof["algorithmic_flops_per_launch"] == pytest.approx(per_launch)
    assert roof["achieved"] == pytest.approx(per_launch / avg_s / 1e12, abs=0.05)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2500.0, abs=1e-4)
    assert kernels["gemm"]["TFLOP/s"] == pytest.approx(1.0e13 / (10.0e-3) / 1e12, abs=0.05)
    assert kernels["norm"]["avg_launch_us"] == pytest.approx(20.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
