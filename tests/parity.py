"""The parity bar for GPU results against the fp64 oracle: cosine similarity
>= 0.9995 and max |gpu - ref| <= 2e-2 * RMS(ref), element by element on the
same seeded inputs."""
import numpy as np

COS_MIN = 0.9995
MAXABS_REL = 2e-2
# Block deltas (h_out - h_in) are a stricter, extra check.  With bf16 GEMM
# inputs, rounding the modulated activations alone gives max|err| up to ~0.03
# x RMS(delta) against exact fp64 (emulated on the CPU at the storage points
# the kernels use), so deltas are held to 5e-2 x RMS and the same cosine.
DELTA_REL = 5e-2
# Sharp attention (q/k RMSNorm gains near 2, logits ~4x the canonical ones):
# the error of a logit from the bf16 rounding of q and k grows with the
# logit, and the same CPU emulation gives max|err| ~0.043 x RMS(delta) for
# the sharp test case (0.034 from rounding q and k alone, against 0.003 with
# gains <= 1.5), so sharp cases are held to 8e-2.
SHARP_DELTA_REL = 8e-2


def stats(gpu, ref):
    g = np.asarray(gpu, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    assert g.shape == r.shape, (g.shape, r.shape)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r) + 1e-300)) if r.size else 1.0
    mx = float(np.max(np.abs(g - r))) if r.size else 0.0
    return cos, mx, rms


def assert_parity(gpu, ref, name="", cos_min=COS_MIN, rel=MAXABS_REL):
    g = np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in the GPU result"
    cos, mx, rms = stats(gpu, ref)
    msg = f"{name}: cos={cos:.7f} maxabs={mx:.3e} rms={rms:.3e} ratio={mx / (rms + 1e-300):.3e}"
    print(msg)
    assert cos >= cos_min and mx <= rel * rms, msg
    return cos, mx, rms
