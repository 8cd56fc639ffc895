"""Comparison rules between the HIP library and the CPU oracle.

* Integer scans, min/max scans and select: bit-exact.
* float32 add: |gpu - ref| <= 1e-5 * A_i + 1e-6, where ref is the oracle's
  double accumulator and A_i = sum_{j<=i} |x_j| (the same bound is used for
  inclusive and exclusive outputs).
* bf16/f16 add: within one output ulp of the oracle's output (the double sum
  rounded to float32, then to the 16-bit format, nearest-even), or within the
  float32 bound above (the union covers prefixes that cancel towards zero,
  where one 16-bit ulp is finer than legitimate float32 regrouping error).
* float64 add (outside the five workloads): |gpu - ref| <= 1e-12 * A_i + 1e-300.
* products (row scans, float32 accumulation): a product of m factors formed
  with m - 1 float32 roundings, in any grouping, is within
  gamma = (m-1)u / (1 - (m-1)u) (u = 2^-24) of the exact product relative to
  it; the oracle's double product adds at most m * 2^-53.  The check is
  |gpu - ref| <= 1.01 * (gamma + m 2^-52) |ref|, plus half an output ulp
  (at the GPU's value) for bf16/f16 outputs, which are rounded once from the
  float32 product.
"""
import numpy as np

import oracle
import torch

FP_REL, FP_ABS = 1e-5, 1e-6


def decode16(bits, dtype):
    """16-bit patterns -> float64, decoded by torch/numpy."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return bits.view(np.float16).astype(np.float64)


def ulp16(y, dtype):
    """Spacing of the 16-bit format at |y| (the subnormal spacing at 0)."""
    p, emin = (8, -126) if dtype == "bf16" else (11, -14)
    a = np.abs(y)
    _, e = np.frexp(a)                        # a = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)               # exponent of the binade, floored at the normal range
    return np.ldexp(1.0, e - (p - 1))


def check_fp_add(gpu, ora_out, ref, absref, dtype, label=""):
    """Assert the float-add tolerance; returns (max abs err, max err / bound)."""
    gpu = np.asarray(gpu)
    if dtype in ("bf16", "f16"):
        g = decode16(gpu, dtype)
        ro = decode16(ora_out, dtype)
        bound = FP_REL * absref + FP_ABS
        ok = (np.abs(g - ro) <= ulp16(ro, dtype)) | (np.abs(g - ref) <= bound)
        err = np.abs(g - ref)
    else:
        g = gpu.astype(np.float64)
        if dtype == "f64":
            bound = 1e-12 * absref + 1e-300
        else:
            bound = FP_REL * absref + FP_ABS
        err = np.abs(g - ref)
        ok = err <= bound
    if not ok.all():
        bad = np.flatnonzero(~ok.ravel())
        i = bad[0]
        raise AssertionError(
            f"{label}: {bad.size} of {ok.size} outputs out of tolerance; first at flat index {i}: "
            f"gpu={g.ravel()[i]!r} ref={ref.ravel()[i]!r} A={absref.ravel()[i]!r}")
    ratio = float(np.max(err / (FP_REL * absref + FP_ABS))) if err.size else 0.0
    return float(err.max()) if err.size else 0.0, ratio


def check_exact(gpu, ora, label=""):
    gpu = np.ascontiguousarray(gpu)
    ora = np.ascontiguousarray(ora)
    assert gpu.shape == ora.shape and gpu.dtype.itemsize == ora.dtype.itemsize, \
        (label, gpu.shape, ora.shape)
    if gpu.size == 0:
        return
    gb = gpu.reshape(-1).view(np.uint8).reshape(gpu.size, -1)
    ob = ora.reshape(-1).view(np.uint8).reshape(ora.size, -1)
    if not np.array_equal(gb, ob):
        diff = np.flatnonzero(~np.all(gb == ob, axis=1))
        i = diff[0]
        raise AssertionError(f"{label}: {diff.size} of {gpu.size} elements differ; first at "
                             f"flat index {i}: gpu={gpu.ravel()[i]!r} oracle={ora.ravel()[i]!r}")


def check_fp_mul(gpu, ref, m, dtype, label=""):
    """Assert the product bound; m[i] = number of factors behind output i.

    Returns the largest error as a fraction of its bound.
    """
    gpu = np.asarray(gpu)
    g = decode16(gpu, dtype) if dtype in ("bf16", "f16") else gpu.astype(np.float64)
    m = np.asarray(m, dtype=np.float64)
    k = np.maximum(m - 1, 0)
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    bound = 1.01 * (gamma + m * 2.0 ** -52) * np.abs(ref)
    if dtype in ("bf16", "f16"):
        bound = bound + 0.5 * ulp16(g, dtype)
    err = np.abs(g - ref)
    ok = err <= bound
    if not ok.all():
        bad = np.flatnonzero(~ok.ravel())
        i = bad[0]
        raise AssertionError(
            f"{label}: {bad.size} of {ok.size} outputs out of tolerance; first at flat index {i}: "
            f"gpu={g.ravel()[i]!r} ref={ref.ravel()[i]!r} m={m.ravel()[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, 0.0)
    return float(r.max()) if r.size else 0.0


def check_stable_by_image(keys_in, keys_out, idx_out, dt, label):
    """The stable ascending order by the oracle's sort image is unique, and an
    output (keys, original index of each key) is that order exactly when:
      - the carried indices are a permutation of [0, n);
      - every output key is the input key at its carried index, bit for bit;
      - the oracle's images of the output keys never decrease, and where two
        neighbours' images are equal their indices increase (stability).
    Checked with numpy, so no library sort is involved: the oracle's order
    definition (oracle.sort_image) applied at sizes where the oracle's own
    argsort would take minutes."""
    n = keys_in.size
    assert keys_out.size == n and idx_out.size == n, f"{label}: length changed"
    if n == 0:
        return
    assert idx_out.min() >= 0 and idx_out.max() < n, f"{label}: index out of range"
    seen = np.zeros(n, dtype=bool)
    seen[idx_out] = True
    assert seen.all(), f"{label}: not a permutation"
    del seen
    assert np.array_equal(keys_out.view(np.uint8), keys_in[idx_out].view(np.uint8)), \
        f"{label}: a key moved without its index"
    img = oracle.sort_image(keys_out, dt)
    step_up = img[1:] > img[:-1]
    tie_ok = (img[1:] == img[:-1]) & (idx_out[1:] > idx_out[:-1])
    bad = ~(step_up | tie_ok)
    assert not bad.any(), f"{label}: out of order at {int(np.argmax(bad))}"
