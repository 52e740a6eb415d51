"""Comparison helpers shared by the GPU parity tests.

Gates (per output tensor, GPU result upcast exactly to float64 against the
float64 oracle on the same stored inputs):
  * max-abs error: 1e-4 (fp32 path), 2e-2 (bf16), 6e-2 (bf16 q with fp8 KV);
  * relative L2 error ||gpu - ref|| / ||ref||: 1e-5 (fp32), 1e-2 (bf16 and
    fp8-KV). Attention outputs at long context have entries of size ~0.02, so
    the max-abs bound alone would accept an all-zero output; the relative L2
    gate does not (the negative-control tests check exactly that).
"""

import numpy as np

TOL = {
    "f32": dict(atol=1e-4, rel=1e-5, lse=1e-4),
    "bf16": dict(atol=2e-2, rel=1e-2, lse=2e-3),
    "fp8_e4m3": dict(atol=6e-2, rel=1e-2, lse=2e-3),
}


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def passes(got, ref, atol, rel):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape or not np.all(np.isfinite(got)):
        return False
    return float(np.max(np.abs(got - ref))) <= atol and rel_l2(got, ref) <= rel


def check(name, got, ref, atol, rel, quiet=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in GPU output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    r = rel_l2(got, ref)
    if not quiet or err > atol or r > rel:
        print(f"[parity] {name}: max_abs={err:.3e} (tol {atol:g}) rel_l2={r:.3e} (tol {rel:g})", flush=True)
    assert err <= atol, f"{name}: max abs error {err:.3e} > {atol}"
    assert r <= rel, f"{name}: relative L2 error {r:.3e} > {rel}"


def check_lse(name, got, ref, atol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_g, inf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(inf_g, inf_r), f"{name}: -inf pattern differs"
    fin = ~inf_r
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    print(f"[parity] {name}: max_abs={err:.3e} (tol {atol:g})", flush=True)
    assert err <= atol, f"{name}: lse error {err:.3e} > {atol}"
