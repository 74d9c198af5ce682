"""Shared helpers for the GPU parity tests: seeded inputs on the device and the
comparison metrics.  Inputs come from sub_quadratic_factorized_amd.workloads
(the same generator feeds the oracle); expected values come from the oracle."""

from __future__ import annotations

import json
import os
import sys

import numpy as np

from sub_quadratic_factorized_amd import workloads as wl

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_REL_L2 = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def workload_device_inputs(w: wl.Workload, seed: int = 0):
    """(q, k, v) device tensors [B, n, heads, d] for a named workload."""
    return wl.device_inputs(w, seed)


def host_to_device(arrs, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return tuple(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdt) for a in arrs)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm((got - ref).ravel()) / den) if den > 0 else max_abs
    return max_abs, rel


def _record(entry):
    path = os.environ.get("PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def assert_close_bf16_output(got, ref, what=""):
    """The bf16 bar for outputs stored in bf16 at any magnitude.

    rel-L2 <= 5e-3, and max |got - ref| <= 2e-2 plus half the bf16 spacing at
    |ref|: an output stored in bf16 cannot lie closer to the exact value than
    that (2^-6 at |ref| in [4, 8), 2^-7 in [2, 4)), and the pages keep all
    attention computation, so the outputs too, in bfloat16.  Below |ref| = 1
    the added term is at most 2^-9.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs, rel = errors(got, ref)
    half = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    excess = float(np.max(np.abs(got - ref) - half)) if got.size else 0.0
    log(f"  {what}: max_abs={max_abs:.3e} max(|err| - half spacing)={excess:.3e} rel_l2={rel:.3e} "
        f"max|ref|={np.max(np.abs(ref)):.3f}")
    _record({"case": what, "dtype": "bf16", "max_abs": max_abs, "max_abs_less_half_spacing": excess,
             "rel_l2": rel, "max_ref": float(np.max(np.abs(ref)))})
    assert excess <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, excess, rel)
    return max_abs, rel


def assert_close(got, ref, dtype, what="", magnitude_scaled=False):
    """Check the parity bar.

    bf16: max |got - ref| <= 2e-2 and rel-L2 <= 5e-3.  With magnitude_scaled the
    absolute bar applies to |got - ref| / max(1, |ref|): bf16 storage of Y and O
    has a half-ulp of 2^-9 |x|, so outputs beyond 1 in magnitude (sharp
    attention copying single values) need the bar scaled with them.
    float32: rel-L2 <= 1e-5.
    """
    max_abs, rel = errors(got, ref)
    scaled = max_abs
    if magnitude_scaled:
        scaled = float(np.max(np.abs(np.asarray(got) - ref) / np.maximum(1.0, np.abs(ref))))
    log(f"  {what}: max_abs={max_abs:.3e} scaled={scaled:.3e} rel_l2={rel:.3e} max|ref|={np.max(np.abs(ref)):.3f}")
    _record({"case": what, "dtype": dtype, "max_abs": max_abs, "scaled_max": scaled, "rel_l2": rel,
             "max_ref": float(np.max(np.abs(ref))), "magnitude_scaled": magnitude_scaled})
    if dtype == "bf16":
        assert scaled <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, scaled, rel)
    else:
        assert rel <= F32_REL_L2, (what, max_abs, rel)
    return max_abs, rel
