"""Shared helpers for the GPU parity tests: uploads, tolerances, seeded inputs."""
import numpy as np

import synth

F32_REL = 1e-5      # f32 paths: |gpu - oracle| <= 1e-5 * S + 1e-6
F32_ABS = 1e-6
BF16_REL = 5e-3     # bf16-MFMA batched path: <= 5e-3 * S


def to_dev(a, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_f32(got, ref, S, what, rel=F32_REL, abs_=F32_ABS):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    tol = rel * S + abs_
    err = np.abs(got - ref)
    bad = err > tol
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                           f"err/tol={np.max(err / tol):.3g} at {np.unravel_index(np.argmax(err / tol), err.shape)}")
    return float(np.max(err / tol))


def swiglu_tol(r):
    """First-order propagation of the per-dot f32 bound through silu(g)*u
    (sup |silu'| < 1.1), plus 1e-6*|out| for the device exp and division."""
    silu_g = r["g"] / (1.0 + np.exp(-r["g"]))
    return (1.1 * (F32_REL * r["Sg"] + F32_ABS) * np.abs(r["u"])
            + np.abs(silu_g) * (F32_REL * r["Su"] + F32_ABS)
            + 1e-6 * np.abs(r["out"]) + 1e-6)


def q8_weights(seed, n_out, n_in):
    raw, _ = synth.q8_0_weights(seed, n_out, n_in)
    return raw


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)
