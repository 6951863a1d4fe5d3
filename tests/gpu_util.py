"""Helpers shared by the GPU parity tests (device plumbing and error metrics)."""
import sys

import numpy as np
import torch

from hybrid_attention_ssm_swa_amd.layer import MixerLayer, make_kv, upload  # noqa: F401

# Parity bars: max |gpu - oracle| <= TOL * RMS(oracle), per checked tensor.
# The bf16 bar is the one stated for bf16 workloads; tensors held in fp16 inside
# a bf16 layer are held to the same bar.
TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}


def tdt(dtype: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def act(dtype: str) -> str:
    """Activation type of a layer of storage type `dtype` (bf16 layers compute in fp16)."""
    return "f16" if dtype == "bf16" else dtype


def dev(a, dtype: str):
    return upload(np.asarray(a, dtype=np.float32), tdt(dtype), "cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms)


def check(name, got, ref, dtype):
    """The spec bar: max |gpu - oracle| <= TOL * RMS(oracle)."""
    e = rel_err(got, ref)
    print(f"  {name}: max|err|/rms = {e:.3e} (bar {TOL[dtype]:.0e})", flush=True)
    assert e <= TOL[dtype], f"{name}: {e:.3e} > {TOL[dtype]}"
    return e


UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def round_to(a, dtype: str) -> np.ndarray:
    """a rounded to the 16-bit storage type (round to nearest even), back in fp64."""
    t = torch.from_numpy(np.asarray(a, np.float64)).to(tdt(dtype))
    return t.double().numpy()


def check_stored(name, got, ref, dtype):
    """For a tensor stored in a 16-bit type (a layer's bf16 output, an fp16 activation):
    each element may also carry its own storage rounding, so the bar is
    |err_i| <= TOL * RMS(ref) + u * |ref_i| (u the type's unit roundoff, 2^-8 for bf16).
    Even the correctly rounded exact answer needs this: a bf16 element with |y| in
    [8, 16) has an ulp of 2^-4, so its rounding alone can exceed 2e-2 x RMS when
    RMS(y) ~ 1.5.  Reports the plain max|err|/RMS and max_i |err_i| / bound_i (<= 1)."""
    if dtype not in UNIT_ROUNDOFF:
        return check(name, got, ref, dtype)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    bound = TOL[dtype] * rms + UNIT_ROUNDOFF[dtype] * np.abs(ref)
    r = float(np.max(np.abs(got - ref) / bound))
    e = rel_err(got, ref)
    # the floor: the exact reference itself rounded to the storage type
    floor = rel_err(round_to(ref, dtype), ref)
    print(f"  {name}: max|err|/rms = {e:.3e} (storage-rounding floor {floor:.3e}); "
          f"max err/(bar*rms + u|ref|) = {r:.3f}", flush=True)
    assert r <= 1.0, f"{name}: {r:.3f} > 1"
    return r


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_bound(name, got, ref, bound):
    """max_i |err_i| / bound_i <= 1 for an elementwise bound derived from the arithmetic."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    r = float(np.max(np.abs(got - ref) / bound))
    print(f"  {name}: max|err|/rms = {rel_err(got, ref):.3e}; max err/bound = {r:.3f}", flush=True)
    assert r <= 1.0, f"{name}: {r:.3f} > 1"
    return r
