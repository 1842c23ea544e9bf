"""Helpers for the GPU parity tests: moving seeded inputs to the device,
reading results back, and the floating-point tolerance of the layer outputs.

Tolerance (written here, used by every floating-point parity check): relative
Frobenius error <= 5e-3 and max |err| <= 2e-2 * RMS(reference), each output
checked against its own reference (fp32 accumulation of bf16 operands, bf16
outputs).
"""

import numpy as np

FRO_TOL = 5e-3
MAX_TOL = 2e-2


def torch_mod():
    import torch
    return torch


def dev_f32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16_bits(t):
    torch = torch_mod()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.contiguous().cpu().numpy()


def bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = got - ref
    ref_norm = np.linalg.norm(ref)
    rms = ref_norm / np.sqrt(ref.size)
    fro = np.linalg.norm(err) / max(ref_norm, 1e-300)
    mx = np.max(np.abs(err)) / max(rms, 1e-300)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert fro <= FRO_TOL, f"{name}: relative Frobenius error {fro:.3e} > {FRO_TOL}"
    assert mx <= MAX_TOL, f"{name}: max error {mx:.3e} x RMS > {MAX_TOL}"
    return fro, mx
