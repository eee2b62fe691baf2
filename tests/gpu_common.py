"""Helpers shared by the GPU parity tests (upload seeded inputs, run, compare)."""
import numpy as np
import torch

import oracle
import weight_quantized_mlp_amd as wq

DEV = torch.device("cuda:0")


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_dev(bits):
    return dev(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def f16_dev(bits):
    return dev(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.float16)


def host(t):
    return t.detach().cpu().numpy()


def same_bits_f32(a, b, signed_zero=True):
    """Bitwise float32 equality (NaNs compared as a class).  signed_zero=False
    accepts +0 for -0: a sum that starts from +0 cannot return -0 for a -0 term."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    nan = np.isnan(a) & np.isnan(b)
    eq = a.view(np.uint32) == b.view(np.uint32)
    if not signed_zero:
        eq |= (a == 0) & (b == 0)
    return np.all(nan | eq)


def gate(y, ref, tol=1e-3, what=""):
    err, scale = oracle.normwise_rel_err(y, ref)
    print(f"[parity] {what}: normwise max rel err {err:.3e} (min row scale {scale:.3e})", flush=True)
    assert scale > 1e-6, "reference magnitude is trivial"
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol}"
    return err
