"""Helpers for the GPU parity tests: device upload through the library's own
entry points, case logging that survives a lost box, tolerance checks."""
import sys

import numpy as np

TOL = 2e-3  # max |y - y64| / sum_k |x w|, fp32 accumulation, fp16 output


def log(msg: str):
    """Write straight to the process stderr (not captured), flushed, so the
    case in flight is named even if the run dies."""
    sys.__stderr__.write(f"[case] {msg}\n")
    sys.__stderr__.flush()


def torch_mod():
    import torch
    return torch


def to_dev(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def upload_layer(q, z, s):
    """Codes, zero points and scales (numpy) -> device qweight, packed zeros,
    scales, packed on the GPU by awq_pack / awq_pack_zeros."""
    import weight_only_bit_awq_amd as awq
    torch = torch_mod()
    qd = to_dev(q)
    zd = to_dev(z)
    sd = to_dev(s.view(np.uint16)).view(torch.float16)
    qw = awq.pack(qd)
    zw = awq.pack_zeros(zd)
    del qd, zd
    return qw, zw, sd


def x_dev(x):
    torch = torch_mod()
    return to_dev(x.view(np.uint16)).view(torch.float16)


def to_np16(t):
    torch = torch_mod()
    return t.detach().cpu().view(torch.int16).numpy().view(np.float16)


def check_close(yhat16, y64, D, tol=TOL, what=""):
    """Normalised error against the oracle; also no NaN/inf."""
    import oracle
    y = yhat16.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = oracle.normalised_error(y, y64, D)
    assert err <= tol, f"{what}: normalised error {err:.3e} > {tol}"
    return err
