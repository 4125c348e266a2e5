"""Shared helpers for the GPU parity tests: host -> device copies and the parity bar."""

import json
import os

import numpy as np


def dev_bf16(bits, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_i32(arr, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(device)


def dev_u8(arr, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to(device)


def to_host(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_parity(o, l, o_ref, l_ref, what=""):
    """The bar: max|O - O_ref| <= 1e-2 * max|O_ref| + 2e-3 over the compared outputs;
    |LSE - LSE_ref| <= 1e-3 on rows with a finite reference; -inf rows match exactly
    (and their O is exactly 0)."""
    assert o.shape == o_ref.shape and l.shape == l_ref.shape
    finite = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref)), "%s: -inf rows differ" % what
    assert np.all(o[~finite] == 0), "%s: empty rows must be 0" % what
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    tol = 1e-2 * np.abs(o_ref).max() + 2e-3
    err = np.abs(o - o_ref).max()
    assert err <= tol, "%s: max|O-O_ref| = %.3g > %.3g" % (what, err, tol)
    if finite.any():
        lerr = np.abs(l[finite] - l_ref[finite]).max()
        assert lerr <= 1e-3, "%s: max|LSE-LSE_ref| = %.3g" % (what, lerr)
    return err, float(np.sqrt(np.mean((o - o_ref) ** 2)))


def record_parity(what, o, l, o_ref, l_ref):
    """Error figures of one compared output (max |O - O_ref| against the bar, RMSE of O against
    the float64 reference, max |LSE - LSE_ref| on finite rows), appended as one JSON line to the
    file named by MLA_PARITY_LOG when it is set.  Returns the figures."""
    finite = np.isfinite(l_ref)
    rec = {"what": what, "rows": int(l_ref.size),
           "max_abs_err": float(np.abs(o - o_ref).max()),
           "tol": float(1e-2 * np.abs(o_ref).max() + 2e-3),
           "rmse": float(np.sqrt(np.mean((o - o_ref) ** 2))),
           "rms_ref": float(np.sqrt(np.mean(o_ref ** 2))),
           "max_lse_err": float(np.abs(l[finite] - l_ref[finite]).max()) if finite.any() else 0.0}
    path = os.environ.get("MLA_PARITY_LOG")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec
