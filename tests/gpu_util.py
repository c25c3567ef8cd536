"""Shared helpers of the GPU parity tests (comparison rule and tolerances).

Tolerance rule for floating-point outputs: max over elements of the error, divided by the
RMS of the oracle's values, must not exceed c, with c = 1e-4 for fp32 inputs and fp32
arithmetic and c = 2e-2 for bf16 inputs with fp32 state.

The error of an element is |gpu - oracle| for outputs stored in fp32.  For outputs stored in
bf16 it is the distance from the oracle's value to the set of reals that round to the stored
bf16 value: max(0, |gpu - oracle| - half_ulp_bf16(gpu)).  In words: the stored value must be
the bf16 rounding of some number within c * RMS of the oracle.  Storage rounding is not
counted against the computation because it cannot be avoided: on the B=4 H=16 T=4096
K=V=128 workload, rounding the exact fp64 oracle output to bf16 already moves the largest
elements by 2.8e-2 * RMS(o) (max|o| is 9.5 RMS there), so the plain rule would reject every
implementation that stores o in bf16, including a perfect one.

The camera-branch scan takes fp32 inputs but forms its products from fp16 operands (the
pages' own scan uses TF32 dots, whose mantissa is as wide): c = 1e-2 there.  Each product
term carries two operand roundings of relative size u = 2^-11, so an output's error is about
2u * RMS in standard deviation; 1e-2 is 5.5 of those standard deviations, doubled.

The camera-branch scan backward splits each fp32 operand into a bf16 pair x = hi + lo and
sums three products (hi*hi + hi*lo + lo*hi), so an operand carries a relative rounding of
about u = 2^-17 (plus the dropped lo*lo term, 2^-18): by the same count as above, 2u * RMS in
standard deviation, 5.5 of those doubled is 1.7e-4, rounded up to c = 2e-4.

Integer tables are compared bit for bit.
"""
import sys

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
FP16_OPERAND_TOL = 1e-2
SPLIT_OPERAND_TOL = 2e-4


def _np(x):
    return x.detach().to("cpu").double().numpy() if hasattr(x, "detach") else np.asarray(x)


def half_ulp_bf16(x):
    """Half the bf16 spacing at each (bf16-representable) value of x; 0 at zero."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def elem_err(got, ref):
    g = _np(got)
    ref = np.asarray(ref, np.float64)
    err = np.abs(g - ref)
    if hasattr(got, "dtype") and got.dtype == torch.bfloat16:
        err = np.maximum(err - half_ulp_bf16(g), 0.0)
    return err


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(elem_err(got, ref))) / max(rms, 1e-30), rms


def assert_close(name, got, ref, tol):
    err, rms = rel_err(got, ref)
    print("  %-10s max err/rms = %.3e (rms %.3e, tol %.0e)" % (name, err, rms, tol), flush=True)
    assert err <= tol, "%s: max err/rms = %.3e > %.0e" % (name, err, tol)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()
