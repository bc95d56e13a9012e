"""Acceptance test of a GEMM result against the oracle -- TEST INFRASTRUCTURE ONLY.

Criteria (stated in the GEMM engine's contract; the pages' own checks are the
SGEMM example's elementwise ``assert_close`` in ``run()`` and the CK Tile
README's ``check_err`` under "Result Verification"):

* integer-valued inputs: the result must equal the oracle rounded to the output
  type, bit for bit;
* otherwise: ||C - C_ref||_F / ||C_ref||_F <= 1e-5 for fp32 output and
  <= 8e-3 for fp16 / bf16 output, norms in fp64;
* a NaN or Inf in C where C_ref is finite fails.
"""
import numpy as np

from . import decode, round_to

TOL = {"f32": 1e-5, "f16": 8e-3, "bf16": 8e-3}


def as_f64(c, out_type):
    """fp64 values of a GPU result given as float32 or as uint16 bit patterns."""
    c = np.asarray(c)
    if out_type == "f32":
        return c.astype(np.float64)
    return decode(c.view(np.uint16), out_type)


def normwise_rel_err(c64, ref):
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt(np.sum(ref * ref))
    diff = np.asarray(c64, dtype=np.float64) - ref
    num = np.sqrt(np.sum(diff * diff))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def check(c, ref, out_type, exact):
    """Return (ok, info) for result ``c`` (float32, or uint16 bits) against
    fp64 ``ref`` of the same logical shape."""
    c = np.asarray(c)
    ref = np.asarray(ref, dtype=np.float64)
    c64 = as_f64(c, out_type)
    info = {"shape": tuple(ref.shape)}
    bad_nonfinite = int(np.sum(~np.isfinite(c64) & np.isfinite(ref)))
    info["nonfinite"] = bad_nonfinite
    if exact:
        want = round_to(ref, out_type)
        got = c.view(np.uint32) if out_type == "f32" else c.view(np.uint16)
        wantb = want.view(np.uint32) if out_type == "f32" else want.view(np.uint16)
        mism = int(np.sum(got != wantb))
        info["mismatches"] = mism
        if mism:
            idx = np.argwhere(got != wantb)[0]
            info["first_mismatch"] = (tuple(int(i) for i in idx), float(c64[tuple(idx)]),
                                      float(ref[tuple(idx)]))
        return mism == 0 and bad_nonfinite == 0, info
    err = normwise_rel_err(c64, ref)
    info["normwise_err"] = err
    info["tol"] = TOL[out_type]
    return err <= TOL[out_type] and bad_nonfinite == 0, info
