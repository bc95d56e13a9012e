"""Helpers for the GPU parity tests: upload a seeded problem, run it through the
C ABI, read C back, and compare with the oracle."""
import numpy as np

import gemm_inputs as gi
import oracle
from oracle import compare

# Sentinels written into C before a call: its padding must keep them.
SENTINEL = {"f32": np.uint32(0x7FC0DEAD), "f16": np.uint16(0x7E5A), "bf16": np.uint16(0x7FDA)}


def torch_mod():
    import torch
    return torch


def to_device(arr):
    torch = torch_mod()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def c_buffer(prob):
    """Device C storage (outer x ldc), filled with the sentinel."""
    torch = torch_mod()
    tout = prob["out_type"]
    outer = prob["N"] if prob["c_first"] else prob["M"]
    n = max(outer * prob["ldc"], 1)
    if tout == "f32":
        fill = int(np.array([SENTINEL["f32"]], np.uint32).view(np.int32)[0])
        return torch.full((n,), fill, dtype=torch.int32, device="cuda").view(torch.float32)
    fill = int(np.array([SENTINEL[tout]], np.uint16).view(np.int16)[0])
    return torch.full((n,), fill, dtype=torch.int16, device="cuda")


def host_c(c_dev, prob):
    """(logical M x N result, full flat storage) as numpy (float32 or uint16 bits)."""
    flat = c_dev.cpu().numpy()
    if prob["out_type"] != "f32":
        flat = flat.view(np.uint16)
    M, N = prob["M"], prob["N"]
    logical = gi.load(flat, M, N, prob["c_first"], prob["ldc"]) if M * N else \
        np.zeros((M, N), flat.dtype)
    return np.ascontiguousarray(logical), flat


def run(prob, config=None, stream=None, dev=None):
    """Run `prob` on the GPU; returns (logical C, flat C storage, status).
    `dev` reuses already uploaded (A, B) device tensors."""
    import dense_gemm_engineering_run_amd as g
    torch = torch_mod()
    if dev is None:
        dev = (to_device(prob["A"]), to_device(prob["B"]))
    a, b = dev
    c = c_buffer(prob)
    s = stream if stream is not None else torch.cuda.current_stream()
    args = (prob["M"], prob["N"], prob["K"], prob["a_major"], prob["b_major"], prob["c_major"],
            prob["dtype"], a.data_ptr(), b.data_ptr(), c.data_ptr(), prob["lda"], prob["ldb"],
            prob["ldc"], s.cuda_stream)
    need = 0 if config is None else g.gemm_workspace_size(
        prob["M"], prob["N"], prob["K"], prob["a_major"], prob["b_major"], prob["c_major"],
        prob["dtype"], config)
    if need:            # a stream-K config: zero-filled workspace of the size it asks for
        ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda")
        st = g.gemm_run_ws(*args[:-1], ws.data_ptr(), need, s.cuda_stream, config)
    elif config is None:
        st = g.gemm_run(*args)
    else:
        st = g.gemm_run_config(*args, config)
    s.synchronize()
    logical, flat = host_c(c, prob)
    return logical, flat, st


def reference(prob, rows=None, threads=None):
    return oracle.gemm_ref(prob["M"], prob["N"], prob["K"], prob["a_major"], prob["b_major"],
                           prob["in_type"], prob["A"], prob["lda"], prob["B"], prob["ldb"],
                           rows=rows, threads=threads)


def padding_intact(flat, prob):
    """True when every element of C's ld padding still holds the sentinel."""
    outer = prob["N"] if prob["c_first"] else prob["M"]
    inner = prob["M"] if prob["c_first"] else prob["N"]
    ld = prob["ldc"]
    if outer == 0 or ld == inner:
        return True
    pad = flat[: outer * ld].reshape(outer, ld)[:, inner:]
    s = SENTINEL[prob["out_type"]]
    if prob["out_type"] == "f32":
        return bool(np.all(pad.view(np.uint32) == s))
    return bool(np.all(pad == s))


def no_sentinel(c_logical, prob):
    """True when no element of the logical C still holds the sentinel that
    c_buffer() wrote (every element was stored)."""
    bits = np.asarray(c_logical)
    if prob["out_type"] == "f32":
        return not bool(np.any(bits.view(np.uint32) == SENTINEL["f32"]))
    return not bool(np.any(bits.view(np.uint16) == SENTINEL[prob["out_type"]]))


def check(c_logical, ref, prob, exact, rows=None):
    sub = c_logical if rows is None else c_logical[rows[0]:rows[1]]
    return compare.check(sub, ref, prob["out_type"], exact)
