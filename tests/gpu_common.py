"""Helpers shared by the GPU tests: move seeded inputs to the device, run the HIP path
through the C ABI, run the oracle on the same inputs (optionally on a sample of
channels), and measure the normalised error the parity bar is stated in."""
import json
import os

import numpy as np

import oracle
import s6_workloads

# max |y_gpu - y_ref| / max |y_ref|, by I/O type (fp32 state in both cases)
TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_STATE = 1e-4


def torch():
    import torch as t
    return t


def dev(x, io):
    """numpy float32 -> torch GPU tensor in the I/O type (bf16 values are already exact)."""
    if x is None:
        return None
    t = torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch().bfloat16) if io == "bf16" else t


def run_gpu(inp, *, path="auto", chunk_len=0, want_last=True, stream=None, workspace=False, scalar_io=False):
    import selective_state_space_s6_amd as ss
    tc = torch()
    io = inp.io
    u = dev(inp.u, io)
    delta = dev(inp.delta, io)
    B = dev(inp.B, io)
    C = dev(inp.C, io)
    z = dev(inp.z, io)
    A = tc.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else tc.from_numpy(inp.Dskip).cuda()
    ws = None
    if workspace:
        need = ss.workspace_size(ss.make_dims(u, delta, A, B, C, z, u, path=path, chunk_len=chunk_len,
                                              scalar_io=scalar_io))
        ws = tc.empty(max(need, 1), dtype=tc.uint8, device="cuda")
    if stream is not None:
        tc.cuda.synchronize()            # inputs were prepared on the current stream
    y, last = ss.selective_scan_fwd(u, delta, A, B, C, Ds, z, return_last_state=want_last, path=path,
                                    chunk_len=chunk_len, stream=stream, workspace=ws, scalar_io=scalar_io)
    tc.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    last = None if last is None else last.cpu().numpy().astype(np.float64)
    return y, last


select_channels = s6_workloads.select_channels


def run_oracle(inp, want_last=True):
    return oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, time_invariant=inp.ti,
                      want_last=want_last)


def rel_err(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(a - ref))) / (scale if scale > 0 else 1.0)


def log_errors(case, **errs):
    """Append the measured errors to $SELSCAN_PARITY_LOG (JSON lines), if set."""
    path = os.environ.get("SELSCAN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(case=case, **errs)) + "\n")
