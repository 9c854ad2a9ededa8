"""The C-ABI library loads, exports every entry point include/selscan.h declares, its
struct layout matches the Python mirror, and argument errors are reported on the host
before anything is enqueued (no GPU needed: none of these calls reaches a HIP API)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import selective_state_space_s6_amd as ss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "selscan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+[\s\*]+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert "selective_scan_fwd" in names and "selective_scan_fwd_ws" in names
    assert len(names) >= 7


def test_every_declared_symbol_is_exported():
    lib = ss.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ss.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_struct_layout_matches_header():
    fields = [f for f, _ in ss.SelscanDims._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"selscan.h\"\nint main(void){printf(\"%zu\\n\", sizeof(selscan_dims));\n"
    for f in fields:
        src += 'printf("%%zu\\n", offsetof(selscan_dims, %s));\n' % f
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        vals = [int(x) for x in subprocess.check_output([exe]).split()]
    assert vals[0] == ctypes.sizeof(ss.SelscanDims)
    for f, off in zip(fields, vals[1:]):
        assert getattr(ss.SelscanDims, f).offset == off, f


def test_strerror_and_version():
    assert ss.abi_version() == ss.SELSCAN_ABI_VERSION
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert ss.strerror(st) and ss.strerror(st) != "unknown status"
    assert ss.strerror(12345) == "unknown status"
    assert ss.last_hip_error() == 0


def test_dims_init_contiguous():
    d = ss.dims_init(ss.SELSCAN_BF16, 4, 100, 24, 16)
    assert (d.u_sb, d.u_sl, d.delta_sb, d.delta_sl) == (2400, 24, 2400, 24)
    assert (d.B_sb, d.B_sl, d.B_sd) == (1600, 16, 0)
    t = ss.dims_init(ss.SELSCAN_F32, 4, 100, 24, 16, time_invariant=True)
    assert (t.delta_sb, t.delta_sl, t.B_sb, t.B_sl, t.B_sd, t.C_sd) == (0, 0, 0, 0, 16, 16)
    assert (d.discretization, d.delta_softplus, t.discretization, t.delta_softplus) == (0, 0, 0, 0)


FAKE = ctypes.c_void_p(0x100000)          # never dereferenced: every call below fails on the host
FAKE_ODD = ctypes.c_void_p(0x100002)


def call(dims, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, Dskip=None, z=None, y=FAKE, last=None):
    return ss.lib().selective_scan_fwd_ws(u, delta, A, B, C, Dskip, z, y, last, ctypes.byref(dims), None, 0, None)


def good_dims(**kw):
    d = ss.dims_init(ss.SELSCAN_F32, 2, 64, 8, 16)
    d.path = ss.PATHS["chunked"]
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_null_pointers():
    for arg in ("u", "delta", "A", "B", "C", "y"):
        assert call(good_dims(), **{arg: None}) == ss.SELSCAN_ERR_NULL
    assert ss.lib().selective_scan_fwd_ws(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None, None, 0,
                                          None) == ss.SELSCAN_ERR_NULL


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 99, ss.SELSCAN_ERR_ABI),
    ("dstate", 0, ss.SELSCAN_ERR_DIMS),
    ("dim", 0, ss.SELSCAN_ERR_DIMS),
    ("batch", -1, ss.SELSCAN_ERR_DIMS),
    ("seqlen", -5, ss.SELSCAN_ERR_DIMS),
    ("u_sl", -1, ss.SELSCAN_ERR_DIMS),
    ("dstate", 65, ss.SELSCAN_ERR_UNSUPPORTED),
    ("io_dtype", 7, ss.SELSCAN_ERR_UNSUPPORTED),
    ("path", 9, ss.SELSCAN_ERR_UNSUPPORTED),
    ("chunk_len", 24, ss.SELSCAN_ERR_UNSUPPORTED),
    ("discretization", 2, ss.SELSCAN_ERR_UNSUPPORTED),
    ("discretization", -1, ss.SELSCAN_ERR_UNSUPPORTED),
    ("B_sd", 16, ss.SELSCAN_ERR_UNSUPPORTED),      # B varying with both token and channel
    ("y_sl", 0, ss.SELSCAN_ERR_UNSUPPORTED),       # overlapping output rows
    ("y_sb", 8, ss.SELSCAN_ERR_UNSUPPORTED),
])
def test_dims_errors(field, value, status):
    assert call(good_dims(**{field: value})) == status
    assert ss.workspace_size(good_dims(**{field: value})) == 0


def test_time_invariant_needs_per_channel_delta():
    d = ss.dims_init(ss.SELSCAN_F32, 2, 64, 8, 16, time_invariant=True)
    d.delta_sl = 8                                   # per-token delta with per-channel B/C
    assert call(d) == ss.SELSCAN_ERR_UNSUPPORTED


def test_alignment():
    assert call(good_dims(), u=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    assert call(good_dims(), A=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    b = good_dims(io_dtype=ss.SELSCAN_BF16)
    assert call(b, u=ctypes.c_void_p(0x100001)) == ss.SELSCAN_ERR_ALIGN


def test_workspace_required_for_chunked_path():
    d = good_dims()
    need = ss.workspace_size(d)
    assert need > 0 and need % 256 == 0
    assert call(d) == ss.SELSCAN_ERR_WORKSPACE         # NULL workspace
    assert ss.lib().selective_scan_fwd_ws(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, ctypes.byref(d),
                                          FAKE, need - 1, None) == ss.SELSCAN_ERR_WORKSPACE
    s = ss.dims_init(ss.SELSCAN_F32, 2, 64, 8, 16)
    s.path = ss.PATHS["single"]
    assert ss.workspace_size(s) == 0


def test_auto_path_chunks_only_when_underfilled():
    small = ss.dims_init(ss.SELSCAN_F32, 2, 1024, 256, 16)        # 128 wavefronts: chunked
    assert ss.workspace_size(small) > 0
    big = ss.dims_init(ss.SELSCAN_BF16, 4, 16384, 2560, 16)       # 2560 wavefronts: one pass
    assert ss.workspace_size(big) == 0
    short = ss.dims_init(ss.SELSCAN_F32, 1, 64, 4, 4)             # too short to chunk
    assert ss.workspace_size(short) == 0


def test_empty_batch_is_a_no_op():
    d = good_dims(batch=0)
    assert call(d) == ss.SELSCAN_OK                    # nothing enqueued, no workspace needed


def call_ex(dims, h0=FAKE, ws=None, ws_bytes=0, bias=None):
    return ss.lib().selective_scan_fwd_ex(FAKE, FAKE, bias, FAKE, FAKE, FAKE, None, None, FAKE, h0, None,
                                          ctypes.byref(dims), ws, ws_bytes, None)


def test_initial_state_errors():
    ti = ss.dims_init(ss.SELSCAN_F32, 2, 64, 8, 16, time_invariant=True)
    assert call_ex(ti) == ss.SELSCAN_ERR_UNSUPPORTED           # time-invariant + initial state
    assert call_ex(good_dims(), h0=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    d = good_dims()                                            # chunked path, workspace too small
    assert call_ex(d, ws=FAKE, ws_bytes=ss.workspace_size(d) - 1) == ss.SELSCAN_ERR_WORKSPACE
    bad = good_dims(dstate=0)
    assert call_ex(bad) == ss.SELSCAN_ERR_DIMS


def call_step(dims, state=FAKE, bias=None):
    return ss.lib().selective_scan_step(FAKE, FAKE, bias, FAKE, FAKE, FAKE, None, None, FAKE, state,
                                        ctypes.byref(dims), None)


def test_step_errors():
    assert call_step(ss.dims_init(ss.SELSCAN_F32, 2, 2, 8, 16)) == ss.SELSCAN_ERR_DIMS    # seqlen != 1
    one = ss.dims_init(ss.SELSCAN_F32, 2, 1, 8, 16)
    assert call_step(one, state=None) == ss.SELSCAN_ERR_NULL
    assert call_step(one, state=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    assert call_step(ss.dims_init(ss.SELSCAN_F32, 2, 1, 8, 65)) == ss.SELSCAN_ERR_UNSUPPORTED
    assert call_step(ss.dims_init(ss.SELSCAN_F32, 0, 1, 8, 16)) == ss.SELSCAN_OK             # empty batch
    assert call_step(one, bias=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    bad = ss.dims_init(ss.SELSCAN_F32, 2, 1, 8, 16)
    bad.discretization = 5
    assert call_step(bad) == ss.SELSCAN_ERR_UNSUPPORTED


def test_step_size_options_errors():
    d = good_dims()
    assert call_ex(d, h0=None, ws=FAKE, ws_bytes=ss.workspace_size(d), bias=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    e = good_dims(discretization=ss.DISCRETIZATIONS["euler"], delta_softplus=1)
    assert call_ex(e, h0=None, ws=FAKE, ws_bytes=ss.workspace_size(e) - 1) == ss.SELSCAN_ERR_WORKSPACE


def call_bwd(dims, du=FAKE, ws=None, ws_bytes=0, dA=FAKE):
    return ss.lib().selective_scan_bwd(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                                       du, FAKE, None, dA, FAKE, FAKE, None, None, None, ctypes.byref(dims), ws,
                                       ws_bytes, None)


def test_backward_errors():
    d = ss.dims_init(ss.SELSCAN_F32, 2, 64, 40, 16)
    need = ss.bwd_workspace_size(d)
    # checkpoints (2 x 4 tiles x 40 x 16) and two partial sums (one 64-channel group x 2 x 64 x 16)
    assert need >= 4 * (2 * 4 * 40 * 16 + 2 * 1 * 2 * 64 * 16)
    ti = ss.dims_init(ss.SELSCAN_F32, 2, 64, 40, 16, time_invariant=True)
    need_ti = ss.bwd_workspace_size(ti)
    # fixed coefficients: checkpoints, and partial sums of dB, dC and dA per (batch row, chunk)
    assert need_ti >= 4 * (2 * 4 * 40 * 16 + 3 * 2 * 40 * 16)
    assert call_bwd(ti, ws=FAKE, ws_bytes=need_ti - 1) == ss.SELSCAN_ERR_WORKSPACE
    assert call_bwd(d, du=None, ws=FAKE, ws_bytes=need) == ss.SELSCAN_ERR_NULL
    assert call_bwd(d, dA=None, ws=FAKE, ws_bytes=need) == ss.SELSCAN_ERR_NULL
    assert call_bwd(d, du=FAKE_ODD, ws=FAKE, ws_bytes=need) == ss.SELSCAN_ERR_ALIGN
    assert call_bwd(d, ws=FAKE, ws_bytes=need - 1) == ss.SELSCAN_ERR_WORKSPACE
    assert call_bwd(good_dims(abi_version=3), ws=FAKE, ws_bytes=need) == ss.SELSCAN_ERR_ABI
    assert ss.bwd_workspace_size(ss.dims_init(ss.SELSCAN_F32, 0, 64, 40, 16)) == 0


def test_ssd_errors():
    d = ss.ssd_dims(2, 200, 3, 64, 128)
    need = ss.ssd_workspace_size(d)
    assert need >= 4 * 2 * 3 * 4 * 128 * 64                 # one fp32 state per (b, h, chunk)
    call = lambda dd, x=FAKE, ws=FAKE, nb=need: ss.lib().selective_scan_ssd_fwd(
        x, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None, ctypes.byref(dd), ws, nb, None)
    assert call(ss.ssd_dims(2, 200, 3, 32, 128)) == ss.SELSCAN_ERR_UNSUPPORTED     # head dimension
    assert call(ss.ssd_dims(2, 200, 3, 64, 96)) == ss.SELSCAN_ERR_UNSUPPORTED      # state size
    assert call(ss.ssd_dims(2, 200, 0, 64, 64)) == ss.SELSCAN_ERR_DIMS
    assert call(d, x=None) == ss.SELSCAN_ERR_NULL
    assert call(d, x=ctypes.c_void_p(0x100001)) == ss.SELSCAN_ERR_ALIGN
    assert call(d, x=ctypes.c_void_p(0x100008)) == ss.SELSCAN_ERR_ALIGN             # 16 bytes needed
    assert call(d, nb=need - 1) == ss.SELSCAN_ERR_WORKSPACE
    bad = ss.ssd_dims(2, 200, 3, 64, 128)
    bad.abi_version = 1
    assert call(bad) == ss.SELSCAN_ERR_ABI
    assert ss.ssd_workspace_size(ss.ssd_dims(0, 200, 3, 64, 128)) == 0
    assert ss.ssd_workspace_size(ss.ssd_dims(2, 200, 3, 64, 128, path="fused")) == 0     # state on chip
    assert ss.ssd_workspace_size(ss.ssd_dims(4, 200, 80, 64, 128)) == 0                  # automatic: on chip
    assert ss.ssd_workspace_size(ss.ssd_dims(8, 200, 24, 64, 128)) == 0                  # automatic: on chip
    assert ss.ssd_workspace_size(ss.ssd_dims(2, 200, 24, 64, 128)) > 0                   # automatic: chunks
    assert ss.ssd_workspace_size(ss.ssd_dims(2, 200, 3, 64, 128, path="chunked")) == need
    bad_path = ss.ssd_dims(2, 200, 3, 64, 128)
    bad_path.path = 4
    assert call(bad_path) == ss.SELSCAN_ERR_UNSUPPORTED
    # segments: only with the segmented path, never negative
    assert call(ss.ssd_dims(2, 200, 3, 64, 128, path="fused", segments=2)) == ss.SELSCAN_ERR_UNSUPPORTED
    assert call(ss.ssd_dims(2, 200, 3, 64, 128, path="segmented", segments=-1)) == ss.SELSCAN_ERR_UNSUPPORTED
    # segmented: one fp32 state and one decay per (batch row, head, segment); 200 tokens are
    # 4 chunks, so 3 segments are runs of 2, 2 (two segments) and 100 are 4 segments of one chunk
    seg_ws = lambda k: ss.ssd_workspace_size(ss.ssd_dims(2, 200, 3, 64, 128, path="segmented", segments=k))
    rnd = lambda v: (v + 255) // 256 * 256
    assert seg_ws(1) == 0
    assert seg_ws(3) == rnd(6 * 2 * 128 * 64 * 4) + rnd(6 * 2 * 4)
    assert seg_ws(100) == rnd(6 * 4 * 128 * 64 * 4) + rnd(6 * 4 * 4)


def test_ssd_struct_layout_matches_header():
    fields = [f for f, _ in ss.SsdDims._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"selscan.h\"\nint main(void){printf(\"%zu\\n\", sizeof(selscan_ssd_dims));\n"
    for f in fields:
        src += 'printf("%%zu\\n", offsetof(selscan_ssd_dims, %s));\n' % f
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        vals = [int(v) for v in subprocess.check_output([exe]).split()]
    assert vals[0] == ctypes.sizeof(ss.SsdDims)
    for f, off in zip(fields, vals[1:]):
        assert getattr(ss.SsdDims, f).offset == off, f


def test_binding_rejects_a_short_dskip_before_any_launch(monkeypatch):
    """Every kernel reads Dskip[d] for all D channels: a Dskip of the wrong length (or not on
    the GPU) is refused by the binding before the library is touched."""
    import torch

    def no_library():
        raise AssertionError("the library was reached")

    monkeypatch.setattr(ss, "lib", no_library)
    batch, L, D, N = 2, 8, 4, 3
    u = torch.zeros(batch, L, D)
    A = -torch.ones(D, N)
    B = torch.zeros(batch, L, N)
    for bad in (torch.ones(D - 1), torch.ones(D + 1), torch.ones(D, 1), torch.ones(D)):   # the last: on the host
        with pytest.raises(ValueError, match="Dskip"):
            ss.selective_scan_fwd(u, u, A, B, B, bad)
        with pytest.raises(ValueError, match="Dskip"):
            ss.selective_scan_bwd(u, u, A, B, B, bad, dy=u)
        with pytest.raises(ValueError, match="Dskip"):
            ss.selective_scan_step(u[:, 0], u[:, 0], A, B[:, 0], B[:, 0], bad, state=torch.zeros(batch, D, N))


def call_noalloc(dims, u=FAKE, h0=None, bias=None):
    return ss.lib().selective_scan_fwd_noalloc(u, FAKE, bias, FAKE, FAKE, FAKE, None, None, FAKE, h0, None,
                                               ctypes.byref(dims), None)


def test_noalloc_errors_before_the_device():
    """The no-allocation forward refuses, on the host, a call whose chunked path needs more
    scratch than its per-GPU array holds, and argument errors, before touching a GPU."""
    big = ss.dims_init(ss.SELSCAN_F32, 64, 4096, 4096, 64)
    big.path = ss.PATHS["chunked"]
    big.chunk_len = 64
    assert ss.workspace_size(big) > ss.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(big) == ss.SELSCAN_ERR_SCRATCH_LIMIT
    assert "scratch" in ss.strerror(ss.SELSCAN_ERR_SCRATCH_LIMIT)
    assert call_noalloc(good_dims(), u=None) == ss.SELSCAN_ERR_NULL
    assert call_noalloc(good_dims(), u=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    assert call_noalloc(good_dims(dstate=0)) == ss.SELSCAN_ERR_DIMS
    ti = ss.dims_init(ss.SELSCAN_F32, 2, 64, 8, 16, time_invariant=True)
    ti.path = ss.PATHS["chunked"]
    assert call_noalloc(ti, h0=FAKE) == ss.SELSCAN_ERR_UNSUPPORTED
    assert call_noalloc(good_dims(), h0=FAKE_ODD) == ss.SELSCAN_ERR_ALIGN
    assert call_noalloc(good_dims(batch=0)) == ss.SELSCAN_OK     # nothing to do, nothing touched


def test_plan_path_resolves_the_automatic_choice():
    small = ss.dims_init(ss.SELSCAN_F32, 2, 1024, 256, 16)               # 128 wavefronts: chunked
    assert ss.plan_path(small) == "chunked"
    big = ss.dims_init(ss.SELSCAN_BF16, 4, 16384, 2560, 16)              # one pass
    assert ss.plan_path(big) == "single"
    ti = ss.dims_init(ss.SELSCAN_F32, 4, 8192, 1024, 64, time_invariant=True)   # fixed coefficients: convolution
    assert ss.plan_path(ti) == "conv" and ss.workspace_size(ti) == 0
    few = ss.dims_init(ss.SELSCAN_F32, 1, 8192, 64, 64, time_invariant=True)    # too few channels: recurrence
    assert ss.plan_path(few) in ("single", "chunked")
    odd = ss.dims_init(ss.SELSCAN_F32, 4, 8192, 1022, 64, time_invariant=True)  # D % 4 != 0: recurrence
    assert ss.plan_path(odd) in ("single", "chunked")
    odd.path = ss.PATHS["conv"]
    assert call(odd) == ss.SELSCAN_ERR_UNSUPPORTED
    sel = ss.dims_init(ss.SELSCAN_F32, 4, 8192, 1024, 16)                # selective: no convolution
    sel.path = ss.PATHS["conv"]
    assert call(sel) == ss.SELSCAN_ERR_UNSUPPORTED
    bad = ss.dims_init(ss.SELSCAN_F32, 4, 8192, 1024, 65)
    assert lib_status(bad) == ss.SELSCAN_ERR_UNSUPPORTED


def lib_status(dims):
    return ss.lib().selective_scan_plan_path(ctypes.byref(dims))
