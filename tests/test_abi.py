"""The C ABI of libmsel.so on the CPU: symbols, struct layout and host-side validation.

Nothing here launches a kernel: only the msel_validate_* checks and entry points called with
invalid arguments (which return before any HIP call) are exercised, with fake device
addresses that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

from selective_state_space_26_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msel.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(msel_\w+)\s*\(", text))
    assert declared == set(_lib.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (msel_\w+)$", nm, re.M))
    assert declared <= exported
    for name in declared:
        assert hasattr(lib, name)


def test_checked_build_exports_the_same_functions(lib):
    """The checked twin (every kernel index range-checked) exports every declared function;
    msel_checked_build tells the two apart; the release build's self-test refuses without
    enqueuing anything, and the violation reader checks its pointers before any HIP call."""
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(msel_\w+)\s*\(", text))
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_CHECKED_PATH],
                        capture_output=True, text=True, check=True).stdout
    assert declared <= set(re.findall(r" T (msel_\w+)$", nm, re.M))
    chk = _lib.load(_lib.LIB_CHECKED_PATH)
    assert chk.msel_checked_build() == 1
    assert lib.msel_checked_build() == 0
    assert lib.msel_bounds_selftest(None) == 5  # MSEL_ERR_UNSUPPORTED
    n, f = ctypes.c_ulonglong(7), ctypes.c_uint32(7)
    assert lib.msel_bound_violations(ctypes.byref(n), ctypes.byref(f), None) == 1  # NULL
    assert chk.msel_bound_violations(None, ctypes.byref(f), ctypes.byref(f)) == 1


def test_binding_switches_to_the_checked_build():
    import selective_state_space_26_amd as msel
    assert not msel.checked_build()
    with _lib.using(_lib.LIB_CHECKED_PATH):
        assert msel.checked_build()
    assert not msel.checked_build()


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "msel.h"\n'
        "#define F(S, m) printf(#S \".\" #m \" %zu\\n\", offsetof(S, m));\n"
        "int main(void) {\n"
        'printf("args %zu\\ngrads %zu\\n", sizeof(msel_scan_args), sizeof(msel_scan_grads));\n'
        'printf("cargs %zu\\ncgrads %zu\\n", sizeof(msel_conv_args), sizeof(msel_conv_grads));\n'
        'printf("targs %zu\\n", sizeof(msel_trap_args));\n'
        + "".join(f"F(msel_scan_args, {f})\n" for f, _ in _lib.ScanArgs._fields_)
        + "".join(f"F(msel_scan_grads, {f})\n" for f, _ in _lib.ScanGrads._fields_)
        + "".join(f"F(msel_conv_args, {f})\n" for f, _ in _lib.ConvArgs._fields_)
        + "".join(f"F(msel_conv_grads, {f})\n" for f, _ in _lib.ConvGrads._fields_)
        + "".join(f"F(msel_trap_args, {f.rstrip('_')})\n" for f, _ in _lib.TrapArgs._fields_)
        + "".join(f"F(msel_trap_grads, {f})\n" for f, _ in _lib.TrapGrads._fields_)
        + "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    assert int(got["args"]) == ctypes.sizeof(_lib.ScanArgs)
    assert int(got["grads"]) == ctypes.sizeof(_lib.ScanGrads)
    for f, _ in _lib.ScanArgs._fields_:
        assert int(got[f"msel_scan_args.{f}"]) == getattr(_lib.ScanArgs, f).offset, f
    for f, _ in _lib.ScanGrads._fields_:
        assert int(got[f"msel_scan_grads.{f}"]) == getattr(_lib.ScanGrads, f).offset, f
    assert int(got["cargs"]) == ctypes.sizeof(_lib.ConvArgs)
    assert int(got["cgrads"]) == ctypes.sizeof(_lib.ConvGrads)
    for f, _ in _lib.ConvArgs._fields_:
        assert int(got[f"msel_conv_args.{f}"]) == getattr(_lib.ConvArgs, f).offset, f
    for f, _ in _lib.ConvGrads._fields_:
        assert int(got[f"msel_conv_grads.{f}"]) == getattr(_lib.ConvGrads, f).offset, f
    assert int(got["targs"]) == ctypes.sizeof(_lib.TrapArgs)
    for f, _ in _lib.TrapArgs._fields_:
        assert int(got[f"msel_trap_args.{f.rstrip('_')}"]) == getattr(_lib.TrapArgs, f).offset, f
    for f, _ in _lib.TrapGrads._fields_:
        assert int(got[f"msel_trap_grads.{f}"]) == getattr(_lib.TrapGrads, f).offset, f


def test_constants(lib):
    assert lib.msel_abi_version() == 1
    T = lib.msel_chunk_len()
    assert T > 0 and T % 64 == 0
    assert lib.msel_num_chunks(0) == 0
    assert lib.msel_num_chunks(1) == 1
    assert lib.msel_num_chunks(T) == 1
    assert lib.msel_num_chunks(T + 1) == 2
    assert lib.msel_num_chunks(65536) == -(-65536 // T)
    for code, name in _lib.STATUS.items():
        assert lib.msel_status_string(code).decode().startswith(name)
    assert lib.msel_status_string(1234).decode() == "MSEL_ERR_UNKNOWN"


_fake = iter(range(0x10000000, 0x7fffffff, 0x100000))


def _addr():
    return next(_fake)


def _good_args(bsz=2, dim=3, N=16, L=100, dtype=0):
    a = _lib.ScanArgs()
    a.abi_version = 1
    a.batch, a.dim, a.dstate, a.seqlen = bsz, dim, N, L
    a.dtype, a.delta_softplus, a.reserved = dtype, 1, 0
    for f in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias", "out", "final_state"):
        setattr(a, f, _addr())
    return a


def _good_grads(a):
    g = _lib.ScanGrads()
    for f in ("dout", "du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        setattr(g, f, _addr())
    return g


def _fwd(lib, a):
    return lib.msel_validate_fwd(ctypes.byref(a))


def test_valid_args_pass_validation(lib):
    a = _good_args()
    assert _fwd(lib, a) == 0
    a.chunk_states = _addr()
    assert lib.msel_validate_chunk_carry(ctypes.byref(a)) == 0
    g = _good_grads(a)
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), _addr(), 1 << 20) == 0


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 2, 9), ("reserved", 1, 9),
    ("batch", 0, 2), ("dim", 0, 2), ("dstate", 0, 2), ("seqlen", 0, 2), ("seqlen", -5, 2),
    ("dtype", 2, 3), ("dtype", -1, 3), ("delta_softplus", 2, 3),
    ("dstate", 17, 5), ("dstate", 64, 5),
    ("u", None, 1), ("delta", None, 1), ("B", None, 1), ("A", None, 1), ("C", None, 1),
    ("out", None, 1),
])
def test_fwd_rejects(lib, field, value, code):
    a = _good_args()
    setattr(a, field, value)
    assert _fwd(lib, a) == code
    # the entry point itself rejects the same way, before any HIP call
    assert lib.msel_scan_fwd(ctypes.byref(a), None) == code


def test_null_args_pointer(lib):
    assert lib.msel_validate_fwd(None) == 1
    assert lib.msel_scan_fwd(None, None) == 1
    assert lib.msel_scan_chunk_carry(None, None) == 1
    assert lib.msel_scan_bwd(None, None, None, 0, None) == 1
    assert lib.msel_scan_bwd_profiled(None, None, None, 0, None, None, None) == 1
    assert lib.msel_scan_bwd_workspace_bytes(None) == 0


def test_size_overflow_is_rejected(lib):
    a = _good_args()
    a.batch, a.dim = 1 << 16, 1 << 15
    assert _fwd(lib, a) == 2
    a = _good_args()
    a.seqlen = (1 << 30) + 1
    assert _fwd(lib, a) == 2
    a.seqlen = (1 << 28) + 1  # byte offsets of an fp32 row must stay below 2^31
    assert _fwd(lib, a) == 2
    a.seqlen = 1 << 28
    assert _fwd(lib, a) == 0


@pytest.mark.parametrize("field", ["u", "delta", "B", "C", "z", "out"])
def test_activation_alignment(lib, field):
    a = _good_args()
    setattr(a, field, getattr(a, field) + 8)
    assert _fwd(lib, a) == 4


@pytest.mark.parametrize("field", ["A", "D", "delta_bias", "final_state"])
def test_fp32_alignment(lib, field):
    a = _good_args()
    setattr(a, field, getattr(a, field) + 2)
    assert _fwd(lib, a) == 4


@pytest.mark.parametrize("out_field,in_field", [("out", "u"), ("out", "z"), ("final_state", "A"),
                                                ("chunk_states", "delta"), ("chunk_states", "h0"),
                                                ("out", "final_state"),
                                                ("chunk_states", "final_state")])
def test_aliasing_is_rejected(lib, out_field, in_field):
    a = _good_args()
    a.h0, a.chunk_states = _addr(), _addr()
    assert _fwd(lib, a) == 0
    setattr(a, out_field, getattr(a, in_field))
    assert _fwd(lib, a) == 7


def test_final_state_may_update_h0_in_place(lib):
    a = _good_args()
    a.h0 = _addr()
    a.final_state = a.h0
    assert _fwd(lib, a) == 0
    a.chunk_states = _addr()
    assert lib.msel_validate_chunk_carry(ctypes.byref(a)) == 0


def test_optional_inputs_may_be_null(lib):
    a = _good_args()
    a.z = a.D = a.delta_bias = a.h0 = a.final_state = a.chunk_states = None
    assert _fwd(lib, a) == 0


def test_chunk_carry_rules(lib):
    a = _good_args()
    a.C = None
    assert lib.msel_validate_chunk_carry(ctypes.byref(a)) == 1  # chunk_states missing
    a.chunk_states = _addr()
    assert lib.msel_validate_chunk_carry(ctypes.byref(a)) == 0  # C not needed
    a.chunk_states = a.u
    assert lib.msel_scan_chunk_carry(ctypes.byref(a), None) == 7


def test_bwd_workspace_rules(lib):
    a = _good_args(bsz=2, dim=3, N=16, L=1000)
    g = _good_grads(a)
    T = lib.msel_chunk_len()
    nch = -(-1000 // T)
    up = lambda x: (x + 255) // 256 * 256
    states, per_chunk = 2 * 3 * nch * 16 * 4, 2 * 3 * nch * 4
    need = lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a))
    assert need == 2 * up(states) + 2 * up(per_chunk)
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), None, 0) == 6
    ws = _addr()
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), ws, need - 1) == 6
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), ws, need) == 0
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), ws + 16, need) == 4
    assert lib.msel_scan_bwd(ctypes.byref(a), ctypes.byref(g), None, 0, None) == 6
    assert lib.msel_scan_bwd_profiled(ctypes.byref(a), ctypes.byref(g), None, 0, None, None,
                                      None) == 6
    # with caller-provided chunk states the workspace only holds the adjoint carries
    a.chunk_states = _addr()
    need2 = lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a))
    assert need2 == up(states) + 2 * up(per_chunk)
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), ws, need2) == 0
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), a.chunk_states, need2) == 7


def test_bwd_plan_choice(lib):
    """The fused plan: chunk states given, at most 4 chunks and a grid of at least 128
    workgroups by default; its workspace holds the partial sums (a pure function of the
    sizes); the setting forces or forbids it; the rebuilt-state backward never takes it."""
    T = lib.msel_chunk_len()
    up = lambda x: (x + 255) // 256 * 256

    def plan(bsz, dim, N, L, given=True):
        a = _good_args(bsz=bsz, dim=dim, N=N, L=L, dtype=1)
        if given:
            a.chunk_states = _addr()
        return lib.msel_scan_bwd_fused(ctypes.byref(a)), lib.msel_scan_bwd_workspace_bytes(
            ctypes.byref(a))

    try:
        fused, need = plan(8, 1536, 16, 2048)  # 32 channel groups per batch row
        assert fused == 1
        nch, cg = 2048 // T, 32
        assert need == (up(8 * 1536 * 16 * 4) + up(8 * cg * nch * 2 * 16 * T * 4) +
                        up(8 * nch * 1536 * 16 * 4) + 2 * up(8 * 1536 * nch * 4))
        assert need > 64 << 20  # beyond the no-allocation scratch: that call stays chunk-parallel
        assert plan(8, 1536, 16, 2048, given=False)[0] == 0  # rebuilt states
        assert plan(1, 5120, 16, 65536)[0] == 0  # 128 chunks
        assert plan(2, 3, 16, 1000)[0] == 0  # a grid of 2 workgroups
        small = plan(2, 3, 16, 1000)[1]
        lib.msel_set_bwd_fused(1)
        fused, need = plan(2, 3, 16, 1000)
        assert fused == 1 and need >= small
        assert plan(1, 5120, 16, 65536)[0] == 1
        assert plan(2, 3, 16, 1000, given=False)[0] == 0
        lib.msel_set_bwd_fused(-1)
        assert plan(8, 1536, 16, 2048) == (0, up(8 * 1536 * 4 * 16 * 4) + 2 * up(8 * 1536 * 4 * 4))
    finally:
        lib.msel_set_bwd_fused(0)
    assert plan(8, 1536, 16, 2048)[0] == 1


def test_bwd_noalloc_checks_before_any_launch(lib):
    """msel_scan_bwd_noalloc refuses bad arguments, and a problem whose workspace would exceed
    its static scratch, on the host (these calls make no HIP call)."""
    a = _good_args(bsz=1, dim=4096, N=16, L=65536)  # rebuilt states: 2 x 33.5 MB + 2 x 2 MB
    g = _good_grads(a)
    need = lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert lib.msel_scan_bwd_noalloc(ctypes.byref(a), ctypes.byref(g), None) == 10
    # with the forward's chunk states the same problem fits (the states are not rebuilt)
    a.chunk_states = _addr()
    assert lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a)) <= _lib.NOALLOC_SCRATCH_BYTES
    g.du = None
    assert lib.msel_scan_bwd_noalloc(ctypes.byref(a), ctypes.byref(g), None) == 1
    g.du = g.dout
    assert lib.msel_scan_bwd_noalloc(ctypes.byref(a), ctypes.byref(g), None) == 7
    a.seqlen = 0
    assert lib.msel_scan_bwd_noalloc(ctypes.byref(a), ctypes.byref(g), None) == 2
    assert lib.msel_scan_bwd_noalloc(None, ctypes.byref(g), None) == 1
    text = open(HEADER).read()
    assert "#define MSEL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text


@pytest.mark.parametrize("field,code", [("dout", 1), ("du", 1), ("ddelta", 1), ("dz", 1)])
def test_bwd_required_grads(lib, field, code):
    a = _good_args()
    a.chunk_states = _addr()
    g = _good_grads(a)
    setattr(g, field, None)
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), _addr(), 1 << 20) == code


def test_bwd_dz_optional_without_gate(lib):
    a = _good_args()
    a.chunk_states = _addr()
    a.z = None
    g = _good_grads(a)
    g.dz = None
    assert lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), _addr(), 1 << 20) == 0


def test_bwd_alias_and_alignment(lib):
    a = _good_args()
    a.chunk_states = _addr()
    ws, big = _addr(), 1 << 20
    check = lambda g: lib.msel_validate_bwd(ctypes.byref(a), ctypes.byref(g), ws, big)
    g = _good_grads(a)
    g.du = a.u
    assert check(g) == 7
    g = _good_grads(a)
    g.ddelta = g.dout
    assert check(g) == 7
    g = _good_grads(a)
    g.dB = ws
    assert check(g) == 7
    g = _good_grads(a)
    g.dz = g.dz + 4
    assert check(g) == 4
    g = _good_grads(a)
    g.dB = g.dB + 1
    assert check(g) == 4


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    from selective_state_space_26_amd import msel_scan_fwd
    x = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        msel_scan_fwd(x, x, torch.zeros(2, 4), torch.zeros(1, 4, 8), torch.zeros(1, 4, 8))


# ---- the short causal convolution --------------------------------------------------------

def _conv_args(bsz=2, dim=3, L=100, W=4, dtype=0):
    a = _lib.ConvArgs()
    a.abi_version = 1
    a.batch, a.dim, a.seqlen, a.width = bsz, dim, L, W
    a.dtype, a.activation, a.reserved = dtype, 1, 0
    for f in ("x", "weight", "bias", "state_in", "out", "state_out"):
        setattr(a, f, _addr())
    return a


def _conv_grads():
    g = _lib.ConvGrads()
    for f in ("dout", "dx", "dweight", "dbias", "dstate_in"):
        setattr(g, f, _addr())
    return g


def _cfwd(lib, a):
    return lib.msel_validate_conv_fwd(ctypes.byref(a))


def _cbwd(lib, a, g):
    return lib.msel_validate_conv_bwd(ctypes.byref(a), ctypes.byref(g))


def test_conv_valid_args_pass(lib):
    a = _conv_args()
    assert _cfwd(lib, a) == 0
    assert _cbwd(lib, a, _conv_grads()) == 0
    a.bias = a.state_in = a.state_out = None
    assert _cfwd(lib, a) == 0
    g = _conv_grads()
    g.dweight = g.dbias = g.dstate_in = None
    assert _cbwd(lib, a, g) == 0


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 2, 9), ("reserved", 3, 9),
    ("batch", 0, 2), ("dim", 0, 2), ("seqlen", 0, 2), ("width", 0, 2), ("width", -1, 2),
    ("seqlen", (1 << 28) + 1, 2),
    ("dtype", 2, 3), ("activation", 2, 3), ("activation", -1, 3),
    ("width", 5, 5), ("width", 64, 5),
    ("x", None, 1), ("weight", None, 1), ("out", None, 1),
])
def test_conv_fwd_rejects(lib, field, value, code):
    a = _conv_args()
    setattr(a, field, value)
    assert _cfwd(lib, a) == code
    assert lib.msel_conv1d_fwd(ctypes.byref(a), None) == code


def test_conv_null_pointers(lib):
    assert lib.msel_validate_conv_fwd(None) == 1
    assert lib.msel_conv1d_fwd(None, None) == 1
    assert lib.msel_conv1d_bwd(None, None, None) == 1
    a = _conv_args()
    assert lib.msel_validate_conv_bwd(ctypes.byref(a), None) == 1
    for f in ("dout", "dx"):
        g = _conv_grads()
        setattr(g, f, None)
        assert _cbwd(lib, a, g) == 1
        assert lib.msel_conv1d_bwd(ctypes.byref(a), ctypes.byref(g), None) == 1


def test_conv_alignment(lib):
    for f in ("x", "out"):
        a = _conv_args()
        setattr(a, f, getattr(a, f) + 8)
        assert _cfwd(lib, a) == 4
    for f, off in (("weight", 2), ("bias", 2), ("state_in", 2), ("state_out", 2)):
        a = _conv_args()
        setattr(a, f, getattr(a, f) + off)
        assert _cfwd(lib, a) == 4, f
    # bf16 states need 2-byte alignment only
    a = _conv_args(dtype=1)
    a.state_in += 2
    a.state_out += 6
    assert _cfwd(lib, a) == 0
    a.state_in += 1
    assert _cfwd(lib, a) == 4
    for f in ("dout", "dx"):
        a, g = _conv_args(), _conv_grads()
        setattr(g, f, getattr(g, f) + 4)
        assert _cbwd(lib, a, g) == 4
    for f in ("dweight", "dbias", "dstate_in"):
        a, g = _conv_args(), _conv_grads()
        setattr(g, f, getattr(g, f) + 2)
        assert _cbwd(lib, a, g) == 4


def test_conv_width_one_ignores_state_pointers(lib):
    a = _conv_args(W=1)
    a.state_in = a.x + 1      # misaligned, but there is no state of width 1
    a.state_out = a.x
    assert _cfwd(lib, a) == 0
    g = _conv_grads()
    g.dstate_in = g.dx
    assert _cbwd(lib, a, g) == 0


@pytest.mark.parametrize("out_field,in_field", [("out", "x"), ("out", "state_in"),
                                                ("out", "bias"), ("state_out", "x"),
                                                ("state_out", "weight"), ("state_out", "out")])
def test_conv_fwd_aliasing_is_rejected(lib, out_field, in_field):
    a = _conv_args()
    setattr(a, out_field, getattr(a, in_field))
    assert _cfwd(lib, a) == 7


def test_conv_state_may_update_in_place(lib):
    a = _conv_args(L=1)
    a.state_out = a.state_in
    assert _cfwd(lib, a) == 0
    a = _conv_args(L=1000)
    a.state_out = a.state_in
    assert _cfwd(lib, a) == 0


@pytest.mark.parametrize("gfield,target", [("dx", "x"), ("dx", "dout"), ("dweight", "weight"),
                                           ("dbias", "bias"), ("dstate_in", "state_in"),
                                           ("dbias", "dweight"), ("dstate_in", "dx")])
def test_conv_bwd_aliasing_is_rejected(lib, gfield, target):
    a, g = _conv_args(), _conv_grads()
    src = getattr(g, target) if hasattr(g, target) and target in dict(g._fields_) else \
        getattr(a, target)
    setattr(g, gfield, src)
    assert _cbwd(lib, a, g) == 7


# ---- the exponential-trapezoidal variant ------------------------------------------------

def _trap():
    t = _lib.TrapArgs()
    t.lambda_, t.u_prev, t.B_prev = _addr(), _addr(), _addr()
    return t


def test_trap_validation(lib):
    a, t = _good_args(), _trap()
    v = lambda: lib.msel_validate_trap_fwd(ctypes.byref(a), ctypes.byref(t))
    assert v() == 0
    t.u_prev = t.B_prev = None
    assert v() == 0
    assert lib.msel_validate_trap_fwd(ctypes.byref(a), None) == 1
    assert lib.msel_scan_trap_fwd(ctypes.byref(a), None, None) == 1
    t.lambda_ = None
    assert v() == 1
    assert lib.msel_scan_trap_fwd(ctypes.byref(a), ctypes.byref(t), None) == 1
    t.lambda_ = _addr() + 8
    assert v() == 4
    t = _trap()
    t.u_prev += 2              # fp32 inputs need 4-byte alignment
    assert v() == 4
    a.dtype = 1                # bf16: 2 bytes
    assert v() == 0
    t.B_prev += 1
    assert v() == 4
    # the checks of the plain forward apply too
    a, t = _good_args(), _trap()
    a.dstate = 17
    assert v() == 5
    a, t = _good_args(), _trap()
    a.out = a.u
    assert v() == 7


@pytest.mark.parametrize("out_field,in_field", [("out", "lambda_"), ("final_state", "u_prev"),
                                                ("out", "B_prev")])
def test_trap_outputs_must_not_alias_its_inputs(lib, out_field, in_field):
    a, t = _good_args(), _trap()
    a.chunk_states = _addr()
    setattr(a, out_field, getattr(t, in_field))
    assert lib.msel_validate_trap_fwd(ctypes.byref(a), ctypes.byref(t)) == 7


# ---- the complex-valued (rotational) variant ---------------------------------------------

def test_complex_validation(lib):
    a = _good_args(N=16)
    assert lib.msel_validate_complex_fwd(ctypes.byref(a)) == 0
    for n in (1, 3, 15):
        a.dstate = n
        assert lib.msel_validate_complex_fwd(ctypes.byref(a)) == 2
        assert lib.msel_scan_complex_fwd(ctypes.byref(a), None) == 2
        assert lib.msel_validate_fwd(ctypes.byref(a)) == 0   # the real scan takes any dstate
    a = _good_args(N=16)
    a.out = a.B
    assert lib.msel_validate_complex_fwd(ctypes.byref(a)) == 7
    assert lib.msel_validate_complex_fwd(None) == 1
    assert lib.msel_scan_complex_fwd(None, None) == 1


def _trap_grads():
    t = _lib.TrapGrads()
    t.dlambda, t.du_prev, t.dB_prev = _addr(), _addr(), _addr()
    return t


def test_trap_bwd_validation(lib):
    a, t = _good_args(L=1000), _trap()
    g, tg = _good_grads(a), _trap_grads()
    a.chunk_states = _addr()
    ws, big = _addr(), 1 << 20
    v = lambda: lib.msel_validate_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g),
                                           ctypes.byref(tg), ws, big)
    assert v() == 0
    tg.du_prev = tg.dB_prev = None
    assert v() == 0
    # without the forward's chunk states they are rebuilt: the workspace must hold them too
    a.chunk_states = None
    need = lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a))
    assert lib.msel_validate_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g),
                                      ctypes.byref(tg), ws, need) == 0
    assert lib.msel_validate_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g),
                                      ctypes.byref(tg), ws, need - 1) == 6
    assert lib.msel_scan_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g),
                                  ctypes.byref(tg), ws, need - 1, None) == 6
    a.chunk_states = _addr()
    assert lib.msel_validate_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g), None,
                                      ws, big) == 1
    tg = _trap_grads()
    tg.dlambda = None
    assert v() == 1
    tg = _trap_grads()
    tg.dlambda += 8
    assert v() == 4
    tg = _trap_grads()
    tg.du_prev += 2
    assert v() == 4
    for target in (a.u, g.du, t.lambda_, ws, a.chunk_states):
        tg = _trap_grads()
        tg.dlambda = target
        assert v() == 7
    tg = _trap_grads()
    tg.dB_prev = g.dB
    assert v() == 7
    tg = _trap_grads()
    tg.du_prev = t.u_prev
    assert v() == 7
    tg = _trap_grads()
    g.dB = t.lambda_
    assert v() == 7
    g = _good_grads(a)
    assert lib.msel_validate_trap_bwd(ctypes.byref(a), ctypes.byref(t), ctypes.byref(g),
                                      ctypes.byref(tg), None, 0) == 6


def test_complex_bwd_validation(lib):
    a = _good_args(N=16, L=1000)
    a.chunk_states = _addr()
    g = _good_grads(a)
    ws, big = _addr(), 1 << 20
    v = lambda: lib.msel_validate_complex_bwd(ctypes.byref(a), ctypes.byref(g), ws, big)
    assert v() == 0
    a.dstate = 15
    assert v() == 2
    a.dstate = 16
    # without the forward's chunk states they are rebuilt: the workspace must hold them too
    a.chunk_states = None
    need = lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a))
    assert lib.msel_validate_complex_bwd(ctypes.byref(a), ctypes.byref(g), ws, need) == 0
    assert lib.msel_validate_complex_bwd(ctypes.byref(a), ctypes.byref(g), ws, need - 1) == 6
    assert lib.msel_scan_complex_bwd(ctypes.byref(a), ctypes.byref(g), ws, need - 1, None) == 6
    a.chunk_states = _addr()
    assert lib.msel_validate_complex_bwd(ctypes.byref(a), ctypes.byref(g), None, 0) == 6
    g.dC = a.C
    assert v() == 7


def test_variant_chunk_carry_validation(lib):
    a = _good_args(N=16, L=1000)
    a.chunk_states = _addr()
    t = _trap()
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t)) == 0
    assert lib.msel_validate_complex_chunk_carry(ctypes.byref(a)) == 0
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), None) == 1
    t2 = _trap()
    t2.lambda_ = None
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t2)) == 1
    assert lib.msel_scan_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t2), None) == 1
    t2 = _trap()
    t2.lambda_ += 8
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t2)) == 4
    t2 = _trap()
    t2.lambda_ = a.chunk_states
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t2)) == 7
    a.dstate = 15
    assert lib.msel_validate_complex_chunk_carry(ctypes.byref(a)) == 2
    assert lib.msel_scan_complex_chunk_carry(ctypes.byref(a), None) == 2
    a.dstate = 16
    a.chunk_states = None  # required: the pass's product
    assert lib.msel_validate_trap_chunk_carry(ctypes.byref(a), ctypes.byref(t)) == 1
    assert lib.msel_validate_complex_chunk_carry(ctypes.byref(a)) == 1
