"""GPU parity of the backward's fused plan (page 4, Appendix D, Speed and Memory: the chunk
carry run backward inside the recomputing gradient kernel), forced with msel_set_bwd_fused(1)
so that it runs at sizes the default leaves to the chunk-parallel plan:

* against the fp64 oracle (oracle/msel_oracle.c) over ragged chunks, dstate 1 to 16, both
  dtypes, the gate and the softplus on and off, h0 and dh0, one step, more chunks than the
  default allows, and several channels per wavefront with idle wavefronts in the last group;
* determinism: with no atomics, two runs give every output bit for bit;
* against the chunk-parallel plan on the same inputs (the same values up to rounding order);
* under the checked build (every kernel index range-checked): no index out of range.

The full-size case, where the default takes the fused plan (8 x 1536 x 16 x 2048), is
test_gpu_full.py's workload-2 backward with the forward's chunk states.  The bar:
max|gpu - oracle| <= tol * max|oracle| per tensor (1e-4 fp32, 1e-2 bf16 inputs).
"""
import numpy as np
import pytest

import msel_inputs
import oracle
from helpers import assert_close, host, log, oracle_vals, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_26_amd as msel  # noqa: E402
from selective_state_space_26_amd import _lib  # noqa: E402

CASES = [
    # batch, dim, dstate, seqlen, dtype, gate, softplus, D and bias, h0
    (1, 4, 4, 64, "f32", True, True, True, True),
    (2, 6, 16, 1100, "f32", True, True, True, True),
    (2, 6, 16, 1100, "bf16", True, True, True, True),
    (2, 5, 16, 2048, "bf16", False, True, True, False),
    (3, 3, 7, 700, "f32", False, False, False, True),
    (1, 3, 16, 1, "f32", True, True, True, True),        # one step
    (2, 13, 11, 700, "f32", True, True, True, True),     # dstate 11: the largest LDS need
    (1, 25, 10, 1030, "bf16", True, True, True, False),  # two accumulator groups, ragged tail
    (1, 1, 1, 777, "bf16", True, True, True, True),      # dstate 1: 12 accumulator groups
    (1, 5, 16, 5000, "f32", True, True, True, True),     # 10 chunks
    (1, 3100, 4, 600, "bf16", True, True, True, True),   # 2 channels per wavefront, idle waves
]


def _ids(c):
    return "x".join(map(str, c[:5]))


def _inputs(bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0, seed=321):
    t = msel_inputs.make(bsz, dim, N, L, dtype, seed, with_z=with_z, with_D=with_db,
                         with_bias=with_db, with_h0=with_h0, with_dout=True)
    if not sp:  # without the softplus keep Delta = delta + bias positive and small
        v = np.abs(t.values("delta")) * np.float32(0.2)
        t["delta"] = msel_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v
        if t.get("bias") is not None:
            t["bias"] = (np.abs(t["bias"]) * np.float32(0.01)).astype(np.float32)
    return t


@pytest.fixture
def plan():
    """Sets the backward's plan for the test (1 fused, -1 chunk-parallel) and restores the
    default after it."""
    yield msel.set_bwd_fused
    msel.set_bwd_fused(0)


def _bwd(dv, sp, want_dh0):
    a = (dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"])
    o = (dv["D"], dv["z"], dv["bias"], sp, dv["h0"])
    _, _, cs = msel.msel_scan_fwd(*a, *o, return_final_state=False, return_chunk_states=True)
    g = msel.msel_scan_bwd(*a, dv["dout"], *o, chunk_states=cs, want_dh0=want_dh0)
    torch.cuda.synchronize()
    return {k: v for k, v in g.items() if v is not None}


@pytest.mark.parametrize("want_dh0", [True, False])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fused_matches_oracle(plan, case, want_dh0):
    bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0 = case
    log(f"fused bwd {case} want_dh0={want_dh0}")
    plan(1)
    t = _inputs(*case)
    dv = to_device(t)
    assert msel.bwd_fused(dv["u"], dv["A"])
    g = _bwd(dv, sp, want_dh0)
    v = oracle_vals(t)
    r = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], v["h0"], softplus=sp)
    names = ["du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias"]
    names += ["dh0"] if want_dh0 else []
    names += ["dz"] if with_z else []
    assert sorted(g) == sorted(names)
    for k in names:
        assert_close(k, host(g[k]), r[k], dtype)


def test_fused_is_deterministic(plan):
    plan(1)
    case = (2, 50, 16, 1500, "bf16", True, True, True, True)
    log(f"fused bwd determinism {case}")
    dv = to_device(_inputs(*case))
    g1 = _bwd(dv, True, True)
    g2 = _bwd(dv, True, True)
    for k, v in g1.items():
        assert torch.equal(v, g2[k]), k


@pytest.mark.parametrize("case", [CASES[2], CASES[7], CASES[10]], ids=_ids)
def test_fused_agrees_with_chunk_parallel(plan, case):
    log(f"fused against chunk-parallel {case}")
    dv = to_device(_inputs(*case))
    plan(1)
    gf = _bwd(dv, case[6], True)
    plan(-1)
    assert not msel.bwd_fused(dv["u"], dv["A"])
    gc = _bwd(dv, case[6], True)
    assert sorted(gf) == sorted(gc)
    for k, v in gc.items():
        assert_close(k, host(gf[k]), host(v), case[4])


@pytest.mark.parametrize("case", [CASES[1], CASES[7], CASES[10]], ids=_ids)
def test_fused_in_range_under_checks(plan, case):
    """No index out of range, and every output equal to the release build's bit for bit (the
    fused plan has no atomics, and the checks change no arithmetic)."""
    log(f"fused bwd, checked build {case}")
    dv = to_device(_inputs(*case))
    plan(1)
    ref = _bwd(dv, case[6], True)
    with _lib.using(_lib.LIB_CHECKED_PATH):
        msel.set_bwd_fused(1)  # the setting is each library's own
        try:
            msel.bound_violations()
            got = _bwd(dv, case[6], True)
            count, f, line = msel.bound_violations()
        finally:
            msel.set_bwd_fused(0)
    assert count == 0, f"{count} out-of-range indexes, the first at {f}:{line}"
    assert sorted(got) == sorted(ref)
    for k, v in ref.items():
        assert torch.equal(got[k], v), k
