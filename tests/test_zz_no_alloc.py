"""mla_verify_noalloc: the single-sequence call with its split partials in the
library's static device scratch instead of a caller workspace. Through the C
ABI, against mla_verify_ex with a torch-allocated workspace (the same kernels,
so the outputs must be bitwise equal) and against the fp64 oracle, on two
calls in a row, the second with a smaller input."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import _lib, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3


def _dev(case):
    return {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}


def _args(d, case):
    return (d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(), d["k_rope"].data_ptr(),
            d["tree_parent"].data_ptr(), case.prefix_len, ctypes.c_float(case.scale))


def _outputs(case):
    q, h = case.q_len, case.num_heads
    return (torch.full((q, h, 512), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((q, h), float("nan"), dtype=torch.float32, device=DEV))


def call_noalloc(lib, case, d, opt=None):
    out, lse = _outputs(case)
    opt = opt or _lib.options()
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.mla_verify_noalloc(*_args(d, case), out.data_ptr(), lse.data_ptr(), case.q_len, case.num_heads,
                                stream, ctypes.byref(opt))
    return rc, out, lse


def call_ex(lib, case, d):
    out, lse = _outputs(case)
    n = case.prefix_len + case.q_len
    need = _lib.workspace_size(case.q_len, case.num_heads, 1, n, n)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    opt = _lib.options()
    rc = lib.mla_verify_ex(*_args(d, case), out.data_ptr(), lse.data_ptr(), case.q_len, case.num_heads,
                           ws.data_ptr(), need, stream, ctypes.byref(opt))
    return rc, out, lse


def assert_oracle(out, lse, case, label):
    ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                            case.prefix_len, case.scale)
    o = out.cpu().double().numpy()
    err = np.abs(o - ro)
    assert (err <= ATOL + RTOL * np.abs(ro)).all(), f"{label}: worst err/tol {(err / (ATOL + RTOL * np.abs(ro))).max()}"
    assert np.abs(lse.cpu().double().numpy() - rl).max() <= LSE_TOL, label


def test_noalloc_equals_workspace_call_twice_second_smaller(lib):
    big = gen.make_workload("q9_p16384")
    small = gen.make_case(9, 1000, tree="random", seed=77)
    n_big = big.prefix_len + big.q_len
    assert 0 < _lib.workspace_size(9, 64, 1, n_big, n_big) <= _lib.MLAV_SCRATCH_BYTES
    results = []
    for case in (big, small):
        d = _dev(case)
        rc, o1, l1 = call_noalloc(lib, case, d)
        assert rc == _lib.MLAV_OK, _lib.strerror(rc)
        rc, o2, l2 = call_ex(lib, case, d)
        assert rc == _lib.MLAV_OK, _lib.strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"prefix {case.prefix_len}: differs from mla_verify_ex"
        results.append((case, o1, l1))
    for case, o, l in results:
        assert_oracle(o, l, case, f"noalloc prefix {case.prefix_len}")


def test_noalloc_back_to_back_in_stream_order(lib):
    """Two calls queued back to back on one stream share the scratch safely."""
    a = gen.make_case(9, 5000, tree="random", seed=78)
    b = gen.make_case(9, 300, tree="chain", seed=79)
    da, db = _dev(a), _dev(b)
    rca, oa, la = call_noalloc(lib, a, da)
    rcb, ob, lb = call_noalloc(lib, b, db)
    assert rca == _lib.MLAV_OK and rcb == _lib.MLAV_OK
    torch.cuda.synchronize()
    assert_oracle(oa, la, a, "first of two")
    assert_oracle(ob, lb, b, "second of two")


def test_noalloc_refuses_plans_beyond_the_scratch(lib):
    """fp32 partials over many forced splits need more than the static scratch:
    refused on the host, nothing launched (the outputs keep their NaN fill)."""
    case = gen.make_case(9, 60000, tree="random", seed=80)
    n = case.prefix_len + case.q_len
    opt = _lib.options(nsplit=512, partials=1)
    need = int(lib.mla_verify_workspace_size(9, 64, 1, n, n, 0, ctypes.byref(opt)))
    assert need > _lib.MLAV_SCRATCH_BYTES
    d = _dev(case)
    rc, out, lse = call_noalloc(lib, case, d, opt)
    torch.cuda.synchronize()
    assert rc == _lib.MLAV_ERR_SCRATCH
    assert torch.isnan(out).all() and torch.isnan(lse).all()
