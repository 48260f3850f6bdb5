"""gdn_forward_noalloc (the forward on the library's static per-device
scratch, for callers that cannot allocate) against gdn_forward with a
caller workspace: the same kernels on the same inputs, so the outputs must be
bit-identical.  Two calls in a row, the second on a smaller problem (the
scratch keeps the first call's contents), both also against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_frame_amd import binding as gb
from gated_deltanet_recurrence_frame_amd import inputs as gin

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc(prob, d, state_in, o, state_out, saved):
    code = gb.lib().gdn_forward_noalloc(
        ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]), gb._p(d["gamma"]),
        gb._p(d["beta"]), gb._p(state_in), gb._p(o), gb._p(state_out), gb._p(saved),
        gb._stream(torch.device(DEV)))
    assert code == 0, gb.STATUS.get(code, code)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    return np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel())


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_noalloc_matches_forward_twice(io):
    shapes = [(1, 20, 9, 880, 112), (2, 3, 5, 100, 48)]   # the second smaller
    tol = 2e-2 if io == "bf16" else 1e-5
    for i, (B, H, T, N, D) in enumerate(shapes):
        inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=30 + i,
                              with_state=True)
        d = {k: v.to(DEV) for k, v in inp.items()}
        plan = gb.ForwardPlan(B, H, T, N, D, io, torch.device(DEV), saved=True)
        o_ref, s_ref = plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["state"])
        o = torch.full_like(o_ref, float("nan"))
        st = torch.full_like(s_ref, float("nan"))
        saved = torch.full_like(plan.saved, 255)
        _noalloc(plan.prob, d, d["state"], o, st, saved)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, s_ref)
        assert torch.equal(saved, plan.saved)
        ro, rs = oracle.forward(*(gin.as_f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta")),
                                N, state_in=gin.as_f64(inp["state"]))
        eo, es = _rel(gin.as_f64(o.cpu()), ro), _rel(gin.as_f64(st.cpu()), rs)
        print("noalloc %s call %d: o %.3e state %.3e" % (io, i, eo, es))
        assert eo <= tol and es <= tol


def test_noalloc_state_carried_in_place_over_windows():
    # the state carried in place over three windows, as a streaming caller
    # would: equal to one gdn_forward over all frames
    B, H, T, N, D = 1, 4, 6, 200, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="bf16", gamma="uniform", seed=33,
                          with_state=True)
    d = {k: v.to(DEV) for k, v in inp.items()}
    o_ref, s_ref = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                              state_in=d["state"])
    st = d["state"].clone()
    outs = []
    for t0, t1 in ((0, 1), (1, 4), (4, 6)):
        prob = gb.make_problem(B, H, t1 - t0, N, D, "bf16")
        w = {k: d[k][:, t0 * N:t1 * N].contiguous() for k in ("q", "k", "v", "beta")}
        w["gamma"] = d["gamma"][:, t0:t1].contiguous()
        o = torch.empty_like(w["v"])
        _noalloc(prob, w, st, o, st, None)
        outs.append(o)
    torch.cuda.synchronize()
    o_cat = torch.cat(outs, dim=1)
    assert _rel(gin.as_f64(o_cat.cpu()), gin.as_f64(o_ref.cpu())) < 5e-3
    assert _rel(gin.as_f64(st.cpu()), gin.as_f64(s_ref.cpu())) < 5e-3
