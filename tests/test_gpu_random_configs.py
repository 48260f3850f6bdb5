"""GPU parity on seeded random configurations against the float64 oracle.

The other GPU tests enumerate each feature on its own; here every case draws
its own combination: io dtype, head size, batch, heads, frames, tokens per
frame, algorithm (auto, frame, direct, token), the block's prologue flags,
the scan's chunk length, an initial state, an explicit key scale, and a
backward with or without the forward's saved buffer.  The draws stay in the
well-conditioned regime of the recurrence (summary page, 方法步骤详情
module 2: keys L2-normalised, by the caller or by the prologue, and a key
scale near 1/sqrt(D N)), where bf16 rounding alone keeps the whole-tensor
error far below the bar; with raw keys and a large explicit scale the
recurrence itself amplifies input roundings past it (the oracle moves by as
much under bf16-sized input noise).  Bars: relative L2 <= 2e-2 (bf16 io),
<= 1e-5 (fp32 io), per output tensor.
"""

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_frame_amd import binding as gb
from gated_deltanet_recurrence_frame_amd import inputs as gin

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NCASES = 48


def rel_l2(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return np.linalg.norm((gpu - ref).ravel()) / (den if den > 0 else 1.0)


def draw(i):
    rng = np.random.default_rng(7000 + i)
    io = "bf16" if rng.random() < 0.75 else "fp32"
    D = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    B, H, T = int(rng.integers(1, 3)), int(rng.integers(1, 6)), int(rng.integers(1, 13))
    N = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 129, 200, 300]))
    algos = ["auto", "frame"] + (["direct"] if io == "bf16" else [])
    if N <= (64 if io == "bf16" else 32):
        algos.append("token")
    algo = str(rng.choice(algos))
    nq = bool(rng.random() < 0.3)          # raw keys only with the prologue's normalisation
    gl = bool(rng.random() < 0.3)
    chunk = int(rng.choice([0, 0, 2, 3, 5])) if algo == "frame" else 0
    state = bool(rng.random() < 0.6)
    # the default scale, or one within a factor of two of it
    ks = 0.0 if rng.random() < 0.6 else float(rng.uniform(0.5, 2.0) / np.sqrt(D * N))
    bwd = algo in ("auto", "frame") and rng.random() < 0.6
    saved = bwd and rng.random() < 0.5
    return dict(io=io, B=B, H=H, T=T, N=N, D=D, algo=algo, nq=nq, gl=gl, chunk=chunk,
                state=state, ks=ks, bwd=bwd, saved=saved)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_configuration(i):
    c = draw(i)
    print("case", i, c)
    N = c["N"]
    inp = gin.make_inputs(B=c["B"], H=c["H"], T=c["T"], N=N, D=c["D"], io=c["io"],
                          gamma="uniform", seed=7000 + i, with_state=c["state"],
                          with_do=c["bwd"], raw=c["nq"])
    d = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    state = d["state"] if c["state"] else None
    flags = dict(normalize_qk=c["nq"], gate_logits=c["gl"])
    res = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, state_in=state,
                     key_scale=c["ks"], scan_chunk=c["chunk"], return_saved=c["saved"],
                     algorithm=c["algo"], **flags)
    torch.cuda.synchronize()
    f64 = gin.as_f64
    args = [f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta")]
    s64 = f64(inp["state"]) if c["state"] else None
    ro, rs = oracle.forward(*args, N, state_in=s64, key_scale=c["ks"], **flags)
    tol = 2e-2 if c["io"] == "bf16" else 1e-5
    errs = {"o": rel_l2(f64(res[0].cpu()), ro), "state": rel_l2(f64(res[1].cpu()), rs)}
    if c["bwd"]:
        g = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                        state_in=state, saved=res[2] if c["saved"] else None,
                        key_scale=c["ks"], scan_chunk=c["chunk"], **flags)
        torch.cuda.synchronize()
        rg = oracle.backward(*args, N, f64(inp["d_o"]), state_in=s64, key_scale=c["ks"],
                             **flags)
        for k in ("dq", "dk", "dv", "dgamma", "dbeta", "dstate_in"):
            errs[k] = rel_l2(f64(g[k].cpu()), rg[k])
    print("rel_l2", {k: "%.2e" % v for k, v in errs.items()})
    for k, v in errs.items():
        assert np.isfinite(v) and v <= tol, (k, v, c)


NSTEPS = 24


def draw_chain(i):
    rng = np.random.default_rng(8000 + i)
    io = "bf16" if rng.random() < 0.8 else "fp32"
    D = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    B, H, T = int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 7))
    N = int(rng.choice([1, 5, 64, 127, 128, 129, 255, 256, 257, 500, 880, 1000]))
    algo = str(rng.choice(["auto", "frame"] + (["direct"] if io == "bf16" else [])))
    return dict(io=io, B=B, H=H, T=T, N=N, D=D, algo=algo, nq=bool(rng.random() < 0.3),
                gl=bool(rng.random() < 0.3), state=bool(rng.random() < 0.7),
                plan=bool(rng.random() < 0.5))


@pytest.mark.parametrize("i", range(NSTEPS))
def test_random_step_chain(i):
    # T gdn_step calls (through a StepPlan or the one-call helper), the state
    # carried in place, against one oracle forward over the T frames
    c = draw_chain(i)
    print("chain", i, c)
    B, H, T, N, D = c["B"], c["H"], c["T"], c["N"], c["D"]
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=c["io"], gamma="uniform", seed=8000 + i,
                          with_state=c["state"], raw=c["nq"])
    d = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    st = d["state"].clone() if c["state"] else torch.zeros(B, H, D, D, device=DEV)
    plan = gb.StepPlan(B, H, N, D, c["io"], torch.device(DEV), algorithm=c["algo"],
                       flags=gb.flags_of(c["nq"], c["gl"])) if c["plan"] else None
    outs = []
    for t in range(T):
        w = {k: d[k][:, t * N:(t + 1) * N].contiguous() for k in ("q", "k", "v", "beta")}
        g = d["gamma"][:, t:t + 1].contiguous()
        if plan is not None:
            outs.append(plan(w["q"], w["k"], w["v"], g, w["beta"], st).clone())
        else:
            outs.append(gb.step(w["q"], w["k"], w["v"], g, w["beta"], st, algorithm=c["algo"],
                                normalize_qk=c["nq"], gate_logits=c["gl"]))
    torch.cuda.synchronize()
    f64 = gin.as_f64
    ro, rs = oracle.forward(*(f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta")), N,
                            state_in=f64(inp["state"]) if c["state"] else None,
                            normalize_qk=c["nq"], gate_logits=c["gl"])
    tol = 2e-2 if c["io"] == "bf16" else 1e-5
    eo = rel_l2(f64(torch.cat(outs, dim=1).cpu()), ro)
    es = rel_l2(f64(st.cpu()), rs)
    print("rel_l2 o %.2e state %.2e" % (eo, es))
    assert eo <= tol and es <= tol, (eo, es, c)
