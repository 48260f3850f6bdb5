"""GPU parity of the direct form (GDN_ALGO_DIRECT; GDN_ALGO_AUTO's choice for
bf16 launches of at most 2 frames) against the float64 oracle.

The direct form walks the frames in turn and applies the module-2 update
(summary page, 方法步骤详情) token by token from the rows: S_t = gamma_t
S_{t-1} + sum_n beta_n (s v_n - s^2 S_{t-1} k_n) k_n^T, O_t = S_t Q_t.  Same
bar as the frame form: relative L2 <= 2e-2 (bf16 io).
"""

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_frame_amd import binding as gb
from gated_deltanet_recurrence_frame_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = "cuda:0"


def rel_l2(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return np.linalg.norm((gpu - ref).ravel()) / (den if den > 0 else 1.0)


def f64(t):
    return gin.as_f64(t)


def dev(inp):
    return {k: v.to(DEV).contiguous() for k, v in inp.items()}


def check(inp, N, with_state=True, key_scale=0.0, **kw):
    d = dev(inp)
    o, so = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                       state_in=d["state"] if with_state else None, key_scale=key_scale,
                       algorithm="direct", **kw)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                            f64(inp["beta"]), N,
                            state_in=f64(inp["state"]) if with_state else None,
                            key_scale=key_scale, normalize_qk=kw.get("normalize_qk", False),
                            gate_logits=kw.get("gate_logits", False))
    og, sg = f64(o.cpu()), f64(so.cpu())
    eo, es = rel_l2(og, ro), rel_l2(sg, rs)
    # the worst (batch, head) block as well: an error confined to one head
    # cannot hide in the whole-tensor figure
    B, L, H, D = og.shape
    wo = max(rel_l2(og[b, :, h], ro[b, :, h]) for b in range(B) for h in range(H))
    ws = max(rel_l2(sg[b, h], rs[b, h]) for b in range(B) for h in range(H))
    print("direct rel_l2: o %.3e (worst head %.3e) state %.3e (worst head %.3e)" % (eo, wo, es, ws))
    assert np.all(np.isfinite(og))
    assert eo <= TOL and wo <= TOL, (eo, wo)
    assert es <= TOL and ws <= TOL, (es, ws)
    return o, so


@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96, 112, 128])
@pytest.mark.parametrize("N", [1, 20, 128, 130, 300])
def test_direct_matches_oracle(D, N):
    # chunks of 128 tokens: N = 130 and 300 leave ragged chunks; two batches,
    # odd H, a carried-in state
    inp = gin.make_inputs(B=2, H=3, T=3, N=N, D=D, io="bf16", gamma="sigmoid", seed=70 + D,
                          with_state=True)
    check(inp, N)


@pytest.mark.parametrize("D", [16, 32, 48, 64, 80, 96, 112, 128])
@pytest.mark.parametrize("N", [129, 256, 300, 1000])
def test_direct_one_frame_token_parts(D, N):
    # one frame of more than 128 tokens: the tokens in parts of 128 (the last
    # ragged: 1, 0, 44 and 104 tokens past whole parts), then their ordered sum
    # with the outputs (D % 32 == 16 takes a last contraction block of 16)
    inp = gin.make_inputs(B=2, H=3, T=1, N=N, D=D, io="bf16", gamma="sigmoid", seed=90 + D,
                          with_state=True)
    check(inp, N)


@pytest.mark.parametrize("D", [16, 112])
def test_direct_one_frame_at_the_parts_cap(D):
    # 4096 tokens: 32 parts, the most the split takes (the sum's loads run in
    # several rounds of eight parts)
    inp = gin.make_inputs(B=1, H=2, T=1, N=4096, D=D, io="bf16", gamma="sigmoid", seed=96,
                          with_state=True)
    check(inp, 4096)


def test_direct_one_frame_beyond_the_parts_cap():
    # more than 32 parts' worth of tokens (4200): the frame's chunks are
    # walked in one workgroup per row block instead
    inp = gin.make_inputs(B=1, H=2, T=1, N=4200, D=48, io="bf16", gamma="sigmoid", seed=97,
                          with_state=True)
    check(inp, 4200)


@pytest.mark.parametrize("with_state", [False, True])
def test_direct_one_frame_parts_prologue_and_no_state(with_state):
    inp = gin.make_inputs(B=1, H=4, T=1, N=520, D=64, io="bf16", seed=95,
                          with_state=with_state, raw=True)
    check(inp, 520, with_state=with_state, normalize_qk=True, gate_logits=True)


@pytest.mark.parametrize("T", [1, 2, 8])
def test_direct_layer_shape(T):
    # the layer's heads and frame size (20 x 112, 880 tokens)
    inp = gin.make_inputs(B=1, H=20, T=T, N=880, D=112, io="bf16", gamma="uniform", seed=80 + T,
                          with_state=True)
    o, so = check(inp, 880)
    d = dev(inp)
    of, sf = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], 880,
                        state_in=d["state"], algorithm="frame")
    torch.cuda.synchronize()
    # two bf16 roundings of different intermediates: close to each other
    assert rel_l2(f64(o.cpu()), f64(of.cpu())) < 1e-2
    assert rel_l2(f64(so.cpu()), f64(sf.cpu())) < 1e-2


def test_direct_delta_stress():
    # key scale sqrt(D / N): the correction term changes O by O(1)
    inp = gin.make_inputs(B=1, H=4, T=6, N=880, D=112, io="bf16", gamma="uniform", seed=83)
    check(inp, 880, with_state=False, key_scale=float(np.sqrt(112 / 880)))


def test_direct_is_auto_for_short_bf16_launches():
    inp = gin.make_inputs(B=1, H=2, T=2, N=100, D=64, io="bf16", seed=84, with_state=True)
    d = dev(inp)
    args = (d["q"], d["k"], d["v"], d["gamma"], d["beta"], 100)
    o_d, s_d = gb.forward(*args, state_in=d["state"], algorithm="direct")
    o_a, s_a = gb.forward(*args, state_in=d["state"])
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_a) and torch.equal(s_d, s_a)
    # with a saved buffer auto takes the frame form (which fills it)
    o_s, s_s, saved = gb.forward(*args, state_in=d["state"], return_saved=True)
    o_f, s_f = gb.forward(*args, state_in=d["state"], algorithm="frame")
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_f) and torch.equal(s_s, s_f)


def test_direct_steps_in_place():
    # streaming: one gdn_step per frame, the state carried in place
    B, H, T, N, D = 1, 3, 5, 300, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="bf16", gamma="uniform", seed=85,
                          with_state=True)
    d = dev(inp)
    state = d["state"].clone()
    outs = []
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        outs.append(gb.step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                            d["v"][:, sl].contiguous(), d["gamma"][:, t:t + 1].contiguous(),
                            d["beta"][:, sl].contiguous(), state).clone())
    torch.cuda.synchronize()
    ro, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                            f64(inp["beta"]), N, state_in=f64(inp["state"]))
    assert rel_l2(f64(torch.cat(outs, dim=1).cpu()), ro) <= TOL
    assert rel_l2(f64(state.cpu()), rs) <= TOL


@pytest.mark.parametrize("nq,gl", [(True, False), (False, True), (True, True)])
def test_direct_prologue(nq, gl):
    inp = gin.make_inputs(B=1, H=3, T=3, N=150, D=112, io="bf16", seed=86, with_state=True,
                          raw=True)
    check(inp, 150, normalize_qk=nq, gate_logits=gl)


def test_step_plan_matches_step():
    # the preallocated streaming plan calls the same entry point
    B, H, T, N, D = 1, 4, 3, 200, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="bf16", seed=87, with_state=True)
    d = dev(inp)
    s1, s2 = d["state"].clone(), d["state"].clone()
    plan = gb.StepPlan(B, H, N, D, "bf16", torch.device(DEV))
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        args = (d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["gamma"][:, t:t + 1],
                d["beta"][:, sl])
        o1 = gb.step(*[x.contiguous() for x in args], s1)
        o2 = plan(*args, s2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)
