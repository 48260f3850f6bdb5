"""GPU parity of libgdn (through its C ABI) against the float64 oracle.

Bars: relative L2 error per output tensor <= 1e-5 when the io dtype is fp32
and <= 2e-2 when it is bf16.  Inputs come from the shared seeded generator;
the oracle reads back the exact values the GPU sees (bf16 or fp32, upcast
to float64).
"""

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_frame_amd import binding as gb
from gated_deltanet_recurrence_frame_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
DEV = "cuda:0"


def rel_l2(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return np.linalg.norm((gpu - ref).ravel()) / (den if den > 0 else 1.0)


def rel_l2_frames(gpu, ref, N):
    """Relative L2 error of every (batch, frame, head) block of a token
    tensor [B, L, H(, D)] (frames of N tokens): an error confined to one
    frame of one head cannot hide in the whole-tensor figure."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    B, L, H = r.shape[:3]
    T = L // N
    g = g.reshape(B, T, N, H, -1)
    r = r.reshape(B, T, N, H, -1)
    num = np.sqrt(((g - r) ** 2).sum(axis=(2, 4)))
    den = np.sqrt((r ** 2).sum(axis=(2, 4)))
    return num / np.where(den > 0, den, 1.0)


def rel_l2_heads(gpu, ref):
    """Relative L2 error of every (batch, head) slice of a state [B, H, D, D]."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((g - r) ** 2).sum(axis=(2, 3)))
    den = np.sqrt((r ** 2).sum(axis=(2, 3)))
    return num / np.where(den > 0, den, 1.0)


def check_blocks(name, gpu, ref, N, tol):
    """Whole-tensor and worst-block relative L2 against `tol` (token tensors
    by (batch, frame, head), states by (batch, head))."""
    whole = rel_l2(gpu, ref)
    is_state = name in ("state", "dstate_in")
    blocks = rel_l2_heads(gpu, ref) if is_state else rel_l2_frames(gpu, ref, N)
    worst = float(np.max(blocks))
    print("  %s: rel_l2 %.3e, worst block %.3e" % (name, whole, worst))
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), name
    assert whole <= tol, (name, whole)
    assert worst <= tol, (name, worst)
    return whole, worst


def to_dev(t):
    return None if t is None else t.to(DEV).contiguous()


def f64(t):
    return gin.as_f64(t)


def run_forward_pair(inp, N, io, key_scale=0.0, scan_chunk=0, with_state=False,
                     algorithm="frame"):
    d = {k: to_dev(v) for k, v in inp.items()}
    st = d.get("state") if with_state else None
    o, so = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, state_in=st,
                       key_scale=key_scale, scan_chunk=scan_chunk, algorithm=algorithm)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                            f64(inp["beta"]), N,
                            state_in=f64(inp["state"]) if with_state else None,
                            key_scale=key_scale)
    return (o.cpu(), so.cpu()), (ro, rs)


def check_forward(inp, N, io, **kw):
    (o, so), (ro, rs) = run_forward_pair(inp, N, io, **kw)
    print("forward:")
    eo, _ = check_blocks("o", f64(o), ro, N, TOL[io])
    es, _ = check_blocks("state", f64(so), rs, N, TOL[io])
    return eo, es


# ---------------------------------------------------------------- forward
def test_forward_tiny_fp32():
    inp = gin.make_config("tiny", seed=0, with_state=True)
    check_forward(inp, 4, "fp32")
    check_forward(inp, 4, "fp32", with_state=True)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 48, 64, 112, 128])
@pytest.mark.parametrize("algorithm", ["frame", "auto"])
def test_forward_head_dims_ragged(io, D, algorithm):
    # several token chunks with a ragged tail (N = 100), two batches, odd H
    # (auto: the direct form for bf16 at two frames)
    T = 2 if algorithm == "auto" else 5
    inp = gin.make_inputs(B=2, H=3, T=T, N=100, D=D, io=io, gamma="uniform", seed=1,
                          with_state=True)
    check_forward(inp, 100, io, with_state=True, algorithm=algorithm)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 16, 37, 64, 65, 200])
def test_forward_token_counts(io, N):
    inp = gin.make_inputs(B=1, H=2, T=6, N=N, D=112, io=io, gamma="sigmoid", seed=2)
    check_forward(inp, N, io)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_forward_items_with_odd_chunk_counts(io):
    # 600 (frame, head pair) items over at most 256 persistent Gram
    # workgroups, each item an odd number of token chunks: consecutive items
    # of one workgroup must alternate their LDS stages across the item
    # boundary as well
    inp = gin.make_inputs(B=1, H=20, T=60, N=65, D=112, io=io, gamma="sigmoid", seed=4)
    check_forward(inp, 65, io)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_short_clip_bf16(seed):
    inp = gin.make_config("short", seed=seed)
    eo, _ = check_forward(inp, 880, "bf16")
    assert eo < 5e-3          # bf16 rounding of S_t and O only


def test_forward_short_clip_fp32_mode():
    inp = gin.make_config("short", seed=0, io="fp32")
    check_forward(inp, 880, "fp32")


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_forward_delta_stress(io):
    # key scale sqrt(Dk/N): the delta correction changes O by O(1), so a
    # wrong or missing erase term cannot hide under the bf16 tolerance.
    inp = gin.make_inputs(B=1, H=4, T=21, N=880, D=112, io=io, gamma="uniform", seed=3)
    ks = float(np.sqrt(112 / 880))
    check_forward(inp, 880, io, key_scale=ks)
    # the erase term really matters at this scale
    ro_off, _ = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                               f64(inp["beta"]), 880, key_scale=ks, erase=0.0)
    ro_on, _ = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                              f64(inp["beta"]), 880, key_scale=ks)
    assert rel_l2(ro_off, ro_on) > 0.5


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_exact_retrieval(io):
    # gamma = 1, beta = 1, key scale 1, keys orthonormal in each frame, Q = K:
    # every frame reads back its own values exactly (up to input rounding).
    B, H, T, N, D = 1, 4, 6, 112, 112
    k, v = gin.orthonormal_frame_keys(B, H, T, N, D, seed=4, io=io)
    g = torch.ones((B, T, H))
    beta = torch.ones((B, T * N, H))
    kd, vd = to_dev(k), to_dev(v)
    o, _ = gb.forward(kd, kd, vd, to_dev(g), to_dev(beta), N, key_scale=1.0)
    ro, _ = oracle.forward(f64(k), f64(k), f64(v), f64(g), f64(beta), N, key_scale=1.0)
    e_or = rel_l2(f64(o.cpu()), ro)
    e_v = rel_l2(f64(o.cpu()), f64(v))
    print("exact retrieval: vs oracle %.3e, vs V %.3e" % (e_or, e_v))
    assert e_or <= TOL[io]
    assert e_v <= (1e-4 if io == "fp32" else 3e-2)


def test_saved_intermediates_fp32():
    inp = gin.make_inputs(B=1, H=2, T=4, N=50, D=32, io="fp32", gamma="uniform", seed=5,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    o, so, saved = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], 50,
                              state_in=d["state"], return_saved=True)
    torch.cuda.synchronize()
    _, _, kept = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                                f64(inp["beta"]), 50, state_in=f64(inp["state"]), keep=True)
    sv = saved.view(torch.float32).cpu().numpy().astype(np.float64)
    n = kept["A"].size
    assert rel_l2(sv[:n].reshape(kept["A"].shape), kept["A"]) < 1e-5
    assert rel_l2(sv[n:].reshape(kept["S"].shape), kept["S"]) < 1e-5


def test_in_place_state():
    inp = gin.make_inputs(B=1, H=2, T=3, N=20, D=16, io="fp32", gamma="uniform", seed=6,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    prob = gb.make_problem(1, 2, 3, 20, 16, "fp32")
    o = torch.empty_like(d["v"])
    ws = torch.empty(gb.workspace_size(prob, gb.GDN_OP_FORWARD), dtype=torch.uint8, device=DEV)
    st = d["state"].clone()
    import ctypes
    code = gb.lib().gdn_forward(ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]),
                                gb._p(d["gamma"]), gb._p(d["beta"]), gb._p(st), gb._p(o),
                                gb._p(st), None, gb._p(ws), ws.numel(), None)
    assert code == 0
    torch.cuda.synchronize()
    _, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                           f64(inp["beta"]), 20, state_in=f64(inp["state"]))
    assert rel_l2(f64(st.cpu()), rs) < 1e-5


# ------------------------------------------------------------- properties
def test_deterministic_and_homogeneous_bf16():
    inp = gin.make_inputs(B=1, H=4, T=7, N=200, D=112, io="bf16", gamma="uniform", seed=7)
    d = {k: to_dev(v) for k, v in inp.items()}
    o1, s1 = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], 200)
    o2, s2 = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], 200)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    # O is linear in V with S_0 = 0 and scaling by 2 commutes with rounding
    o3, s3 = gb.forward(d["q"], d["k"], 2 * d["v"], d["gamma"], d["beta"], 200)
    assert torch.equal(o3, 2 * o1) and torch.equal(s3, 2 * s1)


def test_permutation_within_frames_fp32():
    B, H, T, N, D = 1, 2, 4, 48, 32
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="fp32", gamma="uniform", seed=8)
    rng = np.random.default_rng(80)
    perm = torch.from_numpy(np.concatenate([t * N + rng.permutation(N) for t in range(T)]))
    d = {k: to_dev(v) for k, v in inp.items()}
    o, s = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N)
    p = perm.to(DEV)
    op, sp = gb.forward(d["q"][:, p].contiguous(), d["k"][:, p].contiguous(),
                        d["v"][:, p].contiguous(), d["gamma"], d["beta"][:, p].contiguous(), N)
    assert rel_l2(f64(op.cpu()), f64(o[:, p].cpu())) < 1e-5
    assert rel_l2(f64(sp.cpu()), f64(s.cpu())) < 1e-5


# ------------------------------------------------------------------ step
@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_step_chain_equals_forward(io):
    B, H, T, N, D = 1, 3, 9, 130, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=9,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    o_full, s_full = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                                state_in=d["state"], algorithm="frame", scan_chunk=1)
    state = d["state"].clone()
    outs = []
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        outs.append(gb.step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                            d["v"][:, sl].contiguous(), d["gamma"][:, t:t + 1].contiguous(),
                            d["beta"][:, sl].contiguous(), state, algorithm="frame").clone())
    torch.cuda.synchronize()
    o_step = torch.cat(outs, dim=1)
    # the step path runs the same kernels frame by frame, the Gram/write sums
    # split over token ranges (fixed order): equal up to summation order
    tol_same = 1e-6 if io == "fp32" else 2e-3
    assert rel_l2(f64(o_step.cpu()), f64(o_full.cpu())) <= tol_same
    assert rel_l2(f64(state.cpu()), f64(s_full.cpu())) <= tol_same
    ro, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                            f64(inp["beta"]), N, state_in=f64(inp["state"]))
    assert rel_l2(f64(o_step.cpu()), ro) <= TOL[io]
    assert rel_l2(f64(state.cpu()), rs) <= TOL[io]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_chunk_causal_windows_equal_one_call(io):
    # streaming by windows of frames: the first latent frame alone, then
    # windows of 8, each a gdn_forward that carries the state in place
    B, H, T, N, D = 1, 3, 17, 130, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=21,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    o_full, s_full = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                                state_in=d["state"], algorithm="frame", scan_chunk=1)
    state = d["state"].clone()
    outs = []
    for t0, t1 in [(0, 1), (1, 9), (9, 17)]:
        sl = slice(t0 * N, t1 * N)
        plan = gb.ForwardPlan(B, H, t1 - t0, N, D, io, torch.device(DEV), algorithm="frame",
                              scan_chunk=1)
        o, st = plan(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                     d["v"][:, sl].contiguous(), d["gamma"][:, t0:t1].contiguous(),
                     d["beta"][:, sl].contiguous(), state_in=state, state_out=state)
        assert st.data_ptr() == state.data_ptr()
        outs.append(o.clone())
    torch.cuda.synchronize()
    o_win = torch.cat(outs, dim=1)
    # same kernels over fewer frames per launch: equal up to summation order
    tol_same = 1e-6 if io == "fp32" else 2e-3
    assert rel_l2(f64(o_win.cpu()), f64(o_full.cpu())) <= tol_same
    assert rel_l2(f64(state.cpu()), f64(s_full.cpu())) <= tol_same
    ro, rs = oracle.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                            f64(inp["beta"]), N, state_in=f64(inp["state"]))
    assert rel_l2(f64(o_win.cpu()), ro) <= TOL[io]
    assert rel_l2(f64(state.cpu()), rs) <= TOL[io]


# ------------------------------------------------------------ token form
@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("N,T,D", [(1, 150, 112), (2, 70, 112), (3, 50, 48), (5, 27, 112),
                                   (7, 20, 128), (16, 9, 112), (32, 5, 16), (1, 100, 16),
                                   (2, 40, 32)])
def test_token_form_matches_oracle(io, N, T, D):
    # chunks of floor(CP / N) frames, a ragged last chunk, a carried state;
    # small D leaves fewer waves than 16-token blocks of a chunk
    inp = gin.make_inputs(B=1, H=3, T=T, N=N, D=D, io=io, gamma="sigmoid", seed=40 + N,
                          with_state=True)
    check_forward(inp, N, io, with_state=True, algorithm="token")


@pytest.mark.parametrize("io,N,T,D", [("bf16", 1, 2000, 32), ("fp32", 1, 1000, 32),
                                      ("bf16", 3, 700, 48), ("bf16", 1, 1500, 112),
                                      ("fp32", 2, 600, 16)])
def test_token_form_segments(io, N, T, D):
    # long sequences: segments of chunks walked in parallel (composites, the
    # fold, a replay), with a carried state and a ragged last segment
    inp = gin.make_inputs(B=1, H=2, T=T, N=N, D=D, io=io, gamma="sigmoid", seed=70 + N,
                          with_state=True)
    check_forward(inp, N, io, with_state=True, algorithm="token")


@pytest.mark.parametrize("N", [33, 64])
def test_token_form_long_frames_bf16(N):
    # frames longer than half a chunk: one frame per chunk (fp32 stops at 32)
    inp = gin.make_inputs(B=2, H=2, T=6, N=N, D=112, io="bf16", gamma="uniform", seed=50 + N,
                          with_state=True)
    check_forward(inp, N, "bf16", with_state=True, algorithm="token")


@pytest.mark.parametrize("io,T", [("fp32", 40), ("bf16", 40), ("bf16", 700)])
def test_token_form_equals_frame_form_in_place(io, T):
    # T = 700 four-token frames: 44 chunks in 4 segments, state in place
    B, H, N, D = 1, 4, 4, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=60,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    o_f, s_f = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                          state_in=d["state"], algorithm="frame")
    plan = gb.ForwardPlan(B, H, T, N, D, io, torch.device(DEV), algorithm="token")
    st = d["state"].clone()
    o_t, s_t = plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"], state_in=st, state_out=st)
    torch.cuda.synchronize()
    assert s_t.data_ptr() == st.data_ptr()
    tol = 1e-5 if io == "fp32" else 2e-2
    assert rel_l2(f64(o_t.cpu()), f64(o_f.cpu())) <= tol
    assert rel_l2(f64(st.cpu()), f64(s_f.cpu())) <= tol


def test_token_form_gates_far_from_one_fp32():
    # gamma down to ~0.05 inside a chunk of 64 one-token frames: the decay
    # table's products must not lose the small ones
    B, H, T, N, D = 1, 2, 96, 1, 32
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="fp32", gamma="uniform", seed=61,
                          with_state=True)
    rng = np.random.default_rng(62)
    inp["gamma"] = torch.from_numpy(rng.uniform(0.05, 1.0, (B, T, H)).astype(np.float32))
    check_forward(inp, N, "fp32", with_state=True, algorithm="token")


# -------------------------------------------------------------- backward
def check_backward(inp, N, io, with_state=True, with_dstate=True, use_saved=False,
                   key_scale=0.0, scan_chunk=0):
    d = {k: to_dev(v) for k, v in inp.items()}
    st = d["state"] if with_state else None
    dst = d["d_state"] if with_dstate else None
    saved = None
    if use_saved:
        _, _, saved = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                                 state_in=st, key_scale=key_scale, return_saved=True)
    gr = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                     state_in=st, d_state_out=dst, saved=saved, key_scale=key_scale,
                     scan_chunk=scan_chunk)
    torch.cuda.synchronize()
    ref = oracle.backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["gamma"]),
                          f64(inp["beta"]), N, f64(inp["d_o"]),
                          state_in=f64(inp["state"]) if with_state else None,
                          d_state_out=f64(inp["d_state"]) if with_dstate else None,
                          key_scale=key_scale)
    print("backward:")
    errs = check_grads(gr, ref, N, io)
    return errs, gr


def check_grads(gr, ref, N, io):
    errs = {}
    for name in ["dq", "dk", "dv", "dbeta", "dstate_in"]:
        errs[name], _ = check_blocks(name, f64(gr[name].cpu()), ref[name], N, TOL[io])
    # dgamma: one value per (frame, head); whole tensor and per head
    g, r = f64(gr["dgamma"].cpu()), ref["dgamma"]
    errs["dgamma"] = rel_l2(g, r)
    per_head = [rel_l2(g[:, :, h], r[:, :, h]) for h in range(r.shape[2])]
    print("  dgamma: rel_l2 %.3e, worst head %.3e" % (errs["dgamma"], max(per_head)))
    assert errs["dgamma"] <= TOL[io] and max(per_head) <= TOL[io], ("dgamma", per_head)
    return errs


def test_backward_tiny_fp32():
    inp = gin.make_config("tiny", seed=0, with_do=True, with_dstate=True, with_state=True)
    check_backward(inp, 4, "fp32")
    check_backward(inp, 4, "fp32", with_state=False, with_dstate=False, use_saved=True)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [16, 64, 112])
def test_backward_ragged(io, D):
    inp = gin.make_inputs(B=2, H=3, T=5, N=100, D=D, io=io, gamma="uniform", seed=10,
                          with_do=True, with_dstate=True, with_state=True)
    check_backward(inp, 100, io)
    check_backward(inp, 100, io, use_saved=True)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_backward_delta_stress(io):
    inp = gin.make_inputs(B=1, H=2, T=12, N=880, D=112, io=io, gamma="uniform", seed=11,
                          with_do=True, with_dstate=True, with_state=True)
    check_backward(inp, 880, io, key_scale=float(np.sqrt(112 / 880)))


def test_backward_short_clip_bf16():
    inp = gin.make_config("short", seed=0, with_do=True)
    check_backward(inp, 880, "bf16", with_state=False, with_dstate=False, use_saved=True)


# ------------------------------------------ chunked (composite) scan
# The transition / input composites of the context-parallel scheme (summary
# page, 技术新颖性 point 1), with chunks of frames standing in for devices:
# the chunked forward and backward must give the sequential result.
# Sequential and chunked GPU runs differ only in rounding order (fp32 fold of
# the composites), so they are compared with a bar well under the oracle's.
SAME = {"fp32": 2e-6, "bf16": 5e-3}


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [2, 3, 4, 11])
def test_chunked_forward_matches_oracle(io, chunk):
    B, H, T, N, D = 2, 3, 11, 100, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=30 + chunk,
                          with_state=True)
    (o, so), (ro, rs) = run_forward_pair(inp, N, io, scan_chunk=chunk, with_state=True)
    eo, es = rel_l2(f64(o), ro), rel_l2(f64(so), rs)
    print("chunk %d forward rel_l2: o %.3e state %.3e" % (chunk, eo, es))
    assert eo <= TOL[io] and es <= TOL[io]
    # the oracle's own composite path agrees with its sequential one
    co, cs = oracle.composite_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                      f64(inp["gamma"]), f64(inp["beta"]), N, chunk,
                                      state_in=f64(inp["state"]))
    assert rel_l2(f64(o), co) <= TOL[io] and rel_l2(f64(so), cs) <= TOL[io]
    (o1, so1), _ = run_forward_pair(inp, N, io, scan_chunk=1, with_state=True)
    assert rel_l2(f64(o), f64(o1)) <= SAME[io]
    assert rel_l2(f64(so), f64(so1)) <= SAME[io]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [16, 48, 128])
def test_chunked_forward_long_ragged(io, D):
    # 64 frames in chunks of 5 (last chunk of 4): longer than the prefetch
    # ring inside a chunk, 13 chunks in the fold
    B, H, T, N = 1, 2, 64, 40
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=40 + D,
                          with_state=True)
    check_forward(inp, N, io, scan_chunk=5, with_state=True)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_chunked_forward_in_place(io):
    # state_out == state_in: the first chunk reads the entering state only
    # through the fold's copy, so the last chunk may overwrite it
    B, H, T, N, D = 1, 3, 20, 64, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=50,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    st = d["state"].clone()
    prob = gb.make_problem(B, H, T, N, D, io, scan_chunk=3)
    o = torch.empty_like(d["v"])
    ws = torch.empty(gb.workspace_size(prob, gb.GDN_OP_FORWARD), dtype=torch.uint8, device=DEV)
    import ctypes
    code = gb.lib().gdn_forward(ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]),
                                gb._p(d["gamma"]), gb._p(d["beta"]), gb._p(st), gb._p(o),
                                gb._p(st), None, gb._p(ws), ws.numel(),
                                gb._stream(torch.device(DEV)))
    assert code == 0
    o_ref, s_ref = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                              state_in=d["state"], scan_chunk=3)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [2, 3, 5])
def test_chunked_backward(io, chunk):
    inp = gin.make_inputs(B=2, H=3, T=11, N=100, D=112, io=io, gamma="uniform", seed=60 + chunk,
                          with_do=True, with_dstate=True, with_state=True)
    _, g_chunk = check_backward(inp, 100, io, scan_chunk=chunk)
    _, g_seq = check_backward(inp, 100, io, scan_chunk=1, use_saved=True)
    for name in ["dq", "dk", "dv", "dgamma", "dbeta", "dstate_in"]:
        e = rel_l2(f64(g_chunk[name].cpu()), f64(g_seq[name].cpu()))
        assert e <= SAME[io], (name, e)


# ---------------------------------------------------- host-side failures
def test_errors_write_nothing():
    inp = gin.make_inputs(B=1, H=2, T=3, N=20, D=16, io="fp32", gamma="uniform", seed=12)
    d = {k: to_dev(v) for k, v in inp.items()}
    import ctypes
    prob = gb.make_problem(1, 2, 3, 20, 16, "fp32")
    need = gb.workspace_size(prob, gb.GDN_OP_FORWARD)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o = torch.full_like(d["v"], 7.0)
    code = gb.lib().gdn_forward(ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]),
                                gb._p(d["gamma"]), gb._p(d["beta"]), None, gb._p(o), None, None,
                                gb._p(ws), need - 1, None)
    assert gb.STATUS[code] == "GDN_ERR_WORKSPACE_TOO_SMALL"
    # output aliasing an input
    code = gb.lib().gdn_forward(ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]),
                                gb._p(d["gamma"]), gb._p(d["beta"]), None, gb._p(d["q"]), None,
                                None, gb._p(ws), need, None)
    assert gb.STATUS[code] == "GDN_ERR_ALIASING"
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)


# ------------------------------------------------------ longer sequences
@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_forward_long_sequence_in_place(io):
    # more frames than the scan's prefetch ring and gamma window split, in
    # place and against the allocating call
    B, H, T, N, D = 1, 3, 64, 100, 112
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=20,
                          with_state=True)
    check_forward(inp, N, io, with_state=True)
    # in place, and with the saved buffer
    d = {k: to_dev(v) for k, v in inp.items()}
    st = d["state"].clone()
    prob = gb.make_problem(B, H, T, N, D, io)
    o = torch.empty_like(d["v"])
    ws = torch.empty(gb.workspace_size(prob, gb.GDN_OP_FORWARD), dtype=torch.uint8, device=DEV)
    import ctypes
    code = gb.lib().gdn_forward(ctypes.byref(prob), gb._p(d["q"]), gb._p(d["k"]), gb._p(d["v"]),
                                gb._p(d["gamma"]), gb._p(d["beta"]), gb._p(st), gb._p(o),
                                gb._p(st), None, gb._p(ws), ws.numel(),
                                gb._stream(torch.device(DEV)))
    assert code == 0
    o_ref, s_ref = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                              state_in=d["state"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


_MINUTE = {}


def _minute_inputs():
    if not _MINUTE:
        _MINUTE.update(gin.make_config("minute", seed=0, with_do=True))
    return _MINUTE


_MINUTE_REF = {}


def _minute_oracle_forward():
    """oracle.forward over all 20 heads of the one-minute inputs (cached)."""
    if not _MINUTE_REF:
        inp = _minute_inputs()
        _MINUTE_REF["fwd"] = oracle.forward(*(f64(inp[k]) for k in ("q", "k", "v", "gamma",
                                                                      "beta")), 880)
    return _MINUTE_REF["fwd"]


def test_forward_minute_config_all_heads():
    # the benchmark's own configuration and launch path, every head
    inp = _minute_inputs()
    d = {k: to_dev(v) for k, v in inp.items() if k != "d_o"}
    N = 880
    plan = gb.ForwardPlan(1, 20, 121, N, 112, "bf16", torch.device(DEV))
    o, st = plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    torch.cuda.synchronize()
    ro, rs = _minute_oracle_forward()
    print("minute forward, 20 heads:")
    check_blocks("o", f64(o.cpu()), ro, N, TOL["bf16"])
    check_blocks("state", f64(st.cpu()), rs, N, TOL["bf16"])


def test_stream_minute_chain_all_heads():
    # streaming: frame 0 from a zero state, then 120 gdn_step calls, the
    # state carried in place, with the plan the benchmark times (AUTO: the
    # direct form); the concatenated outputs and the final state against the
    # oracle's one-shot forward, every head and frame
    inp = _minute_inputs()
    d = {k: to_dev(v) for k, v in inp.items() if k != "d_o"}
    B, H, T, N, D = 1, 20, 121, 880, 112
    plan = gb.StepPlan(B, H, N, D, "bf16", torch.device(DEV))
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device=DEV)
    o = torch.empty_like(d["v"])
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        plan.o.view(torch.uint8).fill_(255)        # NaN before every call
        out = plan(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["gamma"][:, t:t + 1],
                   d["beta"][:, sl], state)
        o[:, sl].copy_(out)
    torch.cuda.synchronize()
    ro, rs = _minute_oracle_forward()
    print("minute stream, 121 calls, 20 heads:")
    check_blocks("o", f64(o.cpu()), ro, N, TOL["bf16"])
    check_blocks("state", f64(state.cpu()), rs, N, TOL["bf16"])


def test_train_minute_config_all_heads():
    inp = _minute_inputs()
    d = {k: to_dev(v) for k, v in inp.items()}
    N = 880
    plan = gb.ForwardPlan(1, 20, 121, N, 112, "bf16", torch.device(DEV), saved=True)
    plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    gr = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                     saved=plan.saved)
    torch.cuda.synchronize()
    ref = oracle.backward(*(f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta")), N,
                          f64(inp["d_o"]))
    print("minute backward, 20 heads:")
    check_grads(gr, ref, N, "bf16")


@pytest.mark.parametrize("seed", [1, 2])
def test_minute_config_other_seeds(seed):
    # the one-minute configuration repeated at seeds 1 and 2: forward (o,
    # state) and backward (every gradient), all 20 heads, per-block bars
    inp = gin.make_config("minute", seed=seed, with_do=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    N = 880
    plan = gb.ForwardPlan(1, 20, 121, N, 112, "bf16", torch.device(DEV), saved=True)
    o, st = plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    gr = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                     saved=plan.saved)
    torch.cuda.synchronize()
    f = {k: f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta", "d_o")}
    ro, rs = oracle.forward(f["q"], f["k"], f["v"], f["gamma"], f["beta"], N)
    print("minute seed %d, 20 heads:" % seed)
    check_blocks("o", f64(o.cpu()), ro, N, TOL["bf16"])
    check_blocks("state", f64(st.cpu()), rs, N, TOL["bf16"])
    ref = oracle.backward(f["q"], f["k"], f["v"], f["gamma"], f["beta"], N, f["d_o"])
    check_grads(gr, ref, N, "bf16")


def test_train_minute_prologue_all_heads():
    # the one-minute shape through the block's prologue as the bench's
    # prologue leg launches it (saved buffer, normalisation and gate logits
    # fused, the one-pass backward that takes dq and dk through the
    # normalisation's chain rule), on raw rows (per-row factors exp(N(0, 1)))
    # and gate logits: forward and every gradient, all 20 heads, per-block bars
    inp = gin.make_config("minute", seed=3, with_do=True, raw=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    N = 880
    plan = gb.ForwardPlan(1, 20, 121, N, 112, "bf16", torch.device(DEV),
                          flags=gb.flags_of(True, True), saved=True)
    o, st = plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    gr = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                     saved=plan.saved, normalize_qk=True, gate_logits=True)
    torch.cuda.synchronize()
    f = {k: f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta", "d_o")}
    flags = dict(normalize_qk=True, gate_logits=True)
    ro, rs = oracle.forward(f["q"], f["k"], f["v"], f["gamma"], f["beta"], N, **flags)
    print("minute prologue, 20 heads:")
    check_blocks("o", f64(o.cpu()), ro, N, TOL["bf16"])
    check_blocks("state", f64(st.cpu()), rs, N, TOL["bf16"])
    ref = oracle.backward(f["q"], f["k"], f["v"], f["gamma"], f["beta"], N, f["d_o"], **flags)
    check_grads(gr, ref, N, "bf16")


def _frag_to_rowmajor(a, D):
    """Undo the bf16 operand order of saved A_t (documented in include/gdn.h):
    element [r][c] of a frame sits at (r / 16) 16 D + (c / 32) 512 +
    (16 ((c % 32) / 8) + r % 16) 8 + c % 8."""
    r, c = np.meshgrid(np.arange(D), np.arange(D), indexing="ij")
    idx = (r // 16) * 16 * D + (c // 32) * 512 + (16 * ((c % 32) // 8) + r % 16) * 8 + c % 8
    return a[..., idx]


def test_saved_intermediates_bf16_short_clip():
    # the bf16 A_t and S_t of the saved buffer against the oracle's, every
    # head and frame.  A_t is one fp32 product rounded once to bf16: each
    # element within 2^-9 relative, so 4e-3 relative L2 (per frame too) is
    # twice the worst case.  S_t is carried in fp32 from bf16 operands
    # (A_t, U_t and the staged rows of S_{t-1}) and rounded to bf16 when
    # stored: 1e-2, the budget those roundings leave over 21 frames (a
    # float64 simulation of the same roundings stays near 3e-3).
    inp = gin.make_config("short", seed=0)
    B, H, T, N, D = 1, 20, 21, 880, 112
    d = {k: to_dev(v) for k, v in inp.items()}
    _, _, saved = gb.forward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N,
                             return_saved=True)
    torch.cuda.synchronize()
    _, _, kept = oracle.forward(*(f64(inp[k]) for k in ("q", "k", "v", "gamma", "beta")), N,
                                keep=True)
    sv = saved.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    n = B * H * T * D * D
    A = _frag_to_rowmajor(sv[:n].reshape(B, H, T, D * D), D)
    S = sv[n:2 * n].reshape(B, H, T, D, D)
    for name, g, r, tol in (("A_t", A, kept["A"], 4e-3), ("S_t", S, kept["S"], 1e-2)):
        assert np.all(np.isfinite(g)), name
        whole = rel_l2(g, r)
        per = np.sqrt(((g - r) ** 2).sum(axis=(3, 4))) / np.sqrt((r ** 2).sum(axis=(3, 4)))
        print("  saved %s: rel_l2 %.3e, worst (head, frame) %.3e" % (name, whole, per.max()))
        assert whole <= tol and per.max() <= tol, (name, whole, per.max())


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_default_scan_is_chunked_for_few_sequences(io):
    # scan_chunk = 0 takes composite chunks of 16 frames for at most 8
    # sequences: bit-identical to asking for them, and on the oracle's result
    B, H, T, N, D = 1, 2, 40, 60, 64
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io=io, gamma="uniform", seed=24,
                          with_state=True)
    d = {k: to_dev(v) for k, v in inp.items()}
    args = (d["q"], d["k"], d["v"], d["gamma"], d["beta"], N)
    o0, s0 = gb.forward(*args, state_in=d["state"], algorithm="frame")
    o16, s16 = gb.forward(*args, state_in=d["state"], algorithm="frame", scan_chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(o0, o16) and torch.equal(s0, s16)
    check_forward(inp, N, io, with_state=True)
