"""CPU checks of the C-ABI library: it loads, exports every function that
include/gdn.h declares, and its host-side validation answers without any
GPU work (every call here fails validation before a launch)."""

import ctypes
import os

import pytest

from gated_deltanet_recurrence_frame_amd import binding as gb

LIB = gb.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return gb.lib()


def test_exports_every_declared_function(lib):
    names = gb.header_functions()
    assert set(names) == {"gdn_abi_version", "gdn_status_string", "gdn_workspace_size",
                          "gdn_saved_size", "gdn_forward", "gdn_forward_events",
                          "gdn_forward_noalloc", "gdn_step", "gdn_backward"}
    for n in names:
        assert hasattr(lib, n), n
    # and the shared object's dynamic symbol table really carries them
    cdll = ctypes.CDLL(LIB)
    for n in names:
        getattr(cdll, n)


def test_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 4 == gb.ABI_VERSION
    for code in range(10):
        s = lib.gdn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.gdn_status_string(99).decode() == "unknown status"


def _ws(prob, op):
    n = ctypes.c_size_t(0)
    code = gb.lib().gdn_workspace_size(ctypes.byref(prob) if prob is not None else None, op,
                                       ctypes.byref(n))
    return code, n.value


def test_workspace_sizes(lib):
    B, H, T, N, D = 1, 20, 121, 880, 112
    p = gb.make_problem(B, H, T, N, D, "bf16")
    mat = B * H * T * D * D * 2            # bf16 intermediates for bf16 io
    assert _ws(p, gb.GDN_OP_FORWARD) == (0, 3 * mat)
    assert _ws(p, gb.GDN_OP_BACKWARD) == (0, 6 * mat)
    assert gb.STATUS[_ws(p, gb.GDN_OP_STEP)[0]] == "GDN_ERR_BAD_SHAPE"     # T != 1
    p1 = gb.make_problem(B, H, 1, N, D, "bf16")
    # a streaming step splits each frame's tokens over 8 workgroups and
    # keeps their fp32 partial A_t, U_t in the workspace
    assert _ws(p1, gb.GDN_OP_STEP) == (0, 3 * B * H * D * D * 2 + 8 * B * H * 2 * D * D * 4)
    # the direct form of one frame splits its tokens into parts of 128 (at most
    # 32) and keeps each part's fp32 update of the state: beyond the Gram's
    # partials from 4096 tokens; past 32 parts the frame is not split
    base = 3 * B * H * D * D * 2
    gram_parts = 8 * B * H * 2 * D * D * 4
    p4096 = gb.make_problem(B, H, 1, 4096, D, "bf16")
    assert _ws(p4096, gb.GDN_OP_STEP) == (0, base + 32 * B * H * D * D * 4)
    p4097 = gb.make_problem(B, H, 1, 4097, D, "bf16")
    assert _ws(p4097, gb.GDN_OP_STEP) == (0, base + gram_parts)
    assert gb.saved_size(p) == 2 * mat
    # a chunked scan (8-frame chunks: 16 chunks) keeps -C_w^T, H_w and the
    # entering state of every chunk in fp32
    pc = gb.make_problem(B, H, T, N, D, "bf16", scan_chunk=8)
    comp = 3 * B * H * 16 * D * D * 4
    assert _ws(pc, gb.GDN_OP_FORWARD) == (0, 3 * mat + comp)
    assert _ws(pc, gb.GDN_OP_BACKWARD) == (0, 6 * mat + comp)
    # a chunk as long as the sequence is the sequential scan
    assert _ws(gb.make_problem(B, H, T, N, D, "bf16", scan_chunk=T), gb.GDN_OP_FORWARD) == (0, 3 * mat)
    assert _ws(gb.make_problem(B, H, T, N, D, "bf16", scan_chunk=500), gb.GDN_OP_FORWARD) == (0, 3 * mat)
    pf = gb.make_problem(B, H, T, N, D, "fp32")
    assert gb.saved_size(pf) == 2 * B * H * T * D * D * 4
    # with normalised rows the saved buffer also keeps 1 / |q| per row (fp32)
    for io, es in (("bf16", 2), ("fp32", 4)):
        pn = gb.make_problem(B, H, T, N, D, io, flags=gb.GDN_FLAG_NORMALIZE_QK)
        assert gb.saved_size(pn) == 2 * B * H * T * D * D * es + B * T * N * H * 4


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, "GDN_ERR_BAD_SHAPE"), ("T", -1, "GDN_ERR_BAD_SHAPE"),
    ("N", 0, "GDN_ERR_BAD_SHAPE"), ("Dk", 24, "GDN_ERR_UNSUPPORTED"),
    ("Dk", 144, "GDN_ERR_UNSUPPORTED"), ("Dv", 64, "GDN_ERR_UNSUPPORTED"),
    ("io_dtype", 5, "GDN_ERR_BAD_DTYPE"), ("scan_chunk", -2, "GDN_ERR_BAD_SHAPE"),
    ("key_scale", float("nan"), "GDN_ERR_BAD_SHAPE"),
    ("N", 1 << 24, "GDN_ERR_BAD_SHAPE"),       # token offsets use 24-bit multiplies
])
def test_problem_validation(lib, field, value, status):
    p = gb.make_problem(1, 2, 4, 8, 32, "bf16")
    setattr(p, field, value)
    code, _ = _ws(p, gb.GDN_OP_FORWARD)
    assert gb.STATUS[code] == status


def test_null_and_alignment_checks_before_any_launch(lib):
    p = gb.make_problem(1, 2, 4, 8, 32, "fp32")
    vp = ctypes.c_void_p
    code = lib.gdn_forward(None, *([None] * 10), 0, None)
    assert gb.STATUS[code] == "GDN_ERR_NULL_POINTER"
    code = lib.gdn_forward(ctypes.byref(p), *([None] * 10), 0, None)
    assert gb.STATUS[code] == "GDN_ERR_NULL_POINTER"
    # fake, never dereferenced addresses: misalignment is caught first
    good = [vp(0x100000 * (i + 1)) for i in range(10)]
    bad = list(good)
    bad[0] = vp(0x100008)
    code = lib.gdn_forward(ctypes.byref(p), *bad, 1 << 30, None)
    assert gb.STATUS[code] == "GDN_ERR_MISALIGNED"
    code = lib.gdn_forward(ctypes.byref(p), *good, 16, None)
    assert gb.STATUS[code] == "GDN_ERR_WORKSPACE_TOO_SMALL"
    # the output overlapping an input
    alias = list(good)
    alias[6] = alias[0]
    code = lib.gdn_forward(ctypes.byref(p), *alias, 1 << 30, None)
    assert gb.STATUS[code] == "GDN_ERR_ALIASING"
    code = lib.gdn_step(ctypes.byref(p), *([vp(0x1000)] * 8), 0, None)
    assert gb.STATUS[code] == "GDN_ERR_BAD_SHAPE"                          # T != 1
    code = lib.gdn_backward(ctypes.byref(p), *([None] * 16), 0, None)
    assert gb.STATUS[code] == "GDN_ERR_NULL_POINTER"


def test_frame_larger_than_2gib_is_rejected(lib):
    # one frame's token rows must stay under 2 GiB (32-bit byte offsets)
    p = gb.make_problem(1, 2000, 1, 300000, 128, "fp32")
    assert gb.STATUS[_ws(p, gb.GDN_OP_FORWARD)[0]] == "GDN_ERR_BAD_SHAPE"
    p = gb.make_problem(1, 2000, 1, 2000, 128, "fp32")
    assert gb.STATUS[_ws(p, gb.GDN_OP_FORWARD)[0]] == "GDN_OK"


def test_algorithm_field(lib):
    vp = ctypes.c_void_p
    p = gb.make_problem(1, 2, 4, 8, 32, "bf16", algorithm="token")
    # chunks of 64 / 8 = 8 frames: one chunk per (b, h), each a record of
    # two 64 x 64 bf16 operators and 5 x 64 fp32 values
    assert _ws(p, gb.GDN_OP_FORWARD) == (0, 2 * 1 * (2 * 64 * 64 * 2 + 5 * 64 * 4))
    pf = gb.make_problem(2, 3, 10, 1, 32, "fp32", algorithm="token")   # 32 frames a chunk
    assert _ws(pf, gb.GDN_OP_FORWARD) == (0, 6 * 1 * (2 * 32 * 32 * 4 + 5 * 32 * 4))
    pl = gb.make_problem(1, 1, 130, 1, 32, "bf16", algorithm="token")  # 3 chunks
    assert _ws(pl, gb.GDN_OP_FORWARD)[1] == 3 * (2 * 64 * 64 * 2 + 5 * 64 * 4)
    n = ctypes.c_size_t(0)
    assert gb.STATUS[lib.gdn_saved_size(ctypes.byref(p), ctypes.byref(n))] == "GDN_ERR_UNSUPPORTED"
    # the backward is the frame form whatever the forward's algorithm
    assert _ws(p, gb.GDN_OP_BACKWARD)[1] == _ws(gb.make_problem(1, 2, 4, 8, 32, "bf16"),
                                                gb.GDN_OP_BACKWARD)[1]
    good = [vp(0x100000 * (i + 1)) for i in range(10)]
    # no saved buffer in the token form
    code = lib.gdn_forward(ctypes.byref(p), *good, 1 << 30, None)
    assert gb.STATUS[code] == "GDN_ERR_UNSUPPORTED"
    for io, nmax in (("bf16", 64), ("fp32", 32)):
        ok = gb.make_problem(1, 2, 3, nmax, 16, io, algorithm="token")
        assert _ws(ok, gb.GDN_OP_FORWARD)[0] == 0   # one frame a chunk
        big = gb.make_problem(1, 2, 3, nmax + 1, 16, io, algorithm="token")
        assert gb.STATUS[_ws(big, gb.GDN_OP_FORWARD)[0]] == "GDN_ERR_UNSUPPORTED"
        # the frame form takes any N
        assert _ws(gb.make_problem(1, 2, 3, nmax + 1, 16, io, algorithm="frame"),
                   gb.GDN_OP_FORWARD)[0] == 0
    bad = gb.make_problem(1, 2, 4, 8, 32, "bf16")
    bad.algorithm = 4
    assert gb.STATUS[_ws(bad, gb.GDN_OP_FORWARD)[0]] == "GDN_ERR_UNSUPPORTED"
    # auto may take the direct form, which falls back to the frame form when
    # a saved buffer is passed: its workspace is the frame form's
    auto = gb.make_problem(1, 2, 4, 1, 32, "bf16")
    assert _ws(auto, gb.GDN_OP_FORWARD) == _ws(gb.make_problem(1, 2, 4, 1, 32, "bf16",
                                                                 algorithm="frame"),
                                                 gb.GDN_OP_FORWARD)
    assert gb.STATUS[lib.gdn_saved_size(ctypes.byref(auto), ctypes.byref(n))] == "GDN_OK"


def test_direct_form_limits(lib):
    vp = ctypes.c_void_p
    n = ctypes.c_size_t(0)
    # bf16 only
    pf = gb.make_problem(1, 2, 4, 8, 32, "fp32", algorithm="direct")
    assert gb.STATUS[_ws(pf, gb.GDN_OP_FORWARD)[0]] == "GDN_ERR_UNSUPPORTED"
    p = gb.make_problem(1, 2, 4, 8, 32, "bf16", algorithm="direct")
    assert _ws(p, gb.GDN_OP_FORWARD)[0] == 0
    # no saved buffer
    assert gb.STATUS[lib.gdn_saved_size(ctypes.byref(p), ctypes.byref(n))] == "GDN_ERR_UNSUPPORTED"
    good = [vp(0x100000 * (i + 1)) for i in range(10)]
    code = lib.gdn_forward(ctypes.byref(p), *good, 1 << 30, None)
    assert gb.STATUS[code] == "GDN_ERR_UNSUPPORTED"
    # normalised rows: copies of q and k in the workspace
    pn = gb.make_problem(1, 2, 4, 8, 32, "bf16", algorithm="direct", flags=1)
    assert _ws(pn, gb.GDN_OP_FORWARD)[1] > _ws(p, gb.GDN_OP_FORWARD)[1]


def test_prologue_flags(lib):
    """The prologue's flags: unknown bits rejected; the gates from logits
    need fp32 copies of gamma and beta in the workspace; normalised rows
    need q / |q| and k / |k| copies where the kernels take them as input
    (the backward, the token form), not in the frame form's forward, which
    takes the norms from the rows it stages.  The bf16 backward of a launch
    long enough for its one-pass dO kernel takes the raw rows too and keeps
    only 1 / |q| per row; shorter launches and fp32 take the copies."""
    B, H, T, N, D = 1, 20, 121, 880, 112
    L = T * N
    mat = B * H * T * D * D * 2
    r256 = lambda n: (n + 255) // 256 * 256
    gates = r256(B * T * H * 4) + r256(B * L * H * 4)
    inv_q = r256(B * L * H * 4)
    for flags, fwd, bwd in ((gb.GDN_FLAG_NORMALIZE_QK, 0, inv_q),
                            (gb.GDN_FLAG_GATE_LOGITS, gates, gates),
                            (3, gates, gates + inv_q)):
        p = gb.make_problem(B, H, T, N, D, "bf16", flags=flags)
        assert _ws(p, gb.GDN_OP_FORWARD) == (0, 3 * mat + fwd)
        assert _ws(p, gb.GDN_OP_BACKWARD) == (0, 6 * mat + bwd)
    # 8 frames of 20 heads: 80 (frame, head pair) items, too few for the
    # one-pass dO kernel: copies of q and k
    # (beside the backward's own buffers and the Gram token-split partials
    # such a short launch takes)
    ps = gb.make_problem(B, H, 8, N, D, "bf16", flags=1)
    plain = _ws(gb.make_problem(B, H, 8, N, D, "bf16"), gb.GDN_OP_BACKWARD)[1]
    assert _ws(ps, gb.GDN_OP_BACKWARD) == (0, r256(plain) + 2 * r256(B * 8 * N * H * D * 2))
    pt = gb.make_problem(1, 2, 4, 8, 32, "bf16", algorithm="token", flags=3)
    base = 2 * (2 * 64 * 64 * 2 + 5 * 64 * 4)
    assert _ws(pt, gb.GDN_OP_FORWARD) == (
        0, r256(base) + r256(4 * 2 * 4) + r256(32 * 2 * 4) + 2 * r256(32 * 2 * 32 * 2))
    for bit in (4, 1 << 30, -1):
        bad = gb.make_problem(1, 2, 4, 8, 32, "bf16")
        bad.flags = bit
        assert gb.STATUS[_ws(bad, gb.GDN_OP_FORWARD)[0]] == "GDN_ERR_UNSUPPORTED"
    assert gb.flags_of(True, False) == 1 and gb.flags_of(False, True) == 2


def _cpu_inputs(B, H, T, N, D, dt):
    import torch
    L = T * N
    return dict(q=torch.zeros((B, L, H, D), dtype=dt), k=torch.zeros((B, L, H, D), dtype=dt),
                v=torch.zeros((B, L, H, D), dtype=dt),
                gamma=torch.zeros((B, T, H), dtype=torch.float32),
                beta=torch.zeros((B, L, H), dtype=torch.float32))


def _mismatches(x, state_name):
    """(argument overrides, expected exception) pairs, each one tensor wrong."""
    import torch
    q = x["q"]
    B, L, H, D = q.shape
    st = torch.zeros((B, H, D, D), dtype=torch.float32)
    return [
        ({"q": q.to(torch.float16)}, TypeError),                      # dtype
        ({"k": x["k"][:, :-1]}, ValueError),                          # short rows
        ({"v": x["v"].transpose(1, 2).contiguous().transpose(1, 2)}, ValueError),  # layout
        ({"gamma": x["gamma"].double()}, TypeError),
        ({"beta": x["beta"][..., :-1]}, ValueError),
        ({state_name: st.to(torch.bfloat16)}, TypeError),             # bf16 state
        ({state_name: st[:, :, :-1]}, ValueError),                    # wrong-sized state
        ({state_name: st.transpose(2, 3)}, ValueError),               # non-contiguous state
    ]


def test_forward_plan_checks_every_tensor(lib):
    # a mismatch in any tensor raises before the library is called
    import torch
    B, H, T, N, D = 1, 2, 3, 5, 16
    plan = gb.ForwardPlan(B, H, T, N, D, "bf16", "cpu")
    x = _cpu_inputs(B, H, T, N, D, torch.bfloat16)
    x["state_in"] = None
    for over, exc in _mismatches(x, "state_in"):
        args = dict(x, **over)
        with pytest.raises(exc):
            plan(**args)
    with pytest.raises(ValueError):
        plan(**dict(x, state_out=torch.zeros((B, H, D, D + 1))))


def test_step_plan_checks_every_tensor(lib):
    import torch
    B, H, N, D = 1, 2, 5, 16
    plan = gb.StepPlan(B, H, N, D, "bf16", "cpu")
    x = _cpu_inputs(B, H, 1, N, D, torch.bfloat16)
    x["state"] = torch.zeros((B, H, D, D), dtype=torch.float32)
    for over, exc in _mismatches(x, "state"):
        with pytest.raises(exc):
            plan(**dict(x, **over))
    with pytest.raises(ValueError):      # gamma of two frames
        plan(**dict(x, gamma=torch.zeros((B, 2, H))))


def test_poisoned_buffers_are_nan(lib):
    import torch
    old = gb.POISON
    gb.POISON = True
    try:
        plan = gb.ForwardPlan(1, 2, 3, 5, 16, "bf16", "cpu", saved=True)
        assert torch.isnan(plan.o.float()).all() and torch.isnan(plan.state_out).all()
        assert bool((plan.ws == 255).all()) and bool((plan.saved == 255).all())
    finally:
        gb.POISON = old


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    # the static scratch holds the one-minute shape's forward workspace, with
    # the prologue; one more frame of fp32 io does not fit, and the call
    # returns before any GPU work
    ok = gb.make_problem(1, 20, 121, 880, 112, "bf16", flags=3)
    assert _ws(ok, gb.GDN_OP_FORWARD)[1] <= gb.NOALLOC_SCRATCH_BYTES
    big = gb.make_problem(1, 20, 121, 880, 112, "fp32")
    assert _ws(big, gb.GDN_OP_FORWARD)[1] > gb.NOALLOC_SCRATCH_BYTES
    z = ctypes.c_void_p(16)
    code = lib.gdn_forward_noalloc(ctypes.byref(big), z, z, z, z, z, None, z, None, None, None)
    assert gb.STATUS[code] == "GDN_ERR_SCRATCH_TOO_SMALL"
    bad = gb.make_problem(1, 20, 121, 880, 100, "bf16")
    code = lib.gdn_forward_noalloc(ctypes.byref(bad), z, z, z, z, z, None, z, None, None, None)
    assert gb.STATUS[code] == "GDN_ERR_UNSUPPORTED"
