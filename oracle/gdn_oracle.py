"""Float64 CPU oracle of the frame-wise Gated DeltaNet (GDN) recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constant tables); both sides receive
the same seeded inputs and nothing else.

What it computes, and where it comes from
-----------------------------------------
The method is defined on the paper.rainbus.top summary of "SANA-WM: Efficient
Minute-Scale World Modeling with Hybrid Linear Diffusion Transformer":

* section 前置知识, "Gated DeltaNet (GDN)": a D x D state S_t per head with a
  decay gate gamma_t and a delta-rule correction, updated as
  S_t = S_{t-1} M_t + U_t;
* section 方法步骤详情, module 2 ("Memory-Efficient Long-Context"): the scan
  runs once per latent frame with
      M_t = gamma_t I - K^_t beta_t K^_t^T,   U_t = V_t beta_t K^_t^T,
      O_t = S_t Q^_t,
  and keys are scaled by 1/sqrt(D S) (the sentence is cut off after that);
* section 技术新颖性, point 1: this is token-wise GDN generalised to one update
  per whole latent frame; the key scaling keeps ||M_t||_2 <= gamma_t <= 1; for
  context-parallel training a transition composite C_p and an input composite
  H_p are combined by a prefix sum that reproduces the single-device result
  exactly.

Notation (the pages' column form): K^_t, Q^_t are Dk x N (one column per
token of frame t), V_t and O_t are Dv x N, beta_t is the N x N diagonal of the
per-token gates, gamma_t is one scalar per frame and head, S is Dv x Dk.

Readings of what the pages leave open (each also listed in the design notes):

* D in 1/sqrt(D S) is the key head dimension Dk and S the number of tokens per
  frame N, so the default key scale is 1/sqrt(Dk * N);
* keys and queries arrive already normalised: the oracle applies only the key
  scale, never a normalisation (the hats are read as "normalised upstream");
* the decay multiplies only the identity, literally gamma_t I - K^ beta K^^T;
* the output of frame t uses S_t, the state after frame t's own update;
* S_0 = 0 unless an initial state is given;
* ``erase`` is a test-only switch (M_t = gamma_t I - erase * A_t) used to pin
  the oracle against gated linear attention; the library has no such switch.

Array layout (shared with the library's interface): q, k: [B, L, H, Dk];
v, o: [B, L, H, Dv]; gamma: [B, T, H]; beta: [B, L, H]; states:
[B, H, Dv, Dk]; token l = t * N + n (frame-major).  All arithmetic is float64.

Parity is pinned for every function here by the tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, invariants, finite
differences); none of them is "parity unpinned".
"""

import numpy as np

__all__ = [
    "default_key_scale",
    "frame_terms",
    "forward",
    "step",
    "backward",
    "composite_forward",
    "tokenspace_forward",
    "prologue",
    "prologue_backward",
]


def default_key_scale(dk, n):
    """Key scale 1/sqrt(D*S) of the GDN recurrence (summary page, 方法步骤详情
    module 2, and 技术新颖性 point 1), read with D = Dk and S = N."""
    return 1.0 / np.sqrt(float(dk) * float(n))


def _scale(key_scale, dk, n):
    return float(key_scale) if key_scale else default_key_scale(dk, n)


def _shapes(q, k, v, gamma, beta, n):
    B, L, H, Dk = k.shape
    Dv = v.shape[-1]
    if L % n:
        raise ValueError("sequence length %d is not a whole number of frames of %d" % (L, n))
    T = L // n
    if q.shape != (B, L, H, Dk) or v.shape[:3] != (B, L, H):
        raise ValueError("q/k/v shapes disagree")
    if gamma.shape != (B, T, H) or beta.shape != (B, L, H):
        raise ValueError("gate shapes disagree")
    return B, L, H, Dk, Dv, T


def _frame_cols(x, b, t, h, n):
    """Columns of one frame for one head: x[b, t*N:(t+1)*N, h, :] as D x N."""
    return np.asarray(x[b, t * n:(t + 1) * n, h, :], dtype=np.float64).T


def frame_terms(k, v, beta, n, key_scale=0.0):
    """Per-frame Gram A_t = K^_t beta_t K^_t^T and write U_t = V_t beta_t K^_t^T
    (summary page, 方法步骤详情 module 2).

    Returns A [B, H, T, Dk, Dk] and U [B, H, T, Dv, Dk], float64.
    """
    B, L, H, Dk = k.shape
    Dv = v.shape[-1]
    T = L // n
    s = _scale(key_scale, Dk, n)
    A = np.zeros((B, H, T, Dk, Dk))
    U = np.zeros((B, H, T, Dv, Dk))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                Kh = s * _frame_cols(k, b, t, h, n)          # K^_t, Dk x N
                Vt = _frame_cols(v, b, t, h, n)              # V_t,  Dv x N
                bt = np.asarray(beta[b, t * n:(t + 1) * n, h], dtype=np.float64)
                # X diag(beta) scales column j of X by beta_j.
                A[b, h, t] = (Kh * bt) @ Kh.T
                U[b, h, t] = (Vt * bt) @ Kh.T
    return A, U


def prologue(q, k, gamma, beta, normalize_qk=False, gate_logits=False):
    """Optional prologue of the GDN block, applied before the recurrence.

    The hats on Q^ and K^ (summary page, 方法步骤详情 module 2) are read as
    per-token normalisation; with ``normalize_qk`` every query and key row
    (one token, one head) is divided by its L2 norm over the head dimension
    (the key scale is applied afterwards, as without the prologue).  With
    ``gate_logits`` gamma and beta arrive as logits and become sigmoid(x),
    the (0, 1) gates the recurrence uses.  Returns (q, k, gamma, beta).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if normalize_qk:
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    if gate_logits:
        gamma = 1.0 / (1.0 + np.exp(-gamma))
        beta = 1.0 / (1.0 + np.exp(-beta))
    return q, k, gamma, beta


def prologue_backward(q, k, gamma, beta, dq, dk, dgamma, dbeta, normalize_qk=False,
                      gate_logits=False):
    """Chain rule through ``prologue``: gradients with respect to the raw
    inputs from those with respect to the prologue's outputs.  For
    x^ = x / |x|: dx = (dx^ - x^ (x^ . dx^)) / |x|; for p = sigmoid(z):
    dz = dp p (1 - p).  Returns (dq, dk, dgamma, dbeta)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if normalize_qk:
        out = []
        for x, dx in ((q, dq), (k, dk)):
            nrm = np.linalg.norm(x, axis=-1, keepdims=True)
            xh = x / nrm
            out.append((dx - xh * np.sum(xh * dx, axis=-1, keepdims=True)) / nrm)
        dq, dk = out
    if gate_logits:
        pg = 1.0 / (1.0 + np.exp(-np.asarray(gamma, dtype=np.float64)))
        pb = 1.0 / (1.0 + np.exp(-np.asarray(beta, dtype=np.float64)))
        dgamma = dgamma * pg * (1.0 - pg)
        dbeta = dbeta * pb * (1.0 - pb)
    return dq, dk, dgamma, dbeta


def forward(q, k, v, gamma, beta, n, state_in=None, key_scale=0.0, erase=1.0,
            keep=False, normalize_qk=False, gate_logits=False):
    """Whole-sequence frame-wise GDN.

    For every (batch, head), in frame order t = 1..T:
        M_t = gamma_t I - erase * K^_t beta_t K^_t^T
        U_t = V_t beta_t K^_t^T
        S_t = S_{t-1} M_t + U_t
        O_t = S_t Q^_t
    (summary page: 前置知识 "Gated DeltaNet" for S_t = S_{t-1} M_t + U_t, and
    方法步骤详情 module 2 for M_t, U_t, O_t and the key scale).

    Returns (o [B, L, H, Dv], state_out [B, H, Dv, Dk]); with keep=True also a
    dict of the per-frame intermediates A_t, U_t, S_t ([B, H, T, D, D]).
    ``normalize_qk`` / ``gate_logits`` run ``prologue`` first.
    """
    if normalize_qk or gate_logits:
        q, k, gamma, beta = prologue(q, k, gamma, beta, normalize_qk, gate_logits)
    B, L, H, Dk, Dv, T = _shapes(q, k, v, gamma, beta, n)
    s = _scale(key_scale, Dk, n)
    o = np.zeros((B, L, H, Dv))
    state_out = np.zeros((B, H, Dv, Dk))
    if keep:
        kept = {"A": np.zeros((B, H, T, Dk, Dk)), "U": np.zeros((B, H, T, Dv, Dk)),
                "S": np.zeros((B, H, T, Dv, Dk))}
    eye = np.eye(Dk)
    for b in range(B):
        for h in range(H):
            S = (np.zeros((Dv, Dk)) if state_in is None
                 else np.asarray(state_in[b, h], dtype=np.float64).copy())
            for t in range(T):
                Kh = s * _frame_cols(k, b, t, h, n)
                Qh = _frame_cols(q, b, t, h, n)
                Vt = _frame_cols(v, b, t, h, n)
                bt = np.asarray(beta[b, t * n:(t + 1) * n, h], dtype=np.float64)
                A = (Kh * bt) @ Kh.T
                U = (Vt * bt) @ Kh.T
                M = float(gamma[b, t, h]) * eye - erase * A
                S = S @ M + U
                o[b, t * n:(t + 1) * n, h, :] = (S @ Qh).T
                if keep:
                    kept["A"][b, h, t] = A
                    kept["U"][b, h, t] = U
                    kept["S"][b, h, t] = S
            state_out[b, h] = S
    if keep:
        return o, state_out, kept
    return o, state_out


def step(q, k, v, gamma, beta, state, key_scale=0.0, normalize_qk=False, gate_logits=False):
    """Streaming step: advance the carried state by one latent frame.

    The autoregressive / streaming variant carries the GDN state across calls
    (CSDN explainer section 六 stage 4; summary page limitations). One call is
    the forward recurrence with T = 1 starting from ``state``: q, k, v are
    [B, N, H, D], gamma [B, 1, H], beta [B, N, H].  Returns (o, new_state).
    """
    n = k.shape[1]
    return forward(q, k, v, gamma, beta, n, state_in=state, key_scale=key_scale,
                   normalize_qk=normalize_qk, gate_logits=gate_logits)


def backward(q, k, v, gamma, beta, n, d_o, state_in=None, d_state_out=None,
             key_scale=0.0, erase=1.0, normalize_qk=False, gate_logits=False):
    """Reverse-mode gradients of ``forward`` (the pages give no backward; this
    is the chain rule applied to the module-2 recurrence, step by step).

    With G_t = dL/dS_t (all paths through S_t):
        G_T      = dO_T Q^_T^T + dS_T(external)
        G_t      = dO_t Q^_t^T + G_{t+1} M_{t+1}^T
        dQ^_t    = S_t^T dO_t
        dM_t     = S_{t-1}^T G_t,    dgamma_t = tr(dM_t),   dA_t = -erase dM_t
        dV_t     = G_t K^_t beta_t
        dK^_t    = G_t^T V_t beta_t + (dA_t + dA_t^T) K^_t beta_t
        dbeta_tn = v_tn^T G_t k^_tn + k^_tn^T dA_t k^_tn
        dK_t     = s dK^_t              (K^ = s K)
        dS_0     = G_1 M_1^T
    Returns dict with dq, dk, dv ([B, L, H, D]), dgamma [B, T, H],
    dbeta [B, L, H], dstate_in [B, H, Dv, Dk].  With ``normalize_qk`` /
    ``gate_logits`` the gradients are with respect to the raw inputs of
    ``prologue`` (``prologue_backward``).
    """
    if normalize_qk or gate_logits:
        qp, kp, gp, bp = prologue(q, k, gamma, beta, normalize_qk, gate_logits)
        gr = backward(qp, kp, v, gp, bp, n, d_o, state_in=state_in, d_state_out=d_state_out,
                      key_scale=key_scale, erase=erase)
        gr["dq"], gr["dk"], gr["dgamma"], gr["dbeta"] = prologue_backward(
            q, k, gamma, beta, gr["dq"], gr["dk"], gr["dgamma"], gr["dbeta"], normalize_qk,
            gate_logits)
        return gr
    B, L, H, Dk, Dv, T = _shapes(q, k, v, gamma, beta, n)
    s = _scale(key_scale, Dk, n)
    dq = np.zeros((B, L, H, Dk))
    dk = np.zeros((B, L, H, Dk))
    dv = np.zeros((B, L, H, Dv))
    dgamma = np.zeros((B, T, H))
    dbeta = np.zeros((B, L, H))
    dstate_in = np.zeros((B, H, Dv, Dk))
    eye = np.eye(Dk)
    for b in range(B):
        for h in range(H):
            # Forward sweep, keeping every state and transition.
            S = (np.zeros((Dv, Dk)) if state_in is None
                 else np.asarray(state_in[b, h], dtype=np.float64).copy())
            states = [S]
            trans = []
            for t in range(T):
                Kh = s * _frame_cols(k, b, t, h, n)
                Vt = _frame_cols(v, b, t, h, n)
                bt = np.asarray(beta[b, t * n:(t + 1) * n, h], dtype=np.float64)
                M = float(gamma[b, t, h]) * eye - erase * ((Kh * bt) @ Kh.T)
                S = S @ M + (Vt * bt) @ Kh.T
                states.append(S)
                trans.append(M)
            # Reverse sweep.
            carry = (np.zeros((Dv, Dk)) if d_state_out is None
                     else np.asarray(d_state_out[b, h], dtype=np.float64).copy())
            for t in reversed(range(T)):
                sl = slice(t * n, (t + 1) * n)
                Kh = s * _frame_cols(k, b, t, h, n)
                Qh = _frame_cols(q, b, t, h, n)
                Vt = _frame_cols(v, b, t, h, n)
                dOt = _frame_cols(d_o, b, t, h, n)
                bt = np.asarray(beta[b, sl, h], dtype=np.float64)
                S_prev, S_t, M = states[t], states[t + 1], trans[t]
                G = dOt @ Qh.T + carry                       # dL/dS_t
                dq[b, sl, h, :] = (S_t.T @ dOt).T
                dM = S_prev.T @ G
                dgamma[b, t, h] = np.trace(dM)
                dA = -erase * dM
                dv[b, sl, h, :] = ((G @ Kh) * bt).T
                dKh = (G.T @ Vt) * bt + ((dA + dA.T) @ Kh) * bt
                dk[b, sl, h, :] = (s * dKh).T
                # dbeta_tn = v_tn^T G_t k^_tn + k^_tn^T dA_t k^_tn, one column
                # (token) at a time: the column sums of V * (G K^) and K^ * (dA K^)
                dbeta[b, sl, h] = (np.sum(Vt * (G @ Kh), axis=0)
                                   + np.sum(Kh * (dA @ Kh), axis=0))
                carry = G @ M.T
            dstate_in[b, h] = carry
    return {"dq": dq, "dk": dk, "dv": dv, "dgamma": dgamma, "dbeta": dbeta,
            "dstate_in": dstate_in}


def composite_forward(q, k, v, gamma, beta, n, chunk, state_in=None,
                      key_scale=0.0, erase=1.0):
    """Forward through the transition / input composites of the context-
    parallel scheme (summary page, 技术新颖性 point 1).

    Frames are cut into consecutive chunks of ``chunk`` frames (the last one
    may be shorter), standing in for the devices of context parallelism.
    Each chunk p first builds, independently of every other chunk,
        C_p = M_{first} ... M_{last}                 (transition composite)
        H_p : H <- H M_t + U_t from H = 0           (input composite)
    so that S_out(p) = S_in(p) C_p + H_p.  A prefix over the chunks then gives
    every chunk's incoming state, S_in(p) = S_out(p-1), and each chunk replays
    its frames from that state to produce its outputs.

    Returns (o, state_out) like ``forward``.
    """
    B, L, H, Dk, Dv, T = _shapes(q, k, v, gamma, beta, n)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    s = _scale(key_scale, Dk, n)
    eye = np.eye(Dk)
    o = np.zeros((B, L, H, Dv))
    state_out = np.zeros((B, H, Dv, Dk))
    bounds = [(c, min(c + chunk, T)) for c in range(0, T, chunk)]
    for b in range(B):
        for h in range(H):
            Ms, Us = [], []
            for t in range(T):
                Kh = s * _frame_cols(k, b, t, h, n)
                Vt = _frame_cols(v, b, t, h, n)
                bt = np.asarray(beta[b, t * n:(t + 1) * n, h], dtype=np.float64)
                Ms.append(float(gamma[b, t, h]) * eye - erase * ((Kh * bt) @ Kh.T))
                Us.append((Vt * bt) @ Kh.T)
            # Per-chunk composites (independent across chunks).
            comps = []
            for (t0, t1) in bounds:
                C = eye.copy()
                Hc = np.zeros((Dv, Dk))
                for t in range(t0, t1):
                    C = C @ Ms[t]
                    Hc = Hc @ Ms[t] + Us[t]
                comps.append((C, Hc))
            # Prefix over chunks: incoming state of every chunk.
            S = (np.zeros((Dv, Dk)) if state_in is None
                 else np.asarray(state_in[b, h], dtype=np.float64).copy())
            incoming = []
            for (C, Hc) in comps:
                incoming.append(S)
                S = S @ C + Hc
            state_out[b, h] = S
            # Each chunk replays its frames from its incoming state.
            for (t0, t1), S_in in zip(bounds, incoming):
                St = S_in
                for t in range(t0, t1):
                    St = St @ Ms[t] + Us[t]
                    o[b, t * n:(t + 1) * n, h, :] = (St @ _frame_cols(q, b, t, h, n)).T
    return o, state_out


def tokenspace_forward(q, k, v, gamma, beta, n, frames_per_chunk, state_in=None,
                       key_scale=0.0):
    """Forward in token space, chunk by chunk, with the per-chunk triangular
    system of the delta rule.

    This is the same recurrence as ``forward`` (summary page, 前置知识 "Gated
    DeltaNet" and 方法步骤详情 module 2) written over the tokens of a chunk of
    F = ``frames_per_chunk`` consecutive frames instead of over D x D
    matrices; 技术新颖性 point 1 describes frame-wise GDN as token-wise GDN
    generalised to whole frames, and this is the token-wise algorithm with
    frames as its steps.  It needs no D x D product per frame, which is what
    makes it cheaper when a frame has fewer tokens than D.

    Derivation (column form; E_f = state entering frame f of the chunk,
    E_0 = the chunk's incoming state): each frame's update
        S = S (gamma_f I - K^_f beta_f K^_f^T) + V_f beta_f K^_f^T
          = gamma_f S + W_f K^_f^T,   W_f = (V_f - S K^_f) beta_f,
    so with P(a, b) = gamma_a ... gamma_b (1 when a > b), for token t of
    frame f(t):
        E_f     = P(0, f-1) E_0 + sum_{u: f(u) < f} P(f(u)+1, f-1) w_u k^_u^T
        w_t     = (v_t - E_{f(t)} k^_t) beta_t
    i.e. W (I + L) = R with
        R[:, t] = (v_t - P(0, f(t)-1) E_0 k^_t) beta_t
        L[u, t] = P(f(u)+1, f(t)-1) (k^_u . k^_t) beta_t   for f(u) < f(t), else 0
    (strictly upper triangular in token order: tokens of one frame do not
    see each other).  Then
        o_t     = P(0, f(t)) E_0 q_t + sum_{u: f(u) <= f(t)} P(f(u)+1, f(t)) w_u (k^_u . q_t)
        E_F     = P(0, F-1) E_0 + sum_u P(f(u)+1, F-1) w_u k^_u^T.
    The triangular solve is a library routine (numpy's solve on the unit
    triangular matrix).

    Returns (o, state_out) like ``forward``.
    """
    B, L, H, Dk, Dv, T = _shapes(q, k, v, gamma, beta, n)
    F = int(frames_per_chunk)
    if F < 1:
        raise ValueError("frames_per_chunk must be >= 1")
    s = _scale(key_scale, Dk, n)
    o = np.zeros((B, L, H, Dv))
    state_out = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            E0 = (np.zeros((Dv, Dk)) if state_in is None
                  else np.asarray(state_in[b, h], dtype=np.float64).copy())
            for t0 in range(0, T, F):
                t1 = min(t0 + F, T)
                nf = t1 - t0
                C = nf * n
                sl = slice(t0 * n, t1 * n)
                Kc = s * np.asarray(k[b, sl, h, :], dtype=np.float64).T     # Dk x C
                Qc = np.asarray(q[b, sl, h, :], dtype=np.float64).T         # Dk x C
                Vc = np.asarray(v[b, sl, h, :], dtype=np.float64).T         # Dv x C
                bc = np.asarray(beta[b, sl, h], dtype=np.float64)           # C
                g = np.asarray(gamma[b, t0:t1, h], dtype=np.float64)        # nf
                fr = np.repeat(np.arange(nf), n)                            # frame of each token

                def P(a, c):
                    return float(np.prod(g[a:c + 1])) if a <= c else 1.0

                Pd = np.array([[P(a + 1, c - 1) for c in range(nf)] for a in range(nf)])
                Po = np.array([[P(a + 1, c) for c in range(nf)] for a in range(nf)])
                before = np.array([P(0, f - 1) for f in range(nf)])         # P(0, f-1)
                upto = np.array([P(0, f) for f in range(nf)])               # P(0, f)
                tail = np.array([P(f + 1, nf - 1) for f in range(nf)])      # P(f+1, F-1)
                KK = Kc.T @ Kc                                              # k^_u . k^_t
                KQ = Kc.T @ Qc                                              # k^_u . q_t
                earlier = fr[:, None] < fr[None, :]
                Lm = np.where(earlier, Pd[fr][:, fr] * KK, 0.0) * bc[None, :]
                R = (Vc - (E0 @ Kc) * before[fr][None, :]) * bc[None, :]
                # W (I + L) = R  <=>  (I + L)^T W^T = R^T
                W = np.linalg.solve((np.eye(C) + Lm).T, R.T).T              # Dv x C
                seen = fr[:, None] <= fr[None, :]
                Om = np.where(seen, Po[fr][:, fr] * KQ, 0.0)
                Oc = (E0 @ Qc) * upto[fr][None, :] + W @ Om
                o[b, sl, h, :] = Oc.T
                E0 = P(0, nf - 1) * E0 + (W * tail[fr][None, :]) @ Kc.T
            state_out[b, h] = E0
    return o, state_out
