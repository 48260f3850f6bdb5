"""CPU emulation of the token form's state pass (token_scan_kernel, fp32 io,
D = 16: one wave) chunk by chunk, with the kernel's own LDS layouts and index
arithmetic, lane by lane, and the fp32 MFMA 16x16x4 lane layout the kernels
rely on (A[m][k] in lane (k, m), B[k][n] in lane (k, n), C[4g + r][n] in
lane (g, n) register r).

Every LDS access runs in program order, as one wave's LDS operations
complete in order on the hardware.  So this checks the chunk body as written
- the reuse of a wave's staged rows Zw (state rows in step 1, R in step 3, W
and W tail in step 4), the transposed operator records, the decay vector -
against the oracle, independently of instruction timing: if it agrees, a
miscompare of a build whose source is unchanged lies in the timing of the
instructions (a missing wait or hazard), not in the data flow.

The chunk records (the inverse (I + L)^-1, the output mixing Om and the
per-token decays) are built here from their definitions on the summary
page's recurrence (方法步骤详情 module 2, as the token form restates it per
chunk of F frames): with P(a, b) the product of the gates of frames a..b,
L[u, t] = P(f(u)+1, f(t)-1) (k^_u . k^_t) beta_t for f(u) < f(t),
Om[u, t] = P(f(u)+1, f(t)) (k^_u . q_t) for f(u) <= f(t).
"""

import numpy as np
import pytest

import oracle

CP = 32          # tokens per chunk at most (fp32)
D = 16           # one wave
KS = 4           # fp32 MFMA contraction depth
NB = CP // 16
KLD = D + 4      # K, Q rows in LDS (DP + PAD)
TLD = CP + 4     # operator rows
ZLD = max(D, 2 * CP) + 4
LANES = np.arange(64)
G, LI = LANES // 16, LANES % 16


def mfma(a, b, c):
    """v_mfma_f32_16x16x4_f32: a, b per-lane values [64]; c, result [64, 4]."""
    A = np.zeros((16, 4))
    B = np.zeros((4, 16))
    A[LI, G] = a
    B[G, LI] = b
    C = A @ B
    out = c.copy()
    for r in range(4):
        out[:, r] += C[4 * G + r, LI]
    return out


def frag_a(M, ld, m0, k0):
    """fragA(M, ld, m0, k0): lane (g, i) reads M[(m0 + i) ld + k0 + g]."""
    return M[(m0 + LI) * ld + k0 + G]


def frag_bn(M, ld, k0, n0):
    """fragBn(M, ld, k0, n0): lane (g, i) reads M[(k0 + g) ld + n0 + i]."""
    return M[(k0 + G) * ld + n0 + LI]


def chunk_records(k, q, beta, gam, N, F, s):
    """TiT, OmT (row t holds column t of (I + L)^-1, of Om) and the vector
    [before | upto | tail | beta | total] of one chunk of F frames."""
    C = F * N
    f = np.arange(CP) // N
    P = lambda a, b: np.prod(gam[a:b + 1]) if a <= b else 1.0
    kh = s * k
    Lm = np.zeros((CP, CP))
    Om = np.zeros((CP, CP))
    for u in range(C):
        for t in range(C):
            if f[u] < f[t]:
                Lm[u, t] = P(f[u] + 1, f[t] - 1) * (kh[u] @ kh[t]) * beta[t]
            if f[u] <= f[t]:
                Om[u, t] = P(f[u] + 1, f[t]) * (kh[u] @ q[t])
    Tinv = np.linalg.inv(np.eye(CP) + Lm)
    vec = np.zeros(5 * CP)
    for t in range(C):
        vec[t] = P(0, f[t] - 1)
        vec[CP + t] = P(0, f[t])
        vec[2 * CP + t] = P(f[t] + 1, F - 1)
        vec[3 * CP + t] = beta[t]
    vec[4 * CP] = P(0, F - 1)
    TiT = np.zeros(CP * TLD)
    OmT = np.zeros(CP * TLD)
    for t in range(CP):
        TiT[t * TLD:t * TLD + CP] = Tinv[:, t]
        OmT[t * TLD:t * TLD + CP] = Om[:, t]
    return TiT, OmT, vec


def emulate_state_pass(k, q, v, beta, gam, N, F, s, S0):
    """One (b, h) sequence through the kernel's chunk body; returns o [L, D]
    and the final state."""
    L = k.shape[0]
    T = L // N
    nck = (T + F - 1) // F
    Sreg = np.zeros((64, 4))               # Sreg[0]: S[4g + r][i]
    Sreg[:, :] = S0[4 * G[:, None] + np.arange(4)[None, :], LI[:, None]]
    o = np.zeros((L, D))
    Ks = np.zeros(CP * KLD)
    Qs = np.zeros(CP * KLD)
    Zw = np.zeros(16 * ZLD)
    for ck in range(nck):
        t0 = ck * F
        Fc = min(F, T - t0)
        C = Fc * N
        tok = slice(t0 * N, t0 * N + C)
        TiT, OmT, vec = chunk_records(k[tok], q[tok], beta[tok], gam[t0:t0 + Fc], N, Fc, s)
        # 1. inputs into LDS (rows past the chunk stay zero), the state rows staged
        Ks[:] = 0.0
        Qs[:] = 0.0
        for u in range(C):
            Ks[u * KLD:u * KLD + D] = k[t0 * N + u]
            Qs[u * KLD:u * KLD + D] = q[t0 * N + u]
        for r in range(4):
            Zw[(4 * G + r) * ZLD + LI] = Sreg[:, r]
        # 2. SK = E_0 K^T, SQ = E_0 Q^T
        af = [frag_a(Zw, ZLD, 0, kb * KS) for kb in range(D // KS)]
        SK, SQ = [], []
        for j in range(NB):
            sk = np.zeros((64, 4))
            sq = np.zeros((64, 4))
            for kb in range(D // KS):
                sk = mfma(af[kb], frag_a(Ks, KLD, 16 * j, kb * KS), sk)
                sq = mfma(af[kb], frag_a(Qs, KLD, 16 * j, kb * KS), sq)
            SK.append(sk)
            SQ.append(sq)
        # 3. R staged over the state rows (columns 0 .. CP-1), W = R (I + L)^-1
        for j in range(NB):
            t = 16 * j + LI
            tt = np.minimum(t, C - 1)
            # this lane's values of token t at features 4g .. 4g + 3 (zero past the chunk)
            vv = np.stack([np.where(t < C, v[t0 * N + tt, 4 * G + r], 0.0) for r in range(4)],
                          axis=1)
            before, bt = vec[t], vec[3 * CP + t]
            for r in range(4):
                Zw[(4 * G + r) * ZLD + t] = (vv[:, r] - s * before * SK[j][:, r]) * bt
        rf = [frag_a(Zw, ZLD, 0, kb * KS) for kb in range(CP // KS)]
        Wr = []
        for j in range(NB):
            acc = np.zeros((64, 4))
            for kb in range(CP // KS):
                acc = mfma(rf[kb], frag_a(TiT, TLD, 16 * j, kb * KS), acc)
            Wr.append(acc)
        # 4. W and W tail staged; O = P(0, f) SQ + W Om
        for j in range(NB):
            t = 16 * j + LI
            tail = vec[2 * CP + t]
            for r in range(4):
                Zw[(4 * G + r) * ZLD + t] = Wr[j][:, r]
                Zw[(4 * G + r) * ZLD + CP + t] = Wr[j][:, r] * tail
        wf = [frag_a(Zw, ZLD, 0, kb * KS) for kb in range(CP // KS)]
        for j in range(NB):
            acc = np.zeros((64, 4))
            for kb in range(CP // KS):
                acc = mfma(wf[kb], frag_a(OmT, TLD, 16 * j, kb * KS), acc)
            t = 16 * j + LI
            upto = vec[CP + t]
            for lane in range(64):
                if t[lane] < C:
                    for r in range(4):
                        o[t0 * N + t[lane], 4 * G[lane] + r] = (
                            upto[lane] * SQ[j][lane, r] + acc[lane, r])
        # 5. E_F = P(0, F-1) E_0 + s (W tail) K
        total = vec[4 * CP]
        acc = np.zeros((64, 4))
        for kb in range(CP // KS):
            acc = mfma(frag_a(Zw[CP:], ZLD, 0, kb * KS), frag_bn(Ks, KLD, kb * KS, 0), acc)
        Sreg = total * Sreg + s * acc
    S = np.zeros((D, D))
    for r in range(4):
        S[4 * G + r, LI] = Sreg[:, r]
    return o, S


@pytest.mark.parametrize("N,T", [(1, 70), (3, 25), (5, 13), (32, 3)])
def test_token_chunk_body_matches_oracle(N, T):
    rng = np.random.default_rng(50 + N)
    L = T * N
    k = rng.standard_normal((L, D))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((L, D))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((L, D))
    beta = rng.uniform(0.05, 1.0, L)
    gam = rng.uniform(0.5, 1.0, T)
    S0 = 0.3 * rng.standard_normal((D, D))
    s = 0.6                               # the delta correction well above rounding
    F = CP // N                           # frames per chunk, as the library takes them
    o, S = emulate_state_pass(k, q, v, beta, gam, N, F, s, S0)
    ro, rs = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                            gam[None, :, None], beta[None, :, None], N, state_in=S0[None, None],
                            key_scale=s)
    assert np.max(np.abs(o - ro[0, :, 0])) < 1e-10 * max(1.0, np.max(np.abs(ro)))
    assert np.max(np.abs(S - rs[0, 0])) < 1e-10 * max(1.0, np.max(np.abs(rs)))
