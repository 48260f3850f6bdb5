"""Seeded synthetic inputs for the frame-wise GDN token mixer.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and distributions of the workloads, so that the library and
the oracle can be fed the very same values.

Shapes come from the SANA-WM pages: a 20-head DiT with model width 2240
(head dim 112), one minute of video at 16 fps (961 raw frames) compressed 8x
in time by the VAE (121 latent frames), and 22 x 40 = 880 latent tokens per
frame at 720p.

Draw order (numpy ``Generator(PCG64(seed))``, float32): Q, K, V, gamma, beta,
then dO, dS_T and S_0 when asked for.  Q and K are L2-normalised per
(token, head) over the head dimension in float32, then every io tensor is
cast to the io dtype (bf16 round-to-nearest-even through torch).  Gates and
states stay float32.

``raw=True`` draws the inputs of the block's prologue instead: Q and K rows
are not normalised but multiplied by per-row factors exp(N(0, 1)) (drawn
after beta, Q's then K's), and gamma, beta are the logits themselves:
gamma ~ N(3, 0.5), beta ~ N(0, 1).
"""

import numpy as np
import torch

# name -> shape / distribution recipe
CONFIGS = {
    # tiny oracle check: fp32 io, gamma = sigmoid(N(3, 0.5)) per head-frame
    "tiny": dict(B=1, H=2, D=16, T=8, N=4, io="fp32", gamma="sigmoid"),
    # one GDN layer, short clip (21 latent frames), bf16 io
    "short": dict(B=1, H=20, D=112, T=21, N=880, io="bf16", gamma="uniform"),
    # one GDN layer at the one-minute 720p shape (121 x 880 = 106,480 tokens)
    "minute": dict(B=1, H=20, D=112, T=121, N=880, io="bf16", gamma="uniform"),
}


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2_normalise(x):
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def _to_io(x, io):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16) if io == "bf16" else t.to(torch.float32)


def make_inputs(B, H, T, N, D, io="bf16", gamma="uniform", seed=0,
                with_do=False, with_dstate=False, with_state=False,
                state_std=0.1, raw=False, **_unused):
    """Draw one problem.  Returns a dict of CPU torch tensors:
    q, k, v [B, L, H, D] (io dtype), gamma [B, T, H] and beta [B, L, H]
    (float32), and optionally d_o [B, L, H, D] (io dtype), d_state
    [B, H, D, D] and state [B, H, D, D] (float32)."""
    if io not in ("bf16", "fp32"):
        raise ValueError(io)
    rng = np.random.Generator(np.random.PCG64(seed))
    L = T * N
    q = rng.standard_normal((B, L, H, D), dtype=np.float32)
    k = rng.standard_normal((B, L, H, D), dtype=np.float32)
    v = rng.standard_normal((B, L, H, D), dtype=np.float32)
    if raw:
        g = rng.normal(3.0, 0.5, size=(B, T, H)).astype(np.float32)
    elif gamma == "sigmoid":
        g = _sigmoid(rng.normal(3.0, 0.5, size=(B, T, H)))
    elif gamma == "uniform":
        g = rng.uniform(0.9, 1.0, size=(B, T, H)).astype(np.float32)
    elif gamma == "one":
        g = np.ones((B, T, H), dtype=np.float32)
    else:
        raise ValueError(gamma)
    beta = rng.standard_normal((B, L, H), dtype=np.float32)
    if raw:
        q *= np.exp(rng.standard_normal((B, L, H, 1), dtype=np.float32))
        k *= np.exp(rng.standard_normal((B, L, H, 1), dtype=np.float32))
    else:
        beta = _sigmoid(beta)
        _l2_normalise(q)
        _l2_normalise(k)
    out = {"q": _to_io(q, io), "k": _to_io(k, io), "v": _to_io(v, io),
           "gamma": torch.from_numpy(g), "beta": torch.from_numpy(beta)}
    del q, k, v
    if with_do:
        out["d_o"] = _to_io(rng.standard_normal((B, L, H, D), dtype=np.float32), io)
    if with_dstate:
        out["d_state"] = torch.from_numpy(
            rng.standard_normal((B, H, D, D), dtype=np.float32))
    if with_state:
        out["state"] = torch.from_numpy(
            (state_std * rng.standard_normal((B, H, D, D))).astype(np.float32))
    return out


def make_config(name, seed=0, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make_inputs(seed=seed, **cfg)


def orthonormal_frame_keys(B, H, T, N, D, seed=0, io="fp32"):
    """Keys orthonormal within every (frame, head) (needs N <= D), plus
    values, for the exact-retrieval case: returns (k, v) as torch tensors.
    The orthonormal columns come from a QR factorisation of a Gaussian."""
    if N > D:
        raise ValueError("orthonormal keys need N <= D")
    rng = np.random.Generator(np.random.PCG64(seed))
    k = np.zeros((B, T * N, H, D), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                qm, _ = np.linalg.qr(rng.standard_normal((D, N)))
                k[b, t * N:(t + 1) * N, h, :] = qm.T
    v = rng.standard_normal((B, T * N, H, D))
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32, "fp64": torch.float64}[io]
    return torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt)


def as_f64(t):
    """Exact float64 copy of a tensor's values (bf16 and fp32 embed exactly)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
