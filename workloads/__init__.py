"""Seeded synthetic inputs for the MuonClip step (shared by tests, smoke and bench).

This module only draws random tensors and projects activations through
weights (the model's forward, which produces the Q and K the step consumes);
it holds none of the MuonClip step's own arithmetic and imports neither the
HIP binding nor the oracle.  Shapes follow the model the pages describe:
hidden 7168, expert hidden 2048, 384 experts, 64 heads with a 128 + 64
query/key head dim ("Kimi K2: Open Agentic Intelligence", section 3.4
architecture; the Zhihu thread's MLA compute formula with 128/64/128 dims).

Every generator takes a seed and a device; the same seed and shapes give the
same tensors on the same device type.  "N(0, s)" means standard deviation s.
"""

import math
from dataclasses import dataclass

import torch

__all__ = [
    "generator",
    "normal",
    "TinyAttention",
    "tiny_attention",
    "ExpertBatch",
    "expert_batch",
    "MlaLogits",
    "mla_weights",
    "mla_project",
    "mla_logits",
    "randperm_heads",
    "spectral_momentum",
    "SPECTRAL_KINDS",
]


def generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, gen, device, dtype=torch.float32):
    """N(0, std) drawn in float32 on `device`, then cast (rounded) to dtype."""
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype) if dtype != torch.float32 else t


# ---------------------------------------------------------------------------
# Tiny fp32 single attention layer (MHA): one full MuonClip step on it.
# ---------------------------------------------------------------------------
@dataclass
class TinyAttention:
    X: torch.Tensor       # [B, S, d_model]
    W: dict               # 'q', 'k', 'v' -> [d_model, d_model] ([out, in], head-major rows)
    G: dict               # gradients, same shapes
    n_heads: int
    head_dim: int


def tiny_attention(seed=1, device="cpu", weight_reading="std", d_model=256, n_heads=4, batch=2, seq=128,
                   head0_scale=8.0, grad_std=1e-3):
    """d_model 256, 4 heads x 64; W_q/W_k/W_v ~ N(0, 0.02) with head 0 of W_q
    and W_k scaled x8; X [2, 128, 256] ~ N(0, 1); grads ~ N(0, 1e-3).

    weight_reading='std' takes 0.02 as the standard deviation (head 0 stays
    under tau = 100); 'variance' takes it as the variance (std 0.1414, head 0
    far over tau)."""
    std = {"std": 0.02, "variance": math.sqrt(0.02)}[weight_reading]
    g = generator(seed, device)
    hd = d_model // n_heads
    X = normal((batch, seq, d_model), 1.0, g, device)
    W = {n: normal((d_model, d_model), std, g, device) for n in ("q", "k", "v")}
    for n in ("q", "k"):
        W[n][:hd] *= head0_scale
    G = {n: normal((d_model, d_model), grad_std, g, device) for n in ("q", "k", "v")}
    return TinyAttention(X, W, G, n_heads, hd)


# ---------------------------------------------------------------------------
# A batch of expert matrices for Newton-Schulz
# ---------------------------------------------------------------------------
@dataclass
class ExpertBatch:
    M_prev: torch.Tensor  # float32 [batch, rows, cols]
    G: torch.Tensor       # float32 [batch, rows, cols]


def expert_batch(seed=2, device="cpu", batch=64, rows=2048, cols=7168, std=1e-3):
    """M_{t-1} and G ~ N(0, std) float32 (the 2048 x 7168 expert up-projection shape)."""
    g = generator(seed, device)
    M = normal((batch, rows, cols), std, g, device)
    G = normal((batch, rows, cols), std, g, device)
    return ExpertBatch(M, G)


# ---------------------------------------------------------------------------
# MLA attention projections and their Q / K
# ---------------------------------------------------------------------------
def randperm_heads(n_heads, k, gen, device):
    return torch.randperm(n_heads, generator=gen, device=device)[:k].sort().values


def mla_weights(seed=3, device="cpu", d_model=7168, n_heads=64, d_nope=128, d_rope=64, std=0.02,
                n_hot=4, hot_scale=6.0, dtype=torch.bfloat16):
    """W_q [H*(d_nope+d_rope), d_model] (per head: nope rows then rope rows),
    W_kc [H*d_nope, d_model], W_kr [d_rope, d_model] (shared), ~ N(0, std).
    n_hot heads drawn by randperm get W_q (nope and rope) and W_kc rows x hot_scale;
    W_kr is never scaled.  Returns (Wq, Wkc, Wkr, hot_heads)."""
    g = generator(seed, device)
    dq = d_nope + d_rope
    Wq = normal((n_heads * dq, d_model), std, g, device)
    Wkc = normal((n_heads * d_nope, d_model), std, g, device)
    Wkr = normal((d_rope, d_model), std, g, device)
    hot = randperm_heads(n_heads, n_hot, generator(seed + 1000, "cpu"), "cpu") if n_hot else torch.zeros(0, dtype=torch.long)
    for h in hot.tolist():
        Wq[h * dq:(h + 1) * dq] *= hot_scale
        Wkc[h * d_nope:(h + 1) * d_nope] *= hot_scale
    return Wq.to(dtype), Wkc.to(dtype), Wkr.to(dtype), hot


@dataclass
class MlaLogits:
    Q: torch.Tensor    # [B, H, S, d_nope + d_rope]
    Kc: torch.Tensor   # [B, H, S, d_nope]
    Kr: torch.Tensor   # [B, S, d_rope]
    hot: torch.Tensor  # heads scaled to exceed tau


def mla_project(X, Wq, Wkc, Wkr, n_heads, chunk=1024):
    """Q = X W_q^T etc. split into heads (the forward's projections), in X's dtype,
    computed row-chunk by row-chunk so the float32 intermediate stays small."""
    B, S, _ = X.shape
    dq = Wq.shape[0] // n_heads
    dc = Wkc.shape[0] // n_heads
    dr = Wkr.shape[0]
    Q = torch.empty((B, n_heads, S, dq), dtype=X.dtype, device=X.device)
    Kc = torch.empty((B, n_heads, S, dc), dtype=X.dtype, device=X.device)
    Kr = torch.empty((B, S, dr), dtype=X.dtype, device=X.device)
    # right operands materialised [in, out] once (2-D products, no transposed views)
    WqT, WkcT, WkrT = Wq.t().contiguous(), Wkc.t().contiguous(), Wkr.t().contiguous()
    for b in range(B):
        for s0 in range(0, S, chunk):
            x = X[b, s0:s0 + chunk]
            Q[b, :, s0:s0 + chunk] = (x @ WqT).view(-1, n_heads, dq).transpose(0, 1)
            Kc[b, :, s0:s0 + chunk] = (x @ WkcT).view(-1, n_heads, dc).transpose(0, 1)
            Kr[b, s0:s0 + chunk] = x @ WkrT
    return Q, Kc, Kr


def mla_logits(seed=3, device="cpu", batch=8, seq=4096, d_model=7168, n_heads=64, d_nope=128, d_rope=64,
               std=0.02, n_hot=4, hot_scale=6.0, dtype=torch.bfloat16):
    """X [batch, seq, d_model] ~ N(0, 1) in dtype, projected through mla_weights."""
    Wq, Wkc, Wkr, hot = mla_weights(seed, device, d_model, n_heads, d_nope, d_rope, std, n_hot,
                                    hot_scale, dtype)
    X = normal((batch, seq, d_model), 1.0, generator(seed + 2000, device), device, dtype)
    Q, Kc, Kr = mla_project(X, Wq, Wkc, Wkr, n_heads)
    del X
    return MlaLogits(Q, Kc, Kr, hot)


# ---------------------------------------------------------------------------
# Momentum matrices with prescribed spectra, for Newton-Schulz parity beyond
# Gaussian inputs.  A rarely routed expert's gradient is a sum of a few
# token outer products (low rank); accumulated momentum mixes them with
# small noise; trained weights' momenta have decaying spectra.
# ---------------------------------------------------------------------------
SPECTRAL_KINDS = ("gauss", "decay4", "rank16_noise", "rank1", "rank4")


def spectral_momentum(kind, rows, cols, seed=0, std=1e-3, device="cpu"):
    """A float32 rows x cols matrix with entries of size ~std whose spectrum is:
    'gauss'         i.i.d. N(0, std);
    'decay4'        singular values logspace(0, -4, min(rows, cols)) (four
                    decades) with Haar-random singular vectors (QR of Gaussian
                    matrices);
    'rank16_noise'  a rank-16 product of Gaussian factors plus i.i.d. noise of
                    1e-3 times its entry size;
    'rank1'         an exact outer product u v^T of Gaussian vectors;
    'rank4'         an exact rank-4 product of Gaussian factors.
    Drawn in float64 on the CPU from `seed`, rounded to float32 once."""
    g = generator(seed, "cpu")
    n = min(rows, cols)
    f64 = torch.float64
    if kind == "gauss":
        M = torch.randn(rows, cols, generator=g, dtype=f64)
    elif kind == "decay4":
        U, _ = torch.linalg.qr(torch.randn(rows, n, generator=g, dtype=f64))
        V, _ = torch.linalg.qr(torch.randn(cols, n, generator=g, dtype=f64))
        M = (U * torch.logspace(0, -4, n, dtype=f64)) @ V.T
    elif kind in ("rank16_noise", "rank1", "rank4"):
        r = {"rank16_noise": 16, "rank1": 1, "rank4": 4}[kind]
        M = torch.randn(rows, r, generator=g, dtype=f64) @ torch.randn(r, cols, generator=g, dtype=f64)
        if kind == "rank16_noise":
            M = M + 1e-3 * M.std() * torch.randn(rows, cols, generator=g, dtype=f64)
    else:
        raise ValueError(f"unknown spectrum kind {kind!r}")
    M = M * (std / M.std())
    return M.to(torch.float32).to(device)


def orthonormal_factors(rows, cols, sigma, seed=0):
    """Exact SVD factors of a rank-r matrix M = U diag(sigma) V^T: U (rows x r)
    and V (cols x r) with orthonormal columns (QR of Gaussian matrices drawn
    from `seed`, float64 on the CPU) and the given singular values.  The
    matrix itself is formed wherever it is needed (e.g. on the device for the
    largest shapes), so its SVD is known without computing one."""
    g = generator(seed, "cpu")
    sigma = torch.as_tensor(sigma, dtype=torch.float64)
    r = sigma.numel()
    U, _ = torch.linalg.qr(torch.randn(rows, r, generator=g, dtype=torch.float64))
    V, _ = torch.linalg.qr(torch.randn(cols, r, generator=g, dtype=torch.float64))
    return U, sigma, V
