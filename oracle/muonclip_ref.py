"""fp64 CPU oracle of the MuonClip optimizer step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code, constant table or helper with the HIP library; the product path never
imports it.

What it computes, and where the pages define it:

* Momentum ``M_t = mu * M_{t-1} + G_t`` with ``M_0 = 0``: "Kimi K2 内部机制"
  (Kimi K2 internals deep dive), MuonClip section, Algorithm 1, the Muon
  optimizer step; the same step as two in-place tensor ops (scale, then add) in
  the ``muonclip_step`` pseudocode of "Kimi K2: Open Agentic Intelligence"
  (paper notes), section 3.2 MuonClip.
* ``O_t = NewtonSchulz(M_t) * sqrt(max(n, m)) * 0.2`` and the decoupled-decay
  update ``W_t = W_{t-1} - eta * (O_t + lambda * W_{t-1})``: Algorithm 1 of the
  internals deep dive; the MuonClip formula block of the Zhihu thread
  (freezhihu.org question 1927140506573435010, the K2 author's answer on the
  optimizer), where the orthogonaliser is written msign.
* Newton-Schulz: "Kimi K2, explained." (vibeengines.com), the bullet list under
  the Muon update formula, describes it only qualitatively: a short iteration
  of an odd polynomial in the matrix that moves every singular value close to
  1, so the result approximates the orthogonal factor U V^T of M = U S V^T.  The polynomial coefficients,
  the step count and the normalisation are NOT on the pages; the readings used
  here are listed next to ``NS_COEFFS``.
* Per-head max logit ``S_max^h = (1/sqrt(d)) max_{X in B} max_{i,j} Q_i^h K_j^h^T``:
  internals deep dive, "核心数学" (core maths).  The paper-notes page prints
  1/d there, which is the same formula with the square root lost in extraction.
* Attention forward ``O^h = softmax(Q^h K^h^T / sqrt(d)) V^h`` with the max
  logit of the same logits as a by-product (the internals deep dive: S_max
  is already computed in the forward; the paper notes, section 3.2: the
  per-head max logit comes from the attention forward), optionally causal.
* ``gamma_h = min(1, tau / S_max^h)``, only heads with ``S_max^h > tau`` touched;
  MHA split ``W_q^h <- gamma^alpha W_q^h``, ``W_k^h <- gamma^(1-alpha) W_k^h``;
  MLA split (table "MLA 的特殊处理"): head-specific q^C and k^C by sqrt(gamma),
  head-specific rotary q^R by gamma, shared rotary k^R untouched.  Same
  internals deep dive, and the Zhihu formula block (sqrt(tau/S) on W_qc, W_kc;
  tau/S on W_qr).

Parity pins for every function here live in ``tests/test_oracle_*.py``.
"""

import math

import numpy as np

from .rounding import round_to

__all__ = [
    "MU",
    "TAU",
    "ALPHA",
    "WEIGHT_DECAY",
    "RMS_MATCH",
    "NS_STEPS",
    "NS_COEFFS",
    "NS_EPS",
    "momentum_update",
    "ns_normalise",
    "newton_schulz",
    "ns_polynomial_scalar",
    "muon_scale",
    "muon_orthogonalised_update",
    "apply_update",
    "max_logit",
    "max_logit_bruteforce",
    "attention_forward",
    "attention_forward_bruteforce",
    "clip_factors",
    "qk_clip",
    "qk_clip_total",
    "project_heads",
    "muonclip_step",
]

# Defaults of the step: the muonclip_step signature on the paper-notes page
# (momentum 0.95, weight decay 0.1, tau 100) and alpha = 0.5 from the internals
# deep dive ("alpha usually 0.5, query and key share the scaling").
MU = 0.95
TAU = 100.0
ALPHA = 0.5
WEIGHT_DECAY = 0.1
RMS_MATCH = 0.2  # sqrt(max(n, m)) * 0.2 "match Adam RMS", Algorithm 1

# Newton-Schulz polynomial (NOT on the pages; reading, see module docstring):
# the quintic p(x) = a x + b x^3 + c x^5 of the public Muon optimiser, with the
# same (a, b, c) at every one of 5 steps.  Fixed spec constants; the pins test
# the iteration for any coefficients (spectral identity), not these values.
NS_STEPS = 5
NS_COEFFS = ((3.4445, -4.7750, 2.0315),) * NS_STEPS
# Frobenius-norm pre-scale X_0 = M / (||M||_F + eps) (reading: the Frobenius
# norm bounds the spectral norm, so every singular value of X_0 is <= 1).
NS_EPS = 1e-7


# --------------------------------------------------------------------------
# Momentum
# --------------------------------------------------------------------------
def momentum_update(M_prev, G, mu=MU):
    """``M_t = fl32(fl32(mu * M_{t-1}) + G_t)`` in float32 storage.

    Algorithm 1 of the internals deep dive gives ``M_t = mu M_{t-1} + G_t``; the
    paper-notes pseudocode performs it as two in-place float ops (scale, then
    add), so each of the two results is rounded to float32.  Each op is done
    in fp64 and rounded once to float32: fp64 has 53 >= 2*24 + 2 significand
    bits, so this equals a float32 multiply followed by a float32 add with no
    fused multiply-add (double rounding is innocuous at that width).
    ``mu`` is itself the float32 value nearest the given number.
    """
    M_prev = np.asarray(M_prev, dtype=np.float32)
    G = np.asarray(G, dtype=np.float32)
    mu32 = np.float64(np.float32(mu))
    scaled = round_to(mu32 * M_prev.astype(np.float64), "f32")
    return round_to(scaled + G.astype(np.float64), "f32").astype(np.float32)


# --------------------------------------------------------------------------
# Newton-Schulz
# --------------------------------------------------------------------------
def ns_normalise(M, eps=NS_EPS):
    """``X_0 = M / (||M||_F + eps)`` in fp64 (M = 0 gives X_0 = 0)."""
    M = np.asarray(M, dtype=np.float64)
    return M / (np.linalg.norm(M) + eps)


def newton_schulz(M, coeffs=NS_COEFFS, eps=NS_EPS):
    """Newton-Schulz orthogonalisation of one matrix, fp64.

    X_0 = M / (||M||_F + eps); if M has more rows than columns the iteration
    runs on the transpose (an odd polynomial p satisfies X p(X^T X) = p(X X^T) X,
    so the result is the same, only the Gram matrix is smaller) and the result
    is transposed back.  Each step applies p(X) = a X + b (X X^T) X + c (X X^T)^2 X
    written as A = X X^T, B = b A + c A A, X <- a X + B X.
    """
    X = ns_normalise(M, eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    for a, b, c in coeffs:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T.copy() if transposed else X


def ns_polynomial_scalar(sigma, coeffs=NS_COEFFS):
    """What the iteration does to one singular value: p_s(...p_1(sigma))."""
    s = np.asarray(sigma, dtype=np.float64)
    for a, b, c in coeffs:
        s = a * s + b * s**3 + c * s**5
    return s


def muon_scale(rows, cols):
    """The Adam-RMS matching factor sqrt(max(n, m)) * 0.2 of Algorithm 1."""
    return math.sqrt(max(rows, cols)) * RMS_MATCH


def muon_orthogonalised_update(M, coeffs=NS_COEFFS, eps=NS_EPS):
    """``O_t = NewtonSchulz(M_t) * sqrt(max(n, m)) * 0.2`` (fp64)."""
    M = np.asarray(M, dtype=np.float64)
    return newton_schulz(M, coeffs, eps) * muon_scale(*M.shape)


def apply_update(W, O, lr, weight_decay=WEIGHT_DECAY, w_dtype="bf16"):
    """``W_t = W_{t-1} - eta (O_t + lambda W_{t-1})`` computed in fp64 and
    rounded once to W's storage type (Algorithm 1; paper-notes pseudocode)."""
    W = np.asarray(W, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    return round_to(W - lr * (O + weight_decay * W), w_dtype)


# --------------------------------------------------------------------------
# Per-head max logit
# --------------------------------------------------------------------------
def _head_keys(Kc, Kr, b, h):
    """K^h of one batch element: [Kc[b, h] || Kr[b]] (the rotary key is shared by
    all heads under MLA), or Kc[b, h] alone for MHA (Kr is None)."""
    k = np.asarray(Kc[b, h], dtype=np.float64)
    if Kr is None:
        return k
    return np.concatenate([k, np.asarray(Kr[b], dtype=np.float64)], axis=1)


def max_logit(Q, Kc, Kr=None, block=1024):
    """``S_max^h = (1/sqrt(d)) max_b max_{i,j} Q[b,h,i] . K[b,h,j]`` per head, fp64.

    Q: [B, H, S_q, d]; Kc: [B, H, S_k, d_c]; Kr: [B, S_k, d_r] or None with
    d = d_c + d_r.  The maximum is taken over the logits that are not NaN; a
    head none of whose logits is a number reports -inf.  The max is taken
    before the positive 1/sqrt(d) scale, which cannot change it (rounding is
    monotone).  Blocked over j so the logit matrix is never held whole.
    """
    Q = np.asarray(Q)
    B, H, Sq, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.full(H, -np.inf)
    for h in range(H):
        m = -np.inf
        for b in range(B):
            q = np.asarray(Q[b, h], dtype=np.float64)
            k = _head_keys(Kc, Kr, b, h)
            if k.shape[1] != d:
                raise ValueError("query and key head dims differ")
            for j0 in range(0, k.shape[0], block):
                logits = q @ k[j0:j0 + block].T
                if logits.size:
                    m = np.fmax(m, np.fmax.reduce(logits, axis=None, initial=-np.inf))
        out[h] = m * scale
    return out


def max_logit_bruteforce(Q, Kc, Kr=None):
    """Pure-Python triple loop over (b, i, j) of the same definition; tiny inputs only."""
    Q = np.asarray(Q, dtype=np.float64)
    B, H, Sq, d = Q.shape
    out = []
    for h in range(H):
        best = -math.inf
        for b in range(B):
            k = _head_keys(Kc, Kr, b, h)
            for i in range(Sq):
                for j in range(k.shape[0]):
                    s = 0.0
                    for t in range(d):
                        s += float(Q[b, h, i, t]) * float(k[j, t])
                    if s == s and s > best:
                        best = s
        out.append(best * (1.0 / math.sqrt(d)))  # (1/sqrt(d)) x max, as printed
    return np.array(out)


# --------------------------------------------------------------------------
# Attention forward with the max logit as a by-product
# --------------------------------------------------------------------------
def _causal_allowed(Sq, Sk):
    """Key j is visible to query i when j <= i + (Sk - Sq) (the queries are the
    last Sq positions of the Sk keys; Sq == Sk is the usual square mask)."""
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    return j <= i + (Sk - Sq)


def attention_forward(Q, Kc, Kr, V, causal=False):
    """``O^h = softmax(Q^h K^h^T / sqrt(d)) V^h`` per batch element and head, fp64.

    Q [B, H, Sq, d], Kc [B, H, Sk, d_c], Kr [B, Sk, d_r] or None (MHA),
    V [B, H, Sk, d_v]; K^h = [Kc^h || Kr] as in ``max_logit``.  The logits are
    ``Q K^T / sqrt(d)``; with ``causal`` the keys a query may not see (see
    ``_causal_allowed``) are left out of the softmax and of the max.  Returns
    (O [B, H, Sq, d_v], lse [B, H, Sq] = log sum_j exp(logit_ij),
    smax [H] = max over b, i and visible j of the logits).  The softmax is
    taken as exp(logit - row max) / sum, its plain definition.
    """
    Q = np.asarray(Q)
    B, H, Sq, d = Q.shape
    V = np.asarray(V)
    Sk, d_v = V.shape[2], V.shape[3]
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, Sq, d_v))
    lse = np.zeros((B, H, Sq))
    smax = np.full(H, -np.inf)
    allowed = _causal_allowed(Sq, Sk) if causal else np.ones((Sq, Sk), dtype=bool)
    for b in range(B):
        for h in range(H):
            q = np.asarray(Q[b, h], dtype=np.float64)
            k = _head_keys(Kc, Kr, b, h)
            logits = (q @ k.T) * scale
            logits = np.where(allowed, logits, -np.inf)
            m = logits.max(axis=1)
            p = np.exp(logits - m[:, None])
            l = p.sum(axis=1)
            O[b, h] = (p / l[:, None]) @ np.asarray(V[b, h], dtype=np.float64)
            lse[b, h] = m + np.log(l)
            smax[h] = max(smax[h], m.max())
    return O, lse, smax


def attention_forward_bruteforce(Q, Kc, Kr, V, causal=False):
    """Pure-Python loops over (b, h, i, j) of the same definition; tiny inputs only."""
    Q = np.asarray(Q, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Sq, d = Q.shape
    Sk, d_v = V.shape[2], V.shape[3]
    O = np.zeros((B, H, Sq, d_v))
    smax = [-math.inf] * H
    for b in range(B):
        for h in range(H):
            k = _head_keys(Kc, Kr, b, h)
            for i in range(Sq):
                logits = []
                for j in range(Sk):
                    if causal and j > i + (Sk - Sq):
                        continue
                    s = sum(float(Q[b, h, i, t]) * float(k[j, t]) for t in range(d)) / math.sqrt(d)
                    logits.append((j, s))
                m = max(s for _, s in logits)
                smax[h] = max(smax[h], m)
                w = [(j, math.exp(s - m)) for j, s in logits]
                tot = sum(x for _, x in w)
                for c in range(d_v):
                    O[b, h, i, c] = sum(x * float(V[b, h, j, c]) for j, x in w) / tot
    return O, np.array(smax)


# --------------------------------------------------------------------------
# QK-Clip
# --------------------------------------------------------------------------
def clip_factors(smax, tau=TAU):
    """Per head: gamma_h = min(1, tau / S_max^h) and the clip flag.

    Only heads with S_max^h > tau are clipped (strict: a head exactly at tau is
    untouched, as the paper-notes pseudocode skips ``s_max <= tau``).  Returns
    (gamma, clipped) with clipped = 1 for clipped heads, 0 for untouched ones
    and -1 for a NaN S_max, which compares false and is left untouched.
    """
    smax = np.asarray(smax, dtype=np.float64)
    gamma = np.ones_like(smax)
    clipped = np.zeros(smax.shape, dtype=np.int32)
    for h, s in enumerate(smax):
        if s != s:
            clipped[h] = -1
        elif s > tau:
            gamma[h] = tau / s
            clipped[h] = 1
    return gamma, clipped


def qk_clip(smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head,
            tau=TAU, alpha=ALPHA, w_dtype="bf16"):
    """Rescale the query/key projection rows of every head over tau; fp64, rounded once.

    Weights are [out_features, d_in] with head-major rows.  For head h:
      * W_q rows [h*q_rows_per_head, h*q_rows_per_head + q_c_rows) -> x gamma^alpha
        (q^C under MLA, the whole W_q^h under MHA);
      * the remaining q_rows_per_head - q_c_rows rows of the head -> x gamma
        (the head-specific rotary query q^R under MLA);
      * W_k rows [h*k_rows_per_head, (h+1)*k_rows_per_head) -> x gamma^(1-alpha)
        (k^C under MLA, W_k^h under MHA).
    The shared rotary key is not an argument, so it is never touched.  Heads not
    clipped are returned bit-for-bit unchanged.  Returns (Wq', Wk', gamma, clipped).
    """
    Wq = np.array(Wq, dtype=np.float64, copy=True)
    Wk = np.array(Wk, dtype=np.float64, copy=True)
    gamma, clipped = clip_factors(smax, tau)
    for h in range(len(gamma)):
        if clipped[h] != 1:
            continue
        g = gamma[h]
        q0 = h * q_rows_per_head
        Wq[q0:q0 + q_c_rows] = round_to(Wq[q0:q0 + q_c_rows] * g**alpha, w_dtype)
        Wq[q0 + q_c_rows:q0 + q_rows_per_head] = round_to(
            Wq[q0 + q_c_rows:q0 + q_rows_per_head] * g, w_dtype)
        k0 = h * k_rows_per_head
        Wk[k0:k0 + k_rows_per_head] = round_to(Wk[k0:k0 + k_rows_per_head] * g**(1.0 - alpha), w_dtype)
    return Wq, Wk, gamma, clipped


def qk_clip_total(smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head,
                  tau=TAU, alpha=ALPHA, w_dtype="bf16"):
    """Total clip: one gamma for all heads; fp64, rounded once.

    The naive form of the internals deep dive ("all heads clipped together"):
    ``gamma = min(1, tau / S_max)`` with ``S_max = max_h S_max^h``, and every
    head scaled like a clipped head of ``qk_clip`` (same MHA / MLA split).
    Readings: a NaN S_max^h is skipped in the max (only an all-NaN input gives
    a NaN S_max, which touches nothing and flags -1); the strict ``> tau`` of
    per-head clip.  Returns (Wq', Wk', gamma, clipped), gamma and clipped
    repeated per head.
    """
    smax = np.asarray(smax, dtype=np.float64)
    numeric = smax[smax == smax]
    s_all = numeric.max() if numeric.size else float("nan")
    return qk_clip(np.full(smax.shape, s_all), Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head,
                   tau=tau, alpha=alpha, w_dtype=w_dtype)


def project_heads(X, W, n_heads):
    """Q = X W^T split into heads: X [B, S, d_in], W [H*d_head, d_in] -> [B, H, S, d_head].

    The pages write Q^h = X W_q^h with W as [d_in, d_out]; weights here are
    stored [out, in] (row-major, head-major rows), the transpose of that.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    B, S, _ = X.shape
    d_head = W.shape[0] // n_heads
    Y = X @ W.T
    return Y.reshape(B, S, n_heads, d_head).transpose(0, 2, 1, 3)


# --------------------------------------------------------------------------
# One whole step
# --------------------------------------------------------------------------
def muonclip_step(weights, grads, momenta, smax, attention, lr, weight_decay=WEIGHT_DECAY,
                  mu=MU, tau=TAU, alpha=ALPHA, coeffs=NS_COEFFS, eps=NS_EPS, w_dtype="bf16"):
    """One MuonClip step (Algorithm 1 of the internals deep dive).

    weights, grads, momenta: dicts name -> 2-D array, or a stack of 2-D
    arrays [count, rows, cols] treated as `count` separate matrices (momenta
    float32; missing entries start at zero).  smax: per-head max logits
    measured in the forward that produced ``grads`` (at W_{t-1}), [H] for one
    attention layer or [L, H].  attention: a dict with keys 'q', 'k' (weight
    names), 'q_rows_per_head', 'q_c_rows', 'k_rows_per_head', or a list of L
    such dicts: Algorithm 1 clips every head of every attention layer, each
    layer with its own row of smax.  Muon part: every matrix; then QK-Clip on
    the updated attention weights.
    Returns (new_weights, new_momenta, gamma, clipped), gamma and clipped
    shaped like smax.
    """
    new_w, new_m = {}, {}
    for name, W in weights.items():
        M_prev = momenta.get(name)
        if M_prev is None:
            M_prev = np.zeros(np.shape(W), dtype=np.float32)
        M = momentum_update(M_prev, grads[name], mu)
        if np.ndim(W) == 3:
            new_w[name] = np.stack([apply_update(W[i], muon_orthogonalised_update(M[i].astype(np.float64), coeffs, eps),
                                                 lr, weight_decay, w_dtype) for i in range(np.shape(W)[0])])
        else:
            O = muon_orthogonalised_update(M.astype(np.float64), coeffs, eps)
            new_w[name] = apply_update(W, O, lr, weight_decay, w_dtype)
        new_m[name] = M
    layers = attention if isinstance(attention, (list, tuple)) else [attention]
    smax2 = np.atleast_2d(np.asarray(smax, dtype=np.float64))
    gammas, clips = [], []
    for a, s_l in zip(layers, smax2):
        qn, kn = a["q"], a["k"]
        Wq, Wk, gamma, clipped = qk_clip(s_l, new_w[qn], new_w[kn], a["q_rows_per_head"], a["q_c_rows"],
                                         a["k_rows_per_head"], tau, alpha, w_dtype)
        new_w[qn], new_w[kn] = Wq, Wk
        gammas.append(gamma)
        clips.append(clipped)
    if not isinstance(attention, (list, tuple)):
        return new_w, new_m, gammas[0], clips[0]
    return new_w, new_m, np.stack(gammas), np.stack(clips)
