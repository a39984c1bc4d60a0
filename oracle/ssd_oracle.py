"""Plain, slow, fp64 CPU oracle of the Mamba-2 SSD forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path. It shares no code,
constant or helper with the HIP library.

What is computed
----------------
A selective state-space model whose state-transition matrix is one scalar per
head times the identity (Telegram post "Mamba3", opening paragraph: Mamba-2
reduced the transition matrix to a scalar times the identity; the same fact in
"Mamba-3 : SSM optimise inference", section "Du training-first a
l'inference-first"). The continuous system is discretised with zero-order hold
for the transition and an Euler step for the input ("Mamba3", section on the
new discretisation scheme: Mamba-1/2 used a mix of ZOH and Euler). Per batch b
and head h, with the head's B/C group g:

    alpha_t  = exp(dt[b,t,h] * A[h])                         (ZOH of A)
    h_t[p,n] = alpha_t * h_{t-1}[p,n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
    y[b,t,h,p] = sum_n h_t[p,n] * C[b,t,g,n] + D[h] * x[b,t,h,p]

starting from h_{-1} = init_state[b,h] (zeros when absent); the state after the
last token is the final state. The state is stored [P, N] (P = head dim, N =
state dim).

Readings of points the pages leave open (each also listed in the design doc):
  * y_t reads the state AFTER the update at t, so the diagonal of the
    semiseparable matrix carries dt_t * (C_t . B_t).
  * dt is used as given (no softplus, bias or clamp inside the operator).
  * A is the transition value itself (expected <= 0), not its logarithm.
  * Heads map to groups contiguously: g = h // (H // G).
  * D is one scalar per head, a skip term added after the SSM; None means 0.
  * Inputs are the exact values the GPU receives (bf16 values upcast exactly).

The same semiseparable matrix can be contracted sequentially (the recurrence),
densely as masked attention, or blockwise (chunks in parallel, then per-chunk
states recombined): "Mamba-2 vs Transformers: SSMs, structured state space
duality", sections "How we compared Mamba-2, Transformers, and mixed
SSD+attention models" and "Mamba-2 and the SSD paper: what changed in practice"
(and the contraction-order table there). All three orders are written out
below; the recurrence is the oracle, the other two are independent pins.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "ssd_recurrent",
    "ssd_quadratic",
    "ssd_semiseparable_matrix",
    "ssd_chunked",
    "chunk_cumsum",
    "chunk_local_states",
    "chunk_entry_states",
    "group_of_head",
    "dt_preprocess",
    "causal_conv1d",
]


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> numpy without importing torch
        a = a.detach().cpu().float().numpy() if str(a.dtype) == "torch.bfloat16" else a.detach().cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def _check_shapes(x, dt, A, B, C, D, h0):
    if x.ndim != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim]")
    bsz, L, H, P = x.shape
    if dt.shape != (bsz, L, H):
        raise ValueError(f"dt must be {(bsz, L, H)}, got {dt.shape}")
    if A.shape != (H,):
        raise ValueError(f"A must be {(H,)}, got {A.shape}")
    if B.ndim != 4 or B.shape[:2] != (bsz, L) or C.shape != B.shape:
        raise ValueError("B and C must both be [batch, seqlen, ngroups, dstate]")
    G, N = B.shape[2], B.shape[3]
    if G < 1 or H % G != 0:
        raise ValueError("nheads must be a multiple of ngroups")
    if D is not None and D.shape != (H,):
        raise ValueError(f"D must be {(H,)}")
    if h0 is not None and h0.shape != (bsz, H, P, N):
        raise ValueError(f"init_state must be {(bsz, H, P, N)}")
    return bsz, L, H, P, G, N


def group_of_head(h: int, nheads: int, ngroups: int) -> int:
    """Contiguous head->group map: each run of nheads//ngroups heads shares a group."""
    return h // (nheads // ngroups)


def _expand_groups(M, H):
    """[b, L, G, N] -> [b, L, H, N] with the contiguous head->group map."""
    G = M.shape[2]
    return np.repeat(M, H // G, axis=2)


def dt_preprocess(dt, dt_bias=None, softplus=False, limit=None):
    """dt as the layer may transform it before the recurrence, fp64: a
    per-head bias added first, then softplus(z) = log(1 + e^z), then a clamp
    to [lo, hi]. The pages do not spell this step out (they name the layer's
    parts only); the order is the one the workloads' dt recipe uses (softplus,
    then the clamp), with the bias inside the softplus.

    dt [..., H], dt_bias [H] or None, limit (lo, hi) or None.
    """
    z = _f64(dt)
    if dt_bias is not None:
        z = z + _f64(dt_bias)
    if softplus:
        z = np.logaddexp(0.0, z)  # log(e^0 + e^z), without overflow
    if limit is not None:
        z = np.minimum(np.maximum(z, float(limit[0])), float(limit[1]))
    return z


def causal_conv1d(u, weight, bias=None, silu=False, state=None):
    """The short causal convolution in front of the SSM, fp64: per channel,
    z[t] = bias + sum_k weight[k] * u[t - (K-1) + k], with u before t = 0 taken
    from `state` (the K-1 previous inputs, oldest first; zeros when None);
    then z * sigmoid(z) when `silu`. The pages name this convolution (present
    in Mamba-1 and Mamba-2) but give neither width nor activation; both are
    parameters here.

    u [b, L, CH], weight [CH, K], bias [CH] or None, state [b, CH, K-1] or None.
    Returns (out [b, L, CH], the last K-1 inputs [b, CH, K-1]).
    """
    u = _f64(u)
    w = _f64(weight)
    bsz, L, CH = u.shape
    K = w.shape[1]
    prev = np.zeros((bsz, K - 1, CH)) if state is None else np.transpose(_f64(state), (0, 2, 1))
    full = np.concatenate([prev, u], axis=1)  # [b, K-1+L, CH]: position t at index t + K-1
    z = np.zeros((bsz, L, CH)) if bias is None else np.broadcast_to(_f64(bias), (bsz, L, CH)).copy()
    for k in range(K):
        z += w[None, None, :, k] * full[:, k:k + L, :]
    if silu:
        z = z / (1.0 + np.exp(-z))
    last = np.transpose(full[:, L:L + K - 1, :], (0, 2, 1)) if K > 1 else np.zeros((bsz, CH, 0))
    return z, last


def ssd_recurrent(x, dt, A, B, C, D=None, init_state=None):
    """The definition: the token-by-token recurrence, fp64.

    Shapes: x [b, L, H, P], dt [b, L, H], A [H], B/C [b, L, G, N], D [H] or None,
    init_state [b, H, P, N] or None. Returns (y [b, L, H, P], final [b, H, P, N]).
    Vectorised over (b, h, p, n); sequential over t, exactly as written in the
    module docstring.
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, init_state))
    bsz, L, H, P, G, N = _check_shapes(x, dt, A, B, C, D, h0)
    Bh = _expand_groups(B, H)
    Ch = _expand_groups(C, H)
    h = np.zeros((bsz, H, P, N)) if h0 is None else h0.copy()
    y = np.empty((bsz, L, H, P))
    for t in range(L):
        alpha = np.exp(dt[:, t, :] * A[None, :])  # [b, H]
        inp = (dt[:, t, :, None] * x[:, t])[..., None] * Bh[:, t, :, None, :]  # [b,H,P,N]
        h = alpha[:, :, None, None] * h + inp
        y[:, t] = np.matmul(h, Ch[:, t, :, :, None])[..., 0]
    if D is not None:
        y += D[None, None, :, None] * x
    return y, h


def ssd_quadratic(x, dt, A, B, C, D=None, init_state=None):
    """The dual, attention-like contraction of the same matrix, fp64, O(L^2).

    With the global inclusive cumulative log-decay cs_t = sum_{k<=t} dt_k A,
        y_t = sum_{s<=t} exp(cs_t - cs_s) (C_t . B_s) dt_s x_s
              + exp(cs_t) (h0 C_t) + D x_t,
        final = exp(cs_{L-1}) h0 + sum_s exp(cs_{L-1} - cs_s) dt_s x_s B_s^T.
    Only for small L (a dense L x L mask per (b, h)).
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, init_state))
    bsz, L, H, P, G, N = _check_shapes(x, dt, A, B, C, D, h0)
    Bh = _expand_groups(B, H)
    Ch = _expand_groups(C, H)
    a = dt * A[None, None, :]                      # [b, L, H]
    cs = np.cumsum(a, axis=1)                       # [b, L, H]
    seg = cs[:, :, None, :] - cs[:, None, :, :]    # [b, t, s, H] = cs_t - cs_s
    causal = np.tril(np.ones((L, L), dtype=bool))
    decay = np.where(causal[None, :, :, None], np.exp(np.where(causal[None, :, :, None], seg, 0.0)), 0.0)
    scores = np.einsum("bthn,bshn->btsh", Ch, Bh)  # C_t . B_s
    W = scores * decay * dt[:, None, :, :]          # [b, t, s, H]
    y = np.einsum("btsh,bshp->bthp", W, x)
    if h0 is not None:
        y += np.exp(cs)[..., None] * np.einsum("bhpn,bthn->bthp", h0, Ch)
    if D is not None:
        y += D[None, None, :, None] * x
    wT = np.exp(cs[:, -1:, :] - cs) * dt            # [b, s, H]
    final = np.einsum("bsh,bshp,bshn->bhpn", wT, x, Bh)
    if h0 is not None:
        final += np.exp(cs[:, -1, :])[:, :, None, None] * h0
    return y, final


def ssd_semiseparable_matrix(dt, A, B, C, b: int, h: int):
    """The explicit L x L lower-triangular semiseparable matrix of one (b, h).

    M[t, s] = (C_t . B_s) * dt_s * prod_{k=s+1..t} exp(dt_k A) for s <= t, else 0,
    built entry by entry with plain loops (tiny L only). Then, without an
    initial state, y[b, :, h, p] = M @ x[b, :, h, p] + D x.
    """
    dt, A, B, C = map(_f64, (dt, A, B, C))
    L = dt.shape[1]
    H = dt.shape[2]
    g = group_of_head(h, H, B.shape[2])
    M = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            prod = 1.0
            for k in range(s + 1, t + 1):
                prod *= np.exp(dt[b, k, h] * A[h])
            M[t, s] = float(np.dot(C[b, t, g], B[b, s, g])) * dt[b, s, h] * prod
    return M


def ssd_chunked(x, dt, A, B, C, D=None, init_state=None, chunk: int = 64):
    """The blocked two-pass algorithm in fp64, written independently of the
    recurrence: split the sequence into chunks, compute every chunk's local
    output and local state in parallel, then recombine the per-chunk states
    ("Mamba-2 vs Transformers...", section "Mamba-2 and the SSD paper: what
    changed in practice"). Used only to pin the recurrence and to check that
    the result does not depend on the chunk length.

    Per chunk c (local index i, inclusive local log-decay l_i, chunk total Lam):
      S_c     = sum_j exp(Lam - l_j) dt_j x_j B_j^T          (local state)
      Yin[i]  = sum_{j<=i} exp(l_i - l_j) dt_j (C_i . B_j) x_j (intra-chunk)
      Yst[i]  = exp(l_i) H_in C_i                             (carried state)
      H_in(c+1) = exp(Lam) H_in(c) + S_c
    A partial last chunk is simply shorter.
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, init_state))
    bsz, L, H, P, G, N = _check_shapes(x, dt, A, B, C, D, h0)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    Bh = _expand_groups(B, H)
    Ch = _expand_groups(C, H)
    a = dt * A[None, None, :]
    y = np.empty((bsz, L, H, P))
    Hin = np.zeros((bsz, H, P, N)) if h0 is None else h0.copy()
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        Q = c1 - c0
        l = np.cumsum(a[:, c0:c1], axis=1)            # [b, Q, H]
        lam = l[:, -1, :]                               # [b, H]
        xc, dtc, Bc, Cc = x[:, c0:c1], dt[:, c0:c1], Bh[:, c0:c1], Ch[:, c0:c1]
        # local state
        w = np.exp(lam[:, None, :] - l) * dtc           # [b, Q, H]
        S = np.einsum("bjh,bjhp,bjhn->bhpn", w, xc, Bc)
        # intra-chunk (masked dual form restricted to the chunk)
        causal = np.tril(np.ones((Q, Q), dtype=bool))[None, :, :, None]
        seg = l[:, :, None, :] - l[:, None, :, :]
        decay = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
        CB = np.einsum("bihn,bjhn->bijh", Cc, Bc)
        y_in = np.einsum("bijh,bjhp->bihp", CB * decay * dtc[:, None, :, :], xc)
        # contribution of the state entering the chunk
        y_st = np.exp(l)[..., None] * np.einsum("bhpn,bihn->bihp", Hin, Cc)
        y[:, c0:c1] = y_in + y_st
        Hin = np.exp(lam)[:, :, None, None] * Hin + S
    if D is not None:
        y += D[None, None, :, None] * x
    return y, Hin


# --------------------------------------------------------------------------
# Intermediate quantities of the chunked path, from their plain definitions.
# Layouts match what a chunked implementation naturally produces: per
# (b, h, chunk) with the chunk's positions innermost. Positions past the end
# of the sequence (partial last chunk) behave as dt = 0: the log-decay stays
# constant and nothing is added to the state.
# --------------------------------------------------------------------------

def chunk_cumsum(dt, A, chunk: int):
    """l[b, h, c, i] = sum_{k=cQ}^{cQ+i} dt[b,k,h] * A[h] (inclusive, within the
    chunk), with dt = 0 past the end of the sequence. Returns fp64
    [b, H, nc, Q]; the chunk total is l[..., -1]."""
    dt, A = _f64(dt), _f64(A)
    bsz, L, H = dt.shape
    nc = -(-L // chunk)
    out = np.zeros((bsz, H, nc, chunk))
    for c in range(nc):
        acc = np.zeros((bsz, H))
        for i in range(chunk):
            t = c * chunk + i
            if t < L:
                acc = acc + dt[:, t, :] * A[None, :]
            out[:, :, c, i] = acc
    return out


def chunk_local_states(x, dt, A, B, chunk: int):
    """S[b, h, c] = the state the recurrence reaches at the end of chunk c when
    it starts that chunk from zero (the per-chunk SSM state). [b, H, nc, P, N]."""
    x, dt, A, B = map(_f64, (x, dt, A, B))
    bsz, L, H, P = x.shape
    nc = -(-L // chunk)
    out = np.zeros((bsz, H, nc, P, B.shape[3]))
    for c in range(nc):
        sl = slice(c * chunk, min(L, (c + 1) * chunk))
        _, hT = ssd_recurrent(x[:, sl], dt[:, sl], A, B[:, sl], B[:, sl])
        out[:, :, c] = hT
    return out


def chunk_entry_states(x, dt, A, B, chunk: int, init_state=None):
    """Hin[b, h, c] = the state of the full recurrence just before chunk c's
    first token (init_state for c = 0), and the final state.
    Returns (Hin [b, H, nc, P, N], final [b, H, P, N])."""
    x, dt, A, B, h0 = map(_f64, (x, dt, A, B, init_state))
    bsz, L, H, P = x.shape
    N = B.shape[3]
    nc = -(-L // chunk)
    out = np.zeros((bsz, H, nc, P, N))
    h = np.zeros((bsz, H, P, N)) if h0 is None else h0.copy()
    for c in range(nc):
        out[:, :, c] = h
        sl = slice(c * chunk, min(L, (c + 1) * chunk))
        _, h = ssd_recurrent(x[:, sl], dt[:, sl], A, B[:, sl], B[:, sl], None, h)
    return out, h
