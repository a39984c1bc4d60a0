"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The oracle (``oracle.ssd_oracle``) is the token-by-token recurrence of the
selective SSM with a scalar-times-identity transition, ZOH for A and Euler for
B (Telegram post "Mamba3": opening paragraph and the discretisation section).
Nothing here re-types that loop; each test reaches the expected value by a
different route, chosen so that a dropped term, a wrong sign or index, a
transposed operand or a wrong head->group map fails at least one of them:

  * the dual masked-attention contraction and the explicit semiseparable matrix
    ("Mamba-2 vs Transformers: SSMs, structured state space duality", sections
    "How we compared ..." and "Mamba-2 and the SSD paper: what changed in
    practice": one matrix, several contraction orders);
  * the blocked two-pass (chunked) contraction at many chunk lengths, including
    1 (the recurrence) and L (one dense block) (same section: chunks processed
    in parallel, then per-chunk states recombined);
  * closed forms: dt = 0 (state carried unchanged), A -> -inf (memoryless),
    L = 1, hand-worked rational examples, a first-order IIR filter
    (scipy.signal.lfilter) for P = N = 1 with constant coefficients;
  * invariants: state chaining across a split (fixed-size recurrent state,
    same page, first comparison table), linearity in (x, h0), causality,
    contiguous head->group map.
"""

from fractions import Fraction

import json
import os

import numpy as np
import pytest

from oracle import (
    causal_conv1d,
    dt_preprocess,
    chunk_cumsum,
    chunk_entry_states,
    chunk_local_states,
    group_of_head,
    ssd_chunked,
    ssd_quadratic,
    ssd_recurrent,
    ssd_semiseparable_matrix,
)


def rand_inputs(rng, b=2, L=23, H=4, P=3, N=5, G=2, h0=True, D=True, dt_scale=0.5):
    x = rng.standard_normal((b, L, H, P))
    dt = rng.uniform(0.0, dt_scale, (b, L, H))
    A = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), H))
    B = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    C = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    Dv = rng.standard_normal(H) if D else None
    hh = rng.standard_normal((b, H, P, N)) if h0 else None
    return x, dt, A, B, C, Dv, hh


def rel(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


SHAPES = [
    dict(b=1, L=1, H=1, P=1, N=1, G=1),
    dict(b=2, L=17, H=4, P=3, N=5, G=2),
    dict(b=1, L=40, H=6, P=4, N=2, G=3),
    dict(b=3, L=9, H=2, P=5, N=7, G=1),
    dict(b=1, L=31, H=4, P=2, N=3, G=4),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("with_h0", [False, True])
def test_recurrence_equals_dual_masked_form(shape, with_h0):
    rng = np.random.default_rng(1000 + shape["L"] + 7 * shape["H"] + with_h0)
    args = rand_inputs(rng, h0=with_h0, **shape)
    y_r, h_r = ssd_recurrent(*args)
    y_q, h_q = ssd_quadratic(*args)
    assert rel(y_r, y_q) < 1e-12
    assert rel(h_r, h_q) < 1e-12


@pytest.mark.parametrize("L", [1, 2, 5, 8])
def test_recurrence_equals_explicit_semiseparable_matrix(L):
    rng = np.random.default_rng(77 + L)
    x, dt, A, B, C, D, _ = rand_inputs(rng, b=2, L=L, H=4, P=3, N=4, G=2, h0=False)
    y_r, _ = ssd_recurrent(x, dt, A, B, C, D, None)
    for b in range(2):
        for h in range(4):
            M = ssd_semiseparable_matrix(dt, A, B, C, b, h)
            # lower triangular, with the diagonal present (y_t sees h_t)
            assert np.all(np.triu(M, 1) == 0)
            g = group_of_head(h, 4, 2)
            for t in range(L):
                assert M[t, t] == pytest.approx(dt[b, t, h] * np.dot(C[b, t, g], B[b, t, g]), rel=1e-14, abs=1e-300)
            y_m = M @ x[b, :, h, :] + D[h] * x[b, :, h, :]
            assert rel(y_r[b, :, h, :], y_m) < 1e-12


@pytest.mark.parametrize("Q", [1, 2, 3, 7, 16, 64])
@pytest.mark.parametrize("with_h0", [False, True])
def test_chunked_two_pass_equals_recurrence(Q, with_h0):
    rng = np.random.default_rng(5 + Q)
    args = rand_inputs(rng, b=2, L=45, H=4, P=3, N=4, G=2, h0=with_h0)
    y_r, h_r = ssd_recurrent(*args)
    y_c, h_c = ssd_chunked(*args, chunk=Q)
    assert rel(y_c, y_r) < 1e-11
    assert rel(h_c, h_r) < 1e-11


def test_dt_zero_carries_state_unchanged():
    rng = np.random.default_rng(3)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=2, L=13, H=4, P=3, N=5, G=2)
    dt = np.zeros_like(dt)
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    assert np.array_equal(hT, h0)
    # y_t = h0 C_t + D x_t, with the contiguous group map written per head
    for h in range(4):
        g = h // 2
        expect = np.einsum("bpn,btn->btp", h0[:, h], C[:, :, g]) + D[h] * x[:, :, h]
        assert rel(y[:, :, h], expect) < 1e-14


def test_A_to_minus_infinity_is_memoryless():
    rng = np.random.default_rng(4)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=2, L=11, H=4, P=3, N=5, G=2)
    dt = np.clip(dt, 0.01, None)
    A = np.full_like(A, -1e5)  # dt*A <= -1000: exp underflows to exactly 0
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    for h in range(4):
        g = h // 2
        cb = np.einsum("btn,btn->bt", C[:, :, g], B[:, :, g])
        expect = (dt[:, :, h] * cb)[..., None] * x[:, :, h] + D[h] * x[:, :, h]
        assert rel(y[:, :, h], expect) < 1e-13
        expect_h = dt[:, -1, h, None, None] * x[:, -1, h, :, None] * B[:, -1, g, None, :]
        assert rel(hT[:, h], expect_h) < 1e-13


def test_single_token_closed_form():
    rng = np.random.default_rng(9)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=2, L=1, H=2, P=3, N=4, G=1)
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    for b in range(2):
        for h in range(2):
            decay = np.exp(dt[b, 0, h] * A[h])
            hh = decay * h0[b, h] + dt[b, 0, h] * np.outer(x[b, 0, h], B[b, 0, 0])
            assert rel(hT[b, h], hh) < 1e-15
            assert rel(y[b, 0, h], hh @ C[b, 0, 0] + D[h] * x[b, 0, h]) < 1e-14


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def test_hand_worked_rational_example():
    # tests/golden/hand_worked_scalar_halving.json: P = N = 1, each step halves
    # the state; values derived by hand in exact rationals (derivation inside)
    g = _golden("hand_worked_scalar_halving.json")
    inp = g["inputs"]
    x = np.array(inp["x"], dtype=np.float64).reshape(1, 3, 1, 1)
    dt = np.array(inp["dt"], dtype=np.float64).reshape(1, 3, 1)
    assert inp["A"] == "-ln 2"
    A = np.array([-np.log(2.0)])
    B = np.array(inp["B"], dtype=np.float64).reshape(1, 3, 1, 1)
    C = np.array(inp["C"], dtype=np.float64).reshape(1, 3, 1, 1)
    D = np.array([inp["D"]])
    h0 = np.full((1, 1, 1, 1), float(inp["init_state"]))
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    for t, (num, den) in enumerate(g["expected"]["y"]):
        assert y[0, t, 0, 0] == pytest.approx(float(Fraction(num, den)), rel=1e-15)
    num, den = g["expected"]["final_state"]
    assert hT[0, 0, 0, 0] == pytest.approx(float(Fraction(num, den)), rel=1e-15)


def test_hand_worked_outer_product_example():
    # tests/golden/hand_worked_outer_product.json: two heads of one group,
    # P = N = 2, no decay; the state is a sum of outer products dt x B^T
    g = _golden("hand_worked_outer_product.json")
    inp, exp = g["inputs"], g["expected"]
    x = np.array(inp["x"], dtype=np.float64)[None]                      # [1, t, head, p]
    dt = np.full((1, 2, 2), float(inp["dt"]))
    A = np.array(inp["A"], dtype=np.float64)
    B = np.array(inp["B"], dtype=np.float64)[None, :, None, :]         # [1, t, 1, n]
    C = np.array(inp["C"], dtype=np.float64)[None, :, None, :]
    y, hT = ssd_recurrent(x, dt, A, B, C, None, None)
    assert np.allclose(y[0], np.array(exp["y"]), rtol=0, atol=1e-15)
    assert np.allclose(hT[0], np.array(exp["final_state"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("with_h0", [False, True])
def test_first_order_iir_filter(with_h0):
    scipy_signal = pytest.importorskip("scipy.signal")
    rng = np.random.default_rng(21)
    L = 200
    x = rng.standard_normal((1, L, 1, 1))
    dtv, Av, Bv, Cv, Dv, h0v = 0.07, -3.0, 0.8, -1.3, 0.4, 0.9
    dt = np.full((1, L, 1), dtv)
    A = np.array([Av])
    B = np.full((1, L, 1, 1), Bv)
    C = np.full((1, L, 1, 1), Cv)
    D = np.array([Dv])
    h0 = np.full((1, 1, 1, 1), h0v) if with_h0 else None
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    alpha = np.exp(dtv * Av)
    # (y - D x)_t = alpha (y - D x)_{t-1} + C dt B x_t
    zi = np.array([alpha * Cv * h0v]) if with_h0 else np.zeros(1)
    ref, _ = scipy_signal.lfilter([Cv * dtv * Bv], [1.0, -alpha], x[0, :, 0, 0], zi=zi)
    assert rel(y[0, :, 0, 0], ref + Dv * x[0, :, 0, 0]) < 1e-12
    assert hT[0, 0, 0, 0] == pytest.approx(ref[-1] / Cv, rel=1e-12)


@pytest.mark.parametrize("split", [1, 7, 30, 44])
def test_state_chaining_across_a_split(split):
    rng = np.random.default_rng(31 + split)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=2, L=45, H=4, P=3, N=4, G=2)
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    y1, h1 = ssd_quadratic(x[:, :split], dt[:, :split], A, B[:, :split], C[:, :split], D, h0)
    y2, h2 = ssd_quadratic(x[:, split:], dt[:, split:], A, B[:, split:], C[:, split:], D, h1)
    assert rel(np.concatenate([y1, y2], axis=1), y) < 1e-12
    assert rel(h2, hT) < 1e-12


def test_contiguous_head_to_group_map():
    rng = np.random.default_rng(8)
    H, G = 6, 2
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=1, L=12, H=H, P=2, N=3, G=G)
    y, hT = ssd_recurrent(x, dt, A, B, C, D, h0)
    # expand groups with an explicit loop: heads 0..2 -> group 0, 3..5 -> group 1
    Bx = np.stack([B[:, :, [0, 0, 0, 1, 1, 1][h]] for h in range(H)], axis=2)
    Cx = np.stack([C[:, :, [0, 0, 0, 1, 1, 1][h]] for h in range(H)], axis=2)
    y2, h2 = ssd_quadratic(x, dt, A, Bx, Cx, D, h0)
    assert rel(y, y2) < 1e-12 and rel(hT, h2) < 1e-12
    # and the map is NOT the interleaved one (h % G)
    Bw = np.stack([B[:, :, h % G] for h in range(H)], axis=2)
    Cw = np.stack([C[:, :, h % G] for h in range(H)], axis=2)
    y3, _ = ssd_quadratic(x, dt, A, Bw, Cw, D, h0)
    assert rel(y, y3) > 1e-3


def test_linear_in_x_and_initial_state_jointly():
    rng = np.random.default_rng(12)
    x1, dt, A, B, C, D, h1 = rand_inputs(rng, b=1, L=20, H=2, P=3, N=4, G=1)
    x2 = rng.standard_normal(x1.shape)
    h2 = rng.standard_normal(h1.shape)
    a, b = 0.7, -1.9
    y1, s1 = ssd_recurrent(x1, dt, A, B, C, D, h1)
    y2, s2 = ssd_recurrent(x2, dt, A, B, C, D, h2)
    y, s = ssd_recurrent(a * x1 + b * x2, dt, A, B, C, D, a * h1 + b * h2)
    assert rel(y, a * y1 + b * y2) < 1e-12
    assert rel(s, a * s1 + b * s2) < 1e-12


def test_causal():
    rng = np.random.default_rng(13)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=1, L=20, H=2, P=3, N=4, G=1)
    y, _ = ssd_recurrent(x, dt, A, B, C, D, h0)
    t0 = 9
    x2 = x.copy()
    x2[:, t0] += 5.0
    y2, _ = ssd_recurrent(x2, dt, A, B, C, D, h0)
    assert np.array_equal(y[:, :t0], y2[:, :t0])
    assert not np.allclose(y[:, t0], y2[:, t0])


# ---- intermediate quantities of the chunked path ---------------------------

@pytest.mark.parametrize("Q,L", [(4, 16), (5, 17), (8, 3)])
def test_chunk_cumsum_matches_decay_of_the_recurrence(Q, L):
    rng = np.random.default_rng(40 + Q + L)
    x, dt, A, B, C, D, _ = rand_inputs(rng, b=2, L=L, H=3, P=1, N=1, G=1)
    l = chunk_cumsum(dt, A, Q)
    nc = -(-L // Q)
    assert l.shape == (2, 3, nc, Q)
    for c in range(nc):
        t0, t1 = c * Q, min(L, (c + 1) * Q)
        # the pure decay over the chunk, observed through the recurrence
        # (x = 0, state starts at 1): exp of the chunk total
        zeros = np.zeros((2, t1 - t0, 3, 1))
        ones = np.ones((2, 3, 1, 1))
        _, hT = ssd_recurrent(zeros, dt[:, t0:t1], A, B[:, t0:t1], C[:, t0:t1], None, ones)
        assert rel(np.exp(l[:, :, c, -1]), hT[:, :, 0, 0]) < 1e-13
        # consecutive differences are the per-token log-decays; padded tail is flat
        for i in range(Q):
            t = t0 + i
            prev = l[:, :, c, i - 1] if i else 0.0
            step = l[:, :, c, i] - prev
            if t < L:
                assert np.allclose(step, dt[:, t, :] * A[None, :], rtol=1e-12, atol=1e-14)
            else:
                assert np.all(step == 0)


@pytest.mark.parametrize("Q,L", [(4, 16), (6, 17), (16, 16)])
def test_chunk_states_closed_form_and_recombination(Q, L):
    rng = np.random.default_rng(50 + Q + L)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=2, L=L, H=4, P=3, N=4, G=2)
    S = chunk_local_states(x, dt, A, B, Q)
    Hin, final = chunk_entry_states(x, dt, A, B, Q, h0)
    l = chunk_cumsum(dt, A, Q)
    nc = S.shape[2]
    for c in range(nc):
        t0, t1 = c * Q, min(L, (c + 1) * Q)
        lam = l[:, :, c, -1]
        # closed form of the local state: sum_j exp(Lam - l_j) dt_j x_j B_j^T
        for h in range(4):
            g = h // 2
            w = np.exp(lam[:, h, None] - l[:, h, c, : t1 - t0]) * dt[:, t0:t1, h]
            Sc = np.einsum("bj,bjp,bjn->bpn", w, x[:, t0:t1, h], B[:, t0:t1, g])
            assert rel(S[:, h, c], Sc) < 1e-12
        # entry state = the full state after token t0-1, from the dual form
        if c == 0:
            assert np.array_equal(Hin[:, :, 0], h0)
        else:
            _, hq = ssd_quadratic(x[:, :t0], dt[:, :t0], A, B[:, :t0], C[:, :t0], None, h0)
            assert rel(Hin[:, :, c], hq) < 1e-12
        # recombination: Hin_{c+1} = exp(Lam_c) Hin_c + S_c
        nxt = Hin[:, :, c + 1] if c + 1 < nc else final
        assert rel(nxt, np.exp(lam)[:, :, None, None] * Hin[:, :, c] + S[:, :, c]) < 1e-12


def test_oracle_rejects_bad_shapes():
    rng = np.random.default_rng(1)
    x, dt, A, B, C, D, h0 = rand_inputs(rng, b=1, L=4, H=3, P=2, N=2, G=2, h0=True)
    with pytest.raises(ValueError):
        ssd_recurrent(x, dt, A, B, C, D, h0)  # H % G != 0


# ---- dt preprocessing (bias, softplus, clamp) -----------------------------

def test_softplus_closed_forms():
    # softplus(0) = ln 2; softplus(ln(e^a - 1)) = a; softplus(z) - softplus(-z) = z
    assert dt_preprocess(np.array([0.0]), softplus=True)[0] == pytest.approx(np.log(2.0), rel=1e-15)
    a = np.array([1e-3, 0.1, 1.0, 7.5])
    assert np.allclose(dt_preprocess(np.log(np.expm1(a)), softplus=True), a, rtol=1e-13, atol=0)
    z = np.random.default_rng(40).normal(0, 5, 1000)
    sp = dt_preprocess(z, softplus=True)
    sn = dt_preprocess(-z, softplus=True)
    assert np.max(np.abs(sp - sn - z)) < 1e-12
    assert np.all(sp > 0) and np.all(sp >= z)
    # far in the tails: z itself above, e^z below, no overflow
    big = dt_preprocess(np.array([800.0, -800.0, 40.0]), softplus=True)
    assert big[0] == 800.0 and big[1] == 0.0 and big[2] == pytest.approx(40.0, rel=1e-15)


def test_dt_bias_goes_inside_the_softplus_and_clamp_comes_last():
    H = 5
    bias = np.linspace(-1.0, 1.0, H)
    dt = -np.tile(bias, (2, 3, 1))  # [b, L, H] with dt = -bias: softplus(0) everywhere
    out = dt_preprocess(dt, bias, softplus=True)
    assert np.allclose(out, np.log(2.0), rtol=1e-15, atol=0)
    # clamp after softplus: ln 2 ~ 0.693 is clipped to the upper limit
    out = dt_preprocess(dt, bias, softplus=True, limit=(0.1, 0.5))
    assert np.all(out == 0.5)
    out = dt_preprocess(dt, bias, softplus=True, limit=(0.9, 2.0))
    assert np.all(out == 0.9)
    # without softplus the bias is a plain per-head shift
    raw = np.zeros((1, 2, H))
    assert np.array_equal(dt_preprocess(raw, bias), np.broadcast_to(bias, raw.shape))


# ---- the short causal convolution -----------------------------------------

def test_conv_impulse_response_is_the_reversed_kernel():
    K, CH, L = 4, 3, 9
    w = np.random.default_rng(50).normal(size=(CH, K))
    u = np.zeros((1, L, CH))
    u[0, 2, :] = 1.0  # impulse at t = 2
    out, _ = causal_conv1d(u, w)
    for t in range(L):
        k = 2 + (K - 1) - t  # out[t] = w[k] with t - (K-1) + k = 2: the kernel reversed in time
        expect = w[:, k] if 0 <= k < K else np.zeros(CH)
        assert np.array_equal(out[0, t], expect)


def test_conv_equals_numpy_convolve_per_channel():
    rng = np.random.default_rng(51)
    K, CH, L = 3, 5, 40
    w = rng.normal(size=(CH, K))
    b = rng.normal(size=CH)
    u = rng.normal(size=(2, L, CH))
    out, last = causal_conv1d(u, w, b)
    for bb in range(2):
        for c in range(CH):
            ref = np.convolve(u[bb, :, c], w[c, ::-1])[:L] + b[c]  # causal: first L terms
            assert np.allclose(out[bb, :, c], ref, rtol=0, atol=1e-12)
    assert np.array_equal(last, np.transpose(u[:, L - (K - 1):, :], (0, 2, 1)))


def test_conv_state_carries_a_split_and_silu():
    rng = np.random.default_rng(52)
    K, CH, L, cut = 4, 6, 30, 11
    w = rng.normal(size=(CH, K))
    u = rng.normal(size=(1, L, CH))
    s0 = rng.normal(size=(1, CH, K - 1))
    whole, last = causal_conv1d(u, w, None, True, s0)
    a, sa = causal_conv1d(u[:, :cut], w, None, True, s0)
    b, sb = causal_conv1d(u[:, cut:], w, None, True, sa)
    assert np.allclose(np.concatenate([a, b], axis=1), whole, rtol=0, atol=1e-13)
    assert np.array_equal(sb, last)
    # silu(z) = z * sigmoid(z): zero at zero, z for large z, tends to 0 for very negative z
    z0, _ = causal_conv1d(np.zeros((1, 2, 1)), np.ones((1, K)), np.array([0.0]), True)
    assert np.all(z0 == 0.0)
    big, _ = causal_conv1d(np.zeros((1, 1, 2)), np.ones((2, 1)), np.array([40.0, -40.0]), True)
    assert big[0, 0, 0] == pytest.approx(40.0, rel=1e-15) and abs(big[0, 0, 1]) < 1e-15
