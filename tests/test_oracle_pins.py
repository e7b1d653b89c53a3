"""Pins for the CPU oracle: closed forms, invariants, exact and brute-force cases.

Each test ties the oracle to something other than itself: exact rational
arithmetic, an independent matrix form of the update, an IEEE closed form, a
numpy routine, or a property the delta rule must have.  Together they are
meant to fail for a dropped term, a wrong sign, a transposed operand, the
wrong clamp bound, the wrong output scale, o read before the update, or a
wrong layout stride.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

F32_EPS = 2.0 ** -23  # f32 ulp at 1.0


def _rand_rows(rng, L, T, H, d, gmin=-5.0, gmax=0.0):
    q = rng.standard_normal((L, T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((L, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, T, H, d))
    g = rng.uniform(gmin, gmax, (L, T, H, d))
    beta = rng.uniform(0.0, 1.0, (L, T, H))
    f = lambda a: a.astype(np.float32)
    return f(q), f(k), f(v), f(g), f(beta)


# ---------------------------------------------------------------- identity / decay / clamp

def test_identity_beta0_g0_leaves_state_and_reads_it():
    rng = np.random.default_rng(10)
    d, T = 128, 5
    S0 = rng.standard_normal((1, 1, d, d)).astype(np.float32)
    q, k, v, _, _ = _rand_rows(rng, 1, T, 1, d)
    g = np.zeros_like(q)
    beta = np.zeros((1, T, 1), np.float32)
    S, o = oracle.scan_rows(S0, q, k, v, g, beta)
    assert np.array_equal(S.view(np.uint32), S0.view(np.uint32))
    for t in range(T):
        ref = S0[0, 0].astype(np.float64).T @ q[0, t, 0].astype(np.float64) / np.sqrt(d)
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=0, atol=4 * F32_EPS * np.abs(ref).max())


def test_decay_closed_form():
    # beta = 0: S_T[i][j] = exp(sum_t clamp(g_t[i])) * S_0[i][j]
    rng = np.random.default_rng(11)
    d, T = 128, 15
    S0 = rng.standard_normal((1, 1, d, d)).astype(np.float32)
    q, k, v, g, _ = _rand_rows(rng, 1, T, 1, d, gmin=-7.0, gmax=1.0)  # some out of range
    beta = np.zeros((1, T, 1), np.float32)
    S, _ = oracle.scan_rows(S0, q, k, v, g, beta, want_o=False)
    gc = np.clip(g[0, :, 0].astype(np.float64), -5.0, 0.0).sum(axis=0)
    ref = np.exp(gc)[:, None] * S0[0, 0].astype(np.float64)
    rel = np.abs(S[0, 0] - ref) / np.maximum(np.abs(ref), 1e-30)
    # one f32 rounding per row plus the f64 exps: well inside (T+1) half-ulps
    assert rel.max() <= (T + 1) * 0.5 * F32_EPS * 1.01


def test_clamp_bounds_are_exactly_minus5_and_0():
    rng = np.random.default_rng(12)
    d, T = 128, 6
    S0 = rng.standard_normal((1, 1, d, d)).astype(np.float32)
    q, k, v, _, beta = _rand_rows(rng, 1, T, 1, d)
    def run(gval):
        g = np.full_like(q, gval)
        return oracle.scan_rows(S0, q, k, v, g, beta)
    for a, b in ((0.7, 0.0), (-9.0, -5.0), (3.0e30, 0.0), (-1.0e30, -5.0)):
        Sa, oa = run(a)
        Sb, ob = run(b)
        assert np.array_equal(Sa.view(np.uint32), Sb.view(np.uint32))
        assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
    # and inside the range the gate does act
    S1, _ = run(-1.0)
    S0_, _ = run(0.0)
    assert not np.array_equal(S1, S0_)


# ---------------------------------------------------------------- writes

def test_one_hot_key_writes_value_into_that_key_row():
    rng = np.random.default_rng(13)
    d = 128
    for m in (0, 37, 127):
        S0 = np.zeros((1, 1, d, d), np.float32)
        k = np.zeros((1, 1, 1, d), np.float32); k[..., m] = 1.0
        q = k.copy()
        v = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
        g = np.zeros_like(k)
        beta = np.ones((1, 1, 1), np.float32)
        S, o = oracle.scan_rows(S0, q, k, v, g, beta)
        assert np.array_equal(S[0, 0, m], v[0, 0, 0])          # key row m == v, bit-exact
        others = np.delete(S[0, 0], m, axis=0)
        assert not others.any()                               # every other key row stays 0
        ref = v[0, 0, 0].astype(np.float64) / np.sqrt(d)
        ulp = np.spacing(np.abs(ref).astype(np.float32))
        assert (np.abs(o[0, 0, 0] - ref) <= ulp).all()


def test_all_one_hot_keys_write_matrix_exactly():
    rng = np.random.default_rng(14)
    d = 128
    T = d
    S0 = np.zeros((1, 1, d, d), np.float32)
    k = np.zeros((1, T, 1, d), np.float32)
    perm = rng.permutation(d)
    for t in range(T):
        k[0, t, 0, perm[t]] = 1.0
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    S, _ = oracle.scan_rows(S0, k, k, v, np.zeros_like(k), np.ones((1, T, 1), np.float32),
                            want_o=False)
    V = np.empty((d, d), np.float32)
    V[perm] = v[0, :, 0]
    assert np.array_equal(S[0, 0], V)


def test_associative_memory_with_orthonormal_keys():
    # beta = 1, g = 0, orthonormal keys: after writing (k_m, v_m), S^T k_m = v_m.
    rng = np.random.default_rng(15)
    d, M = 128, 64
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q[:M].astype(np.float32)
    vals = rng.standard_normal((M, d)).astype(np.float32)
    S0 = np.zeros((1, 1, d, d), np.float32)
    k = keys[None, :, None, :]
    v = vals[None, :, None, :]
    S, _ = oracle.scan_rows(S0, k, k, v, np.zeros_like(k), np.ones((1, M, 1), np.float32),
                            want_o=False)
    recall = keys.astype(np.float64) @ S[0, 0].astype(np.float64)   # row m = S^T k_m
    # keys are orthonormal only to f32 rounding (~1e-7 per entry); the residual
    # cross-talk over 64 writes stays below 1e-5
    assert np.abs(recall - vals).max() < 1e-5


def test_norm_bound_every_row():
    # ||k|| = 1, 0 <= beta <= 1, g <= 0  =>  ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||
    rng = np.random.default_rng(16)
    d, T = 128, 15
    S = rng.standard_normal((1, 1, d, d)).astype(np.float32)
    q, k, v, g, beta = _rand_rows(rng, 1, T, 1, d)
    for t in range(T):
        sl = slice(t, t + 1)
        Sn, _ = oracle.scan_rows(S, q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl],
                                 want_o=False)
        lhs = np.linalg.norm(Sn.astype(np.float64))
        rhs = np.linalg.norm(S.astype(np.float64)) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert lhs <= rhs * (1 + 1e-6)
        S = Sn


# ---------------------------------------------------------------- exact and brute force

def _frac_scan(S, qs, ks, vs, betas):
    """Exact rational recurrence with g = 0 (no decay) and d = len(S)."""
    d = len(S)
    S = [row[:] for row in S]
    outs = []
    for q, k, v, b in zip(qs, ks, vs, betas):
        u = [sum(k[i] * S[i][j] for i in range(d)) for j in range(d)]
        e = [b * (v[j] - u[j]) for j in range(d)]
        S = [[S[i][j] + k[i] * e[j] for j in range(d)] for i in range(d)]
        # 1/sqrt(4) = 1/2 exactly
        outs.append([sum(q[i] * S[i][j] for i in range(d)) / 2 for j in range(d)])
    return S, outs


def _f32_exact(x: Fraction) -> bool:
    f = np.float32(float(x))
    return Fraction(float(f)) == x


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
def test_exact_rational_d4(seed):
    """d = 4 with dyadic inputs: every intermediate is exact in f64 and every
    result exact in f32, so the oracle must reproduce the rational answer bit for bit."""
    rng = np.random.default_rng(100 + seed)
    d, T = 4, 3
    halves = [Fraction(x, 2) for x in (-2, -1, 0, 1, 2)]
    quarters = [Fraction(x, 4) for x in range(-4, 5)]
    S0 = [[quarters[rng.integers(len(quarters))] for _ in range(d)] for _ in range(d)]
    qs = [[halves[rng.integers(5)] for _ in range(d)] for _ in range(T)]
    ks = [[halves[rng.integers(5)] for _ in range(d)] for _ in range(T)]
    vs = [[halves[rng.integers(5)] for _ in range(d)] for _ in range(T)]
    bs = [Fraction(int(rng.integers(1, 5)), 4) for _ in range(T)]
    S_ex, o_ex = _frac_scan(S0, qs, ks, vs, bs)
    assert all(_f32_exact(x) for row in S_ex for x in row)
    assert all(_f32_exact(x) for row in o_ex for x in row)
    A = lambda rows: np.array([[float(x) for x in r] for r in rows], np.float32)
    S, o = oracle.scan_rows(A(S0)[None, None], A(qs)[None, :, None], A(ks)[None, :, None],
                            A(vs)[None, :, None], np.zeros((1, T, 1, d), np.float32),
                            np.array([float(b) for b in bs], np.float32)[None, :, None])
    assert np.array_equal(S[0, 0], A(S_ex))
    assert np.array_equal(o[0, :, 0], A(o_ex))
    # non-vacuity: the case really moves the state
    assert not np.array_equal(A(S_ex), A(S0))


def _matrix_form(S0, q, k, v, g, beta):
    """S_t = (I - beta k k^T) D_t S_{t-1} + beta k v^T, f64 per row, f32 state."""
    d = S0.shape[0]
    S = S0.astype(np.float32)
    outs = []
    for t in range(q.shape[0]):
        kk = k[t].astype(np.float64)
        Dt = np.diag(np.exp(np.clip(g[t].astype(np.float64), -5.0, 0.0)))
        P = np.eye(d) - float(beta[t]) * np.outer(kk, kk)
        Sn = P @ Dt @ S.astype(np.float64) + float(beta[t]) * np.outer(kk, v[t].astype(np.float64))
        outs.append((Sn.T @ q[t].astype(np.float64)) / np.sqrt(d))
        S = Sn.astype(np.float32)
    return S, np.array(outs)


@pytest.mark.parametrize("d,T,seed", [(4, 6, 0), (4, 15, 1), (8, 9, 2), (16, 4, 3)])
def test_matrix_form_with_decay(d, T, seed):
    rng = np.random.default_rng(200 + seed)
    S0 = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal((T, d)).astype(np.float32)
    k = rng.standard_normal((T, d)).astype(np.float32)   # not normalised on purpose
    v = rng.standard_normal((T, d)).astype(np.float32)
    g = rng.uniform(-7.0, 1.0, (T, d)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, T).astype(np.float32)
    S_ref, o_ref = _matrix_form(S0, q, k, v, g, beta)
    S, o = oracle.scan_rows(S0[None, None], q[None, :, None], k[None, :, None], v[None, :, None],
                            g[None, :, None], beta[None, :, None])
    # both sides compute each row in f64 and round the state to f32: they can part
    # only by a last-place rounding flip, which then propagates through the chain
    scale = max(1.0, np.abs(S_ref).max())
    assert np.abs(S[0, 0] - S_ref).max() <= 64 * F32_EPS * scale
    assert np.abs(o[0, :, 0] - o_ref).max() <= 64 * F32_EPS * max(1.0, np.abs(o_ref).max())


# ---------------------------------------------------------------- replay, batched, layout

def test_replay_is_the_scan_prefix():
    rng = np.random.default_rng(17)
    L, T, H, d = 2, 8, 3, 128
    S0 = rng.standard_normal((L, H, d, d)).astype(np.float32)
    rows = _rand_rows(rng, L, T, H, d)
    S_full, o_full = oracle.scan_rows(S0, *rows)
    for keep in (1, 3, T):
        Sr = oracle.replay(S0, *rows, keep=keep)
        sl = [x[:, :keep] for x in rows]
        Sk, ok = oracle.scan_rows(S0, *sl)
        assert np.array_equal(Sr, Sk)
        assert np.array_equal(ok, o_full[:, :keep])
    assert np.array_equal(oracle.replay(S0, *rows, keep=T), S_full)


def test_batched_equals_isolated_single_rows():
    rng = np.random.default_rng(18)
    L, B, H, d = 2, 5, 3, 128
    states = rng.standard_normal((L, B, H, d, d)).astype(np.float32)
    q, k, v, g, beta = _rand_rows(rng, L, B, H, d)   # [L][B][H][d]: B in the row slot
    Sb, ob = oracle.batched(states, q, k, v, g, beta)
    for l in range(L):
        for b in range(B):
            sl = lambda x: x[l:l + 1, b:b + 1]
            S1, o1 = oracle.scan_rows(states[l:l + 1, b], sl(q), sl(k), sl(v), sl(g), sl(beta))
            assert np.array_equal(S1[0], Sb[l, b])
            assert np.array_equal(o1[0, 0], ob[l, b])


def test_chains_are_independent_and_layout_strides_are_right():
    rng = np.random.default_rng(19)
    L, T, H, d = 3, 4, 5, 128
    S0 = rng.standard_normal((L, H, d, d)).astype(np.float32)
    q, k, v, g, beta = _rand_rows(rng, L, T, H, d)
    S, o = oracle.scan_rows(S0, q, k, v, g, beta)
    # every chain run alone, through a 1x1 layout, gives the same bits
    for l in range(L):
        for h in range(H):
            sl = lambda x: x[l:l + 1, :, h:h + 1]
            S1, o1 = oracle.scan_rows(S0[l:l + 1, h:h + 1], sl(q), sl(k), sl(v), sl(g), sl(beta))
            assert np.array_equal(S1[0, 0], S[l, h])
            assert np.array_equal(o1[0, :, 0], o[l, :, h])
    # permuting heads and layers permutes the results
    ph, pl = rng.permutation(H), rng.permutation(L)
    P = lambda x: x[pl][:, :, ph]
    Sp, op = oracle.scan_rows(S0[pl][:, ph], P(q), P(k), P(v), P(g), beta[pl][:, :, ph])
    assert np.array_equal(Sp, S[pl][:, ph])
    assert np.array_equal(op, o[pl][:, :, ph])


def test_threads_do_not_change_bits():
    rng = np.random.default_rng(20)
    L, T, H, d = 2, 3, 4, 128
    S0 = rng.standard_normal((L, H, d, d)).astype(np.float32)
    rows = _rand_rows(rng, L, T, H, d)
    a = oracle.scan_rows(S0, *rows, threads=1)
    b = oracle.scan_rows(S0, *rows, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- bf16 inputs

# (bf16 bits, exact value) from the IEEE binary16-brain layout: 1 sign, 8 exponent
# (bias 127), 7 mantissa bits.
BF16_TABLE = [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0xC040, -3.0), (0x3F00, 0.5),
    (0x3FC0, 1.5), (0x4120, 10.0), (0x3E80, 0.25), (0x0000, 0.0), (0x3F81, 1.0 + 2.0 ** -7),
    (0x0080, 2.0 ** -126), (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0xC2C8, -100.0),
]


def test_bf16_widening_matches_ieee_table():
    # write the bf16 values with a one-hot key from zero state: key row m == widened v
    d = 128
    bits = np.zeros(d, np.uint16)
    vals = np.zeros(d, np.float64)
    for n, (b, x) in enumerate(BF16_TABLE):
        bits[n], vals[n] = b, x
    one = 0x3F80
    k = np.zeros((1, 1, 1, d), np.uint16); k[..., 5] = one
    v = bits[None, None, None, :]
    g = np.zeros_like(k)
    beta = np.full((1, 1, 1), one, np.uint16)
    S, _ = oracle.scan_rows(np.zeros((1, 1, d, d), np.float32), k, k, v, g, beta, want_o=False)
    assert np.array_equal(S[0, 0, 5].astype(np.float64), vals)


def test_bf16_scan_equals_f32_scan_of_torch_widened_values():
    torch = pytest.importorskip("torch")
    from gated_delta_rule_rows_amd import synth
    rng = np.random.default_rng(21)
    L, T, H, d = 1, 5, 2, 128
    S0 = rng.standard_normal((L, H, d, d)).astype(np.float32)
    rows = _rand_rows(rng, L, T, H, d)
    bits = [synth.to_bf16_bits(x) for x in rows]
    widened = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
               for b in bits]
    a = oracle.scan_rows(S0, *bits)
    b = oracle.scan_rows(S0, *widened)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- greedy accept

def test_accept_argmax_matches_numpy_first_occurrence():
    rng = np.random.default_rng(40)
    for t, V in ((1, 1), (3, 32), (15, 1000), (4, 4097)):
        lg = rng.standard_normal((t, V)).astype(np.float32)
        lg[:, rng.integers(V)] += 0.0
        vam, _, _ = oracle.accept_greedy(lg, np.zeros(t - 1, np.uint32))
        assert np.array_equal(vam, np.argmax(lg, axis=1).astype(np.uint32))


def test_accept_tie_break_and_special_values():
    ninf, pinf = -np.inf, np.inf
    rows = np.array([
        [1.0, 5.0, 2.0, 5.0, 5.0],      # ties: lowest index (1)
        [ninf, ninf, ninf, ninf, ninf],  # all -inf: index 0
        [0.0, pinf, 3.0, pinf, 1.0],     # first +inf
        [-0.0, 0.0, -1.0, -0.0, -2.0],   # +0 == -0: index 0
        [2.0, 1.0, np.nan, 3.0, 0.0],    # a NaN anywhere: sentinel
        [np.nan, 1.0, 2.0, 3.0, 4.0],    # NaN first: sentinel
    ], np.float32)
    vam, _, _ = oracle.accept_greedy(rows, np.zeros(len(rows) - 1, np.uint32))
    assert vam.tolist() == [1, 0, 1, 0, 0xFFFFFFFF, 0xFFFFFFFF]


@pytest.mark.parametrize("m", [0, 1, 3, 7])
def test_accept_prefix_walk(m):
    # row r's argmax is planted at position p[r]; drafts agree on the first m rows
    rng = np.random.default_rng(50 + m)
    t, V = 8, 64
    lg = rng.uniform(-1, 0, (t, V)).astype(np.float32)
    p = rng.integers(V, size=t)
    lg[np.arange(t), p] = 1.0
    drafts = p[: t - 1].copy()
    if m < t - 1:
        drafts[m] = (p[m] + 1) % V          # first disagreement at draft m
    vam, j, bonus = oracle.accept_greedy(lg, drafts)
    assert j == m and bonus == p[m]
    assert np.array_equal(vam, p.astype(np.uint32))


def test_accept_single_row_and_bf16():
    lg = np.array([[0.5, 2.0, 2.0]], np.float32)
    vam, j, bonus = oracle.accept_greedy(lg, [])
    assert (vam.tolist(), j, bonus) == ([1], 0, 1)
    from gated_delta_rule_rows_amd import synth
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    bits = synth.to_bf16_bits(x)
    wide = (bits.astype(np.uint32) << 16).view(np.float32)
    vam, _, _ = oracle.accept_greedy(bits, np.zeros(4, np.uint32))
    assert np.array_equal(vam, np.argmax(wide, axis=1).astype(np.uint32))


# ---------------------------------------------------------------- conv ring re-roll

def _ring_case(seed, L=2, T=6, C=5):
    rng = np.random.default_rng(seed)
    snap = rng.standard_normal((L, 3, C)).astype(np.float32)
    raw = rng.standard_normal((L, T, C)).astype(np.float32)
    return snap, raw


@pytest.mark.parametrize("keep", [1, 2, 3, 4, 6])
def test_reroll_is_the_last_three_rows_of_snapshot_then_kept_rows(keep):
    # closed form: the committed ring is the window of the last 3 entries of the
    # sequence (ring rows 0..2, raw rows 0..keep-1), oldest first
    snap, raw = _ring_case(60 + keep)
    out = oracle.conv_reroll(snap, raw, keep)
    seq = np.concatenate([snap, raw[:, :keep]], axis=1)
    assert np.array_equal(out, seq[:, -3:])
    if keep >= 3:
        assert np.array_equal(out, raw[:, keep - 3:keep])


def test_reroll_composes_and_keeps_layers_apart():
    snap, raw = _ring_case(70, L=3, T=7, C=9)
    full = oracle.conv_reroll(snap, raw, 5)
    # rolling 2 rows, then the next 3 from that ring, is rolling 5
    mid = oracle.conv_reroll(snap, raw, 2)
    two_step = oracle.conv_reroll(mid, np.ascontiguousarray(raw[:, 2:]), 3)
    assert np.array_equal(full, two_step)
    # each layer depends on its own ring and rows only
    raw2 = raw.copy()
    raw2[1] += 1.0
    out2 = oracle.conv_reroll(snap, raw2, 5)
    assert np.array_equal(out2[0], full[0]) and np.array_equal(out2[2], full[2])
    assert not np.array_equal(out2[1], full[1])


def test_reroll_bf16_rows_widen_exactly():
    from gated_delta_rule_rows_amd import synth
    snap, raw = _ring_case(80)
    bits = synth.to_bf16_bits(raw)
    wide = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.conv_reroll(snap, bits, 4), oracle.conv_reroll(snap, wide, 4))
    with pytest.raises(ValueError):
        oracle.conv_reroll(snap, raw, 0)
    with pytest.raises(ValueError):
        oracle.conv_reroll(snap, raw, 7)


# ---------------------------------------------------------------- pre-scan row ops

LN3 = float(np.log(3.0))


def _ops_inputs(L, T, H, d, seed=0, taps=None):
    rng = np.random.default_rng(seed)
    C = 3 * H * d
    x = rng.standard_normal((L, T, C)).astype(np.float32)
    a = rng.standard_normal((L, T, H * d)).astype(np.float32)
    b = rng.standard_normal((L, T, H)).astype(np.float32)
    if taps is None:
        w = rng.uniform(-0.6, 0.6, (L, C, 4)).astype(np.float32)
    else:
        w = np.broadcast_to(np.asarray(taps, np.float32), (L, C, 4)).copy()
    ring = rng.standard_normal((L, 3, C)).astype(np.float32)
    return x, a, b, w, ring


def test_row_ops_identity_taps_give_silu_closed_forms():
    # taps (0,0,0,1): the conv passes the current row, so v = SiLU(x);
    # SiLU(0) = 0, SiLU(ln 3) = (3/4) ln 3, SiLU(-ln 3) = -(1/4) ln 3
    L, T, H, d = 1, 2, 2, 4
    x, a, b, w, ring = _ops_inputs(L, T, H, d, taps=(0, 0, 0, 1))
    HD = H * d
    x[0, 0, 2 * HD:] = [0, LN3, -LN3, 0, LN3, LN3, 0, -LN3]
    out = oracle.row_ops(x, a, b, w, ring, H, d)
    want = np.array([0, 0.75 * LN3, -0.25 * LN3, 0, 0.75 * LN3, 0.75 * LN3, 0, -0.25 * LN3])
    np.testing.assert_allclose(out["v"][0, 0].reshape(-1), want, rtol=1e-6, atol=1e-7)


def test_row_ops_taps_reach_back_through_the_ring():
    # taps (1,0,0,0): row t sees the raw input three rows earlier, from the
    # ring for t < 3 and from the round's own rows after that
    L, T, H, d = 1, 5, 1, 4
    x, a, b, w, ring = _ops_inputs(L, T, H, d, taps=(1, 0, 0, 0))
    v0 = 2 * H * d
    ring[0, :, v0:] = 0.0
    ring[0, 0, v0] = LN3         # oldest ring row -> output row 0
    ring[0, 2, v0 + 1] = -LN3    # newest ring row -> output row 2
    x[0, :, v0:] = 0.0
    x[0, 0, v0 + 2] = LN3        # round row 0 -> output row 3
    x[0, 1, v0 + 3] = LN3        # round row 1 -> output row 4
    out = oracle.row_ops(x, a, b, w, ring, H, d)
    v = out["v"][0, :, 0, :]
    want = np.zeros((5, 4))
    want[0, 0] = 0.75 * LN3
    want[2, 1] = -0.25 * LN3
    want[3, 2] = 0.75 * LN3
    want[4, 3] = 0.75 * LN3
    np.testing.assert_allclose(v, want, rtol=1e-6, atol=1e-7)


def test_row_ops_norms_gate_and_beta_closed_forms():
    L, T, H, d = 1, 1, 3, 4
    x, a, b, w, ring = _ops_inputs(L, T, H, d, taps=(0, 0, 0, 1))
    HD = H * d
    x[0, 0, :2 * HD] = 0.0
    x[0, 0, 0] = LN3             # q head 0 = SiLU(ln 3) e_0 -> unit vector e_0
    x[0, 0, HD + 4 + 1] = 1.0    # k head 1 = SiLU(1) e_1 -> e_1
    a[0, 0, :] = 0.0             # softplus(0) = ln 2
    a[0, 0, 4] = 10.0            # -softplus(10) < -5: the bound
    a[0, 0, 5] = float(np.log(np.e ** 2 - 1))   # softplus = 2
    a[0, 0, 6] = -20.0           # ~ -2.06e-9
    b[0, 0, :] = [0.0, LN3, -LN3]
    out = oracle.row_ops(x, a, b, w, ring, H, d)
    q, k, g = out["q"][0, 0], out["k"][0, 0], out["g"][0, 0]
    # unit vectors up to the 1e-6 under the square root; zero rows stay zero
    np.testing.assert_allclose(q[0], [1, 0, 0, 0], atol=2e-6)
    np.testing.assert_array_equal(q[1], 0)
    np.testing.assert_allclose(k[1], [0, 1, 0, 0], atol=2e-6)
    np.testing.assert_array_equal(k[0], 0)
    assert g[0, 0] == np.float32(-np.log(2.0))
    assert g[1, 0] == -5.0 and g[1, 1] == np.float32(-2.0)
    np.testing.assert_allclose(g[1, 2], -np.exp(-20.0), rtol=1e-6)
    np.testing.assert_allclose(out["beta"][0, 0], [0.5, 0.75, 0.25], rtol=1e-7)
    # normalised rows have unit length whatever the conv produced
    x2, a2, b2, w2, r2 = _ops_inputs(2, 3, 2, 8, seed=4)
    o2 = oracle.row_ops(x2, a2, b2, w2, r2, 2, 8)
    for n in ("q", "k"):
        np.testing.assert_allclose(np.linalg.norm(o2[n], axis=-1), 1.0, rtol=1e-5)


def test_row_ops_norm_epsilon_dominates_small_rows():
    # reading r15 fixes the norm as y / sqrt(sum y^2 + 1e-6).  With one nonzero
    # channel per head, q = y / sqrt(y^2 + eps): at y^2 = eps the row comes out
    # at 1/sqrt(2), not 1, and the three heads below tell eps = 1e-6 apart
    # from 1e-7, 1e-8 or 0 by far more than any rounding.
    L, T, H, d = 1, 1, 3, 4
    x, a, b, w, ring = _ops_inputs(L, T, H, d, taps=(0, 0, 0, 2))
    HD = H * d
    x[0, 0, :2 * HD] = 0.0
    # conv output = SiLU(2 x); pick x so that y^2 is 1e-4, 1e-6, 1e-8 (to a
    # few parts in 1e3: SiLU(z) = z / (1 + e^-z) ~ z / 2 for small z)
    ys = np.array([1e-2, 1e-3, 1e-4])
    for h, y in enumerate(ys):
        x[0, 0, h * d] = y             # q block, head h, channel 0
        x[0, 0, HD + h * d + 1] = y    # k block, head h, channel 1
    out = oracle.row_ops(x, a, b, w, ring, H, d)
    z = 2.0 * x[0, 0, :HD].astype(np.float64)
    y = z / (1.0 + np.exp(-z))          # SiLU of the conv output, f64
    for h in range(H):
        yq = y[h * d]
        want = yq / np.sqrt(yq * yq + 1e-6)
        np.testing.assert_allclose(out["q"][0, 0, h, 0], want, rtol=1e-6)
        np.testing.assert_allclose(out["k"][0, 0, h, 1], want, rtol=1e-6)
        assert np.all(out["q"][0, 0, h, 1:] == 0) and out["k"][0, 0, h, 0] == 0
    # y^2 = eps (head 1, to 0.2%): the unit row shrinks to about 1/sqrt(2)
    assert abs(out["q"][0, 0, 1, 0] - 2 ** -0.5) < 2e-3
    # y^2 = 1e-2 eps: about 0.1, and y^2 = 100 eps: within 0.5% of 1
    assert abs(out["q"][0, 0, 2, 0] - 0.1) < 1e-3
    assert abs(out["q"][0, 0, 0, 0] - 1.0) < 6e-3


def test_row_ops_split_rounds_chain_through_the_ring():
    # causality: rows 0..2 then rows 3..5 (ring carried) equal rows 0..5;
    # the ring after the round is the conv-ring roll of all T rows
    L, T, H, d = 2, 6, 2, 8
    x, a, b, w, ring = _ops_inputs(L, T, H, d, seed=9)
    full = oracle.row_ops(x, a, b, w, ring, H, d)
    first = oracle.row_ops(x[:, :3].copy(), a[:, :3].copy(), b[:, :3].copy(), w, ring, H, d)
    second = oracle.row_ops(x[:, 3:].copy(), a[:, 3:].copy(), b[:, 3:].copy(), w,
                            first["ring"], H, d)
    for n in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(np.concatenate([first[n], second[n]], axis=1), full[n])
    np.testing.assert_array_equal(full["ring"], oracle.conv_reroll(ring, x, T))


def test_row_ops_channels_heads_and_layers_stay_apart():
    L, T, H, d = 2, 3, 3, 8
    x, a, b, w, ring = _ops_inputs(L, T, H, d, seed=12)
    base = oracle.row_ops(x, a, b, w, ring, H, d)
    HD = H * d
    x2 = x.copy()
    x2[1, 1, HD + 2 * d + 3] += 1.0   # layer 1, row 1, a k channel of head 2
    o = oracle.row_ops(x2, a, b, w, ring, H, d)
    changed = {n: np.argwhere(o[n] != base[n]) for n in ("q", "k", "v", "g", "beta")}
    assert changed["q"].size == 0 and changed["v"].size == 0 and changed["g"].size == 0
    assert changed["beta"].size == 0
    # the raw input of row 1 also reaches rows 2.. through the causal conv
    ks = set(map(tuple, changed["k"][:, :3]))
    assert ks == {(1, 1, 2), (1, 2, 2)}


def test_row_ops_bf16_inputs_widen_exactly():
    from gated_delta_rule_rows_amd import synth
    L, T, H, d = 1, 4, 2, 8
    x, a, b, w, ring = _ops_inputs(L, T, H, d, seed=15)
    bits = [synth.to_bf16_bits(z) for z in (x, a, b)]
    wide = [(z.astype(np.uint32) << 16).view(np.float32) for z in bits]
    o1 = oracle.row_ops(*bits, w, ring, H, d)
    o2 = oracle.row_ops(*wide, w, ring, H, d)
    for n in ("q", "k", "v", "g", "beta", "ring"):
        np.testing.assert_array_equal(o1[n], o2[n])
