"""GPU parity: the HIP path against the CPU oracle (1e-4) and against itself (bit for bit).

Every call goes through libkda.so's C ABI via the Python binding.  Inputs come
from the seeded generator; expected values come only from the oracle.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_delta_rule_rows_amd as kda  # noqa: E402
from gated_delta_rule_rows_amd import synth  # noqa: E402
import oracle  # noqa: E402

TOL = 1e-4          # max abs error on outputs and states, GPU vs oracle
D = 128
SAMPLE_HEADS = [0, 21, 42, 63]


def dev(a):
    """numpy -> device tensor (float32, or bf16 from uint16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def rows_dev(r):
    return [dev(r[n]) for n in ("q", "k", "v", "g", "beta")]


def rows_np(r):
    return [r[n] for n in ("q", "k", "v", "g", "beta")]


def maxerr(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def bits_equal(a, b):
    a = host(a) if isinstance(a, torch.Tensor) else a
    b = host(b) if isinstance(b, torch.Tensor) else b
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b).view(np.uint32))


def scan(s_in, rows, want_o=True, inplace=False):
    L, T, H = rows[0].shape[:3]
    s_out = s_in if inplace else torch.empty_like(s_in)
    o = torch.empty(L, T, H, D, device="cuda") if want_o else None
    kda.kda_scan_rows(s_in, s_out, *rows, o=o)
    return s_out, o


def slice_rows(rows, t0, t1):
    return [x[:, t0:t1].contiguous() for x in rows]


def rand_rows(seed, L, T, H, bf16=False):
    r = synth.rows(seed, 0, L, T, H)
    if bf16:
        r = {n: synth.to_bf16_bits(a) for n, a in r.items()}
    return r


def rand_state(seed, L, H, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((L, H, D, D))).astype(np.float32)


# ----------------------------------------------------------------- oracle parity

def test_tiny_workload_rounds_with_replay():
    w = synth.WORKLOADS["tiny"]
    js = synth.accepts(w.seed, w.rounds, w.T - 1)
    s_gpu = torch.zeros(w.L, w.H, D, D, device="cuda")
    s_ref = np.zeros((w.L, w.H, D, D), np.float32)
    for r in range(w.rounds):
        rw = synth.rows(w.seed, r, w.L, w.T, w.H)
        rd = rows_dev(rw)
        s_full, o = scan(s_gpu, rd)
        S_ref, o_ref = oracle.scan_rows(s_ref, *rows_np(rw))
        assert maxerr(host(o), o_ref) <= TOL
        assert maxerr(host(s_full), S_ref) <= TOL
        keep = int(js[r]) + 1
        s_rep = torch.empty_like(s_gpu)
        kda.kda_replay(s_gpu, s_rep, *rd, keep=keep)     # s_gpu is the snapshot
        S_rep = oracle.replay(s_ref, *rows_np(rw), keep=keep)
        assert maxerr(host(s_rep), S_rep) <= TOL
        s_gpu, s_ref = s_rep, S_rep
    assert np.abs(s_ref).max() > 0.1   # non-vacuous: the state is populated


def test_one_layer_workload_replay_sweep():
    w = synth.WORKLOADS["one_layer"]
    warm = synth.warmup_rows(w.seed, w.warmup_rows, w.L, w.H)
    s0, _ = oracle.scan_rows(np.zeros((w.L, w.H, D, D), np.float32), *rows_np(warm),
                             want_o=False, threads=oracle.max_threads())
    rw = synth.rows(w.seed, 0, w.L, w.T, w.H)
    rd = rows_dev(rw)
    s_in = dev(s0)
    s_full, o = scan(s_in, rd)
    S_ref, o_ref = oracle.scan_rows(s0, *rows_np(rw), threads=oracle.max_threads())
    assert maxerr(host(o), o_ref) <= TOL
    assert maxerr(host(s_full), S_ref) <= TOL
    for j in range(w.T):
        keep = j + 1
        s_rep = torch.empty_like(s_in)
        kda.kda_replay(s_in, s_rep, *rd, keep=keep)
        S_rep = oracle.replay(s0, *rows_np(rw), keep=keep, threads=oracle.max_threads())
        assert maxerr(host(s_rep), S_rep) <= TOL, f"keep={keep}"
    assert bits_equal(s_in, dev(s0))   # the scan was out of place: the snapshot is intact


@pytest.mark.parametrize("L,T,H,bf16", [(1, 1, 1, False), (2, 15, 3, False), (3, 5, 7, True),
                                        (1, 15, 64, True)])
def test_ragged_shapes_vs_oracle(L, T, H, bf16):
    rw = rand_rows(7, L, T, H, bf16)
    s0 = rand_state(8, L, H, scale=0.5)
    s_out, o = scan(dev(s0), rows_dev(rw))
    S_ref, o_ref = oracle.scan_rows(s0, *rows_np(rw), threads=oracle.max_threads())
    assert maxerr(host(o), o_ref) <= TOL
    assert maxerr(host(s_out), S_ref) <= TOL


def test_verify_k14_full_size_sampled_chains():
    w = synth.WORKLOADS["verify_k14"]
    js = synth.accepts(w.seed, w.rounds, w.T - 1)
    s_gpu = torch.zeros(w.L, w.H, D, D, device="cuda")
    s_ref = np.zeros((w.L, len(SAMPLE_HEADS), D, D), np.float32)
    for r in range(3):
        rw = synth.rows(w.seed, r, w.L, w.T, w.H)
        rd = rows_dev(rw)
        s_full, o = scan(s_gpu, rd)
        sub = [x[:, :, SAMPLE_HEADS] for x in rows_np(rw)]
        S_ref, o_ref = oracle.scan_rows(s_ref, *sub, threads=oracle.max_threads())
        assert maxerr(host(o)[:, :, SAMPLE_HEADS], o_ref) <= TOL
        assert maxerr(host(s_full)[:, SAMPLE_HEADS], S_ref) <= TOL
        keep = int(js[r]) + 1
        if keep < w.T:
            s_rep = torch.empty_like(s_gpu)
            kda.kda_replay(s_gpu, s_rep, *rd, keep=keep)
            S_ref = oracle.replay(s_ref, *sub, keep=keep, threads=oracle.max_threads())
            assert maxerr(host(s_rep)[:, SAMPLE_HEADS], S_ref) <= TOL
            s_gpu = s_rep
        else:
            s_gpu = s_full
        s_ref = S_ref


def test_batched_b15_full_size_sampled_chains():
    w = synth.WORKLOADS["batched_b15"]
    sess = [0, 7, 14]
    states = torch.zeros(w.L, w.B, w.H, D, D, device="cuda")
    table = kda.state_table(states)
    s_ref = np.zeros((w.L, len(sess), len(SAMPLE_HEADS), D, D), np.float32)
    for step in range(2):
        rw = synth.rows(w.seed, step, w.L, w.B, w.H)      # [L][B][H][D]
        o = torch.empty(w.L, w.B, w.H, D, device="cuda")
        kda.kda_scan_batched(table, *rows_dev(rw), o=o)
        sub = [x[:, sess][:, :, SAMPLE_HEADS] for x in rows_np(rw)]
        s_ref, o_ref = oracle.batched(s_ref, *sub, threads=oracle.max_threads())
        got_s = host(states)[:, sess][:, :, SAMPLE_HEADS]
        got_o = host(o)[:, sess][:, :, SAMPLE_HEADS]
        assert maxerr(got_o, o_ref) <= TOL
        assert maxerr(got_s, s_ref) <= TOL


@pytest.mark.parametrize("K", [1, 14])
def test_serving_mix_bf16_sampled_chains(K):
    w = synth.WORKLOADS["serving_mix_bf16"]
    T = K + 1
    heads = SAMPLE_HEADS
    s_gpu = torch.zeros(w.L, w.H, D, D, device="cuda")
    s_ref = np.zeros((w.L, len(heads), D, D), np.float32)
    for r, j in enumerate([K, 0]):          # full accept, then worst-case j = 0
        rw = synth.rows_bf16(w.seed, r, w.L, T, w.H)
        rd = rows_dev(rw)
        s_full, o = scan(s_gpu, rd)
        sub = [x[:, :, heads] for x in rows_np(rw)]
        S_ref, o_ref = oracle.scan_rows(s_ref, *sub, threads=oracle.max_threads())
        assert maxerr(host(o)[:, :, heads], o_ref) <= TOL
        if j == K:
            s_gpu, s_ref = s_full, S_ref
        else:
            s_rep = torch.empty_like(s_gpu)
            kda.kda_replay(s_gpu, s_rep, *rd, keep=j + 1)
            s_ref = oracle.replay(s_ref, *sub, keep=j + 1, threads=oracle.max_threads())
            s_gpu = s_rep
        assert maxerr(host(s_gpu)[:, heads], s_ref) <= TOL


# ----------------------------------------------------------------- closed forms on the GPU

def test_gpu_identity_and_clamp_and_one_hot():
    L, T, H = 1, 6, 2
    rw = rand_rows(3, L, T, H)
    s0 = dev(rand_state(4, L, H))
    # beta = 0, g = 0: the state does not move (bit for bit)
    r0 = dict(rw, g=np.zeros_like(rw["g"]), beta=np.zeros_like(rw["beta"]))
    s1, _ = scan(s0, rows_dev(r0))
    assert bits_equal(s1, s0)
    # clamp: g = 0.7 acts as 0, g = -9 as -5
    for a, b in ((0.7, 0.0), (-9.0, -5.0)):
        ra = dict(rw, g=np.full_like(rw["g"], a))
        rb = dict(rw, g=np.full_like(rw["g"], b))
        sa, oa = scan(s0, rows_dev(ra))
        sb, ob = scan(s0, rows_dev(rb))
        assert bits_equal(sa, sb) and bits_equal(oa, ob)
    # one-hot key from zero state writes v into key row m exactly
    m = 77
    k = np.zeros((1, 1, 1, D), np.float32); k[..., m] = 1
    v = np.random.default_rng(5).standard_normal((1, 1, 1, D)).astype(np.float32)
    r1 = [dev(k), dev(k), dev(v), dev(np.zeros_like(k)), dev(np.ones((1, 1, 1), np.float32))]
    sz, _ = scan(torch.zeros(1, 1, D, D, device="cuda"), r1)
    sz = host(sz)
    assert np.array_equal(sz[0, 0, m], v[0, 0, 0])
    assert not np.delete(sz[0, 0], m, axis=0).any()


def test_gpu_keeps_f32_denormals_like_the_oracle():
    # beta = 0, g = -5 on every row: each row multiplies the state by the one
    # decay factor d.  Reading d back after one row, 19 rows from S = 1 must
    # equal 19 IEEE f32 multiplies by d (numpy keeps denormals): the state
    # falls to about 5e-42, below the smallest normal f32, and is not flushed
    L, H = 1, 1
    rng = np.random.default_rng(7)
    def rows(T):
        q = rng.standard_normal((L, T, H, D)).astype(np.float32)
        k = rng.standard_normal((L, T, H, D)).astype(np.float32)
        v = rng.standard_normal((L, T, H, D)).astype(np.float32)
        g = np.full((L, T, H, D), -5.0, np.float32)
        b = np.zeros((L, T, H), np.float32)
        return [dev(x) for x in (q, k, v, g, b)]
    one = torch.ones(L, H, D, D, device="cuda")
    s1, _ = scan(one, rows(1))
    d = host(s1)[0, 0, 0, 0]
    assert np.all(host(s1) == d) and 0 < d < 1
    s = one
    for T in (15, 4):
        s, _ = scan(s, rows(T))
    ref = np.float32(1.0)
    for _ in range(19):
        ref = np.float32(ref * d)
    assert 0 < ref < np.finfo(np.float32).tiny
    got = host(s)
    assert np.all(got.view(np.int32) == np.float32(ref).view(np.int32)), (got.max(), ref)


def test_snapshot_is_a_bit_copy():
    s = dev(rand_state(6, 3, 5))
    snap = torch.full_like(s, float("nan"))
    kda.kda_snapshot(s, snap)
    assert bits_equal(snap, s)


# ----------------------------------------------------------------- GPU bit-identity gates

@pytest.mark.parametrize("T,bf16", [(2, False), (8, False), (15, False), (15, True)])
def test_t_row_launch_equals_chained_single_rows(T, bf16):
    L, H = 3, 5
    rd = rows_dev(rand_rows(11, L, T, H, bf16))
    s0 = dev(rand_state(12, L, H))
    s_T, o_T = scan(s0, rd)
    s = s0
    for t in range(T):
        s, o1 = scan(s, slice_rows(rd, t, t + 1))
        assert bits_equal(o1[:, 0], o_T[:, t]), f"row {t}"
    assert bits_equal(s, s_T)


@pytest.mark.parametrize("bf16", [False, True])
def test_replay_equals_state_after_keep_rows(bf16):
    L, T, H = 2, 15, 4
    rd = rows_dev(rand_rows(13, L, T, H, bf16))
    snap = dev(rand_state(14, L, H))
    s_full, _ = scan(snap, rd)
    chained = snap
    for keep in range(1, T + 1):
        chained, _ = scan(chained, slice_rows(rd, keep - 1, keep))
        s_rep = torch.empty_like(snap)
        kda.kda_replay(snap, s_rep, *rd, keep=keep)
        assert bits_equal(s_rep, chained), f"keep={keep}"
        s_k, _ = scan(snap, slice_rows(rd, 0, keep), want_o=False)
        assert bits_equal(s_rep, s_k)
    s_rep = torch.empty_like(snap)
    kda.kda_replay(snap, s_rep, *rd, keep=T)
    assert bits_equal(s_rep, s_full)     # keep == T returns the resident bits


@pytest.mark.parametrize("B,bf16", [(1, False), (7, True), (15, False)])
def test_batched_equals_isolated_single_rows(B, bf16):
    L, H = 2, 3
    rw = rand_rows(15, L, B, H, bf16)        # [L][B][H][D]
    rd = rows_dev(rw)
    init = rand_state(16, L * B, H).reshape(L, B, H, D, D)
    states = dev(init)
    o = torch.empty(L, B, H, D, device="cuda")
    kda.kda_scan_batched(kda.state_table(states), *rd, o=o)
    for l in range(L):
        for b in range(B):
            one = [x[l:l + 1, b:b + 1].contiguous() for x in rd]
            s1, o1 = scan(dev(init[l:l + 1, b]), one)
            assert bits_equal(s1[0], states[l, b])
            assert bits_equal(o1[0, 0], o[l, b])


def test_batched_with_scattered_session_buffers():
    L, B, H = 3, 4, 2
    rd = rows_dev(rand_rows(17, L, B, H))
    init = rand_state(18, L * B, H).reshape(L, B, H, D, D)
    bufs = [[dev(init[l, b]) for b in range(B)] for l in range(L)]
    kda.kda_scan_batched(kda.state_table(bufs), *rd)
    ref = dev(init)
    kda.kda_scan_batched(kda.state_table(ref), *rd)
    for l in range(L):
        for b in range(B):
            assert bits_equal(bufs[l][b], ref[l, b])


def test_in_place_equals_out_of_place_and_runs_repeat():
    L, T, H = 2, 9, 6
    rd = rows_dev(rand_rows(19, L, T, H))
    s0 = dev(rand_state(20, L, H))
    a, oa = scan(s0, rd)
    b, ob = scan(s0, rd)
    c = s0.clone()
    _, oc = scan(c, rd, inplace=True)
    assert bits_equal(a, b) and bits_equal(oa, ob)
    assert bits_equal(a, c) and bits_equal(oa, oc)


def test_no_outputs_leaves_state_bits_unchanged():
    L, T, H = 2, 7, 3
    rd = rows_dev(rand_rows(21, L, T, H))
    s0 = dev(rand_state(22, L, H))
    a, _ = scan(s0, rd, want_o=True)
    b, _ = scan(s0, rd, want_o=False)
    assert bits_equal(a, b)


def test_chains_do_not_interact_on_gpu():
    L, T, H = 3, 4, 5
    rw = rand_rows(23, L, T, H)
    s0 = rand_state(24, L, H)
    a, oa = scan(dev(s0), rows_dev(rw))
    ph = [4, 2, 0, 3, 1]
    rp = {n: np.ascontiguousarray(x[:, :, ph]) for n, x in rw.items()}
    b, ob = scan(dev(np.ascontiguousarray(s0[:, ph])), rows_dev(rp))
    assert bits_equal(host(a)[:, ph], b)
    assert bits_equal(host(oa)[:, :, ph], ob)


# ----------------------------------------------------------------- red arms

def test_red_arms_diverge():
    """A wrong rollback must be visible: skipping the replay after a partial
    accept, or replaying from the post-scan state, changes the state bits."""
    L, T, H = 1, 8, 4
    rd = rows_dev(rand_rows(25, L, T, H))
    snap = dev(rand_state(26, L, H))
    s_full, _ = scan(snap, rd)
    keep = 3
    good = torch.empty_like(snap)
    kda.kda_replay(snap, good, *rd, keep=keep)
    # red 1: no replay -- the resident post-row-K state stands in for the rollback
    n1 = int((host(s_full).view(np.uint32) != host(good).view(np.uint32)).sum())
    # red 2: replay from the wrong snapshot (the post-scan state)
    bad = torch.empty_like(snap)
    kda.kda_replay(s_full, bad, *rd, keep=keep)
    n2 = int((host(bad).view(np.uint32) != host(good).view(np.uint32)).sum())
    assert n1 > 0 and n2 > 0, (n1, n2)
    # non-vacuity: the scan really moved the state away from the snapshot
    assert not bits_equal(s_full, snap)
    # and continuing one more row from each keeps them apart
    nxt = slice_rows(rows_dev(rand_rows(27, L, 1, H)), 0, 1)
    c_good, _ = scan(good, nxt)
    c_bad, _ = scan(s_full, nxt)
    assert not bits_equal(c_good, c_bad)


# ----------------------------------------------------------------- stash plane and fused round

def scan_e(s_in, rows):
    L, T, H = rows[0].shape[:3]
    s_out = torch.empty_like(s_in)
    o = torch.empty(L, T, H, D, device="cuda")
    e = torch.empty(L, T, H, D, device="cuda")
    kda.kda_scan_rows_stash(s_in, s_out, *rows, o, e)
    return s_out, o, e


@pytest.mark.parametrize("bf16", [False, True])
def test_stash_replay_equals_recomputed_replay(bf16):
    L, T, H = 2, 15, 5
    rd = rows_dev(rand_rows(31, L, T, H, bf16))
    snap = dev(rand_state(32, L, H))
    s_full, o, e = scan_e(snap, rd)
    s2, o2 = scan(snap, rd)            # writing the stash plane changes nothing else
    assert bits_equal(s_full, s2) and bits_equal(o, o2)
    for keep in range(1, T + 1):
        a = torch.empty_like(snap)
        kda.kda_replay(snap, a, *rd, keep=keep)
        b = torch.empty_like(snap)
        kda.kda_replay_stash(snap, b, rd[1], rd[3], e, keep=keep)
        assert bits_equal(a, b), f"keep={keep}"
    assert bits_equal(b, s_full)       # keep == T: the resident bits


def _prev(rows, e, stash):
    k, v, g, beta = rows[1:]
    return (k, None, g, None, e) if stash else (k, v, g, beta, None)


@pytest.mark.parametrize("bf16,stash", [(False, False), (False, True), (True, True)])
def test_verify_round_equals_replay_then_scan(bf16, stash):
    L, H, T_prev, T = 2, 5, 15, 8
    prev = rows_dev(rand_rows(33, L, T_prev, H, bf16))
    cur = rows_dev(rand_rows(34, L, T, H, bf16))
    snap_prev = dev(rand_state(35, L, H))
    _, _, e_prev = scan_e(snap_prev, prev)
    for keep in (0, 1, 7, T_prev):
        if keep:
            ref_snap = torch.empty_like(snap_prev)
            kda.kda_replay(snap_prev, ref_snap, *prev, keep=keep)
        else:
            ref_snap = snap_prev
        _, ref_o, ref_e = scan_e(ref_snap, cur)
        snap_out = torch.empty_like(snap_prev)
        o = torch.empty(L, T, H, D, device="cuda")
        e = torch.empty(L, T, H, D, device="cuda")
        kda.kda_verify_round(snap_prev, snap_out, _prev(prev, e_prev, stash) if keep else None,
                             keep, *cur, o, e=e)
        assert bits_equal(snap_out, ref_snap), f"keep={keep}"
        assert bits_equal(o, ref_o) and bits_equal(e, ref_e), f"keep={keep}"
    # in place
    x = snap_prev.clone()
    o = torch.empty(L, T, H, D, device="cuda")
    kda.kda_verify_round(x, x, _prev(prev, e_prev, stash), 7, *cur, o)
    ref_snap = torch.empty_like(snap_prev)
    kda.kda_replay(snap_prev, ref_snap, *prev, keep=7)
    assert bits_equal(x, ref_snap)


def max_ulp(a, ref):
    """Largest |a - ref| in units of ref's f32 spacing, over the elements at
    least 1/256 of the largest magnitude (near zero the spacing is so fine that
    any rounding reads as millions of ulp)."""
    ref = np.asarray(ref, np.float32)
    big = np.abs(ref) >= np.abs(ref).max() / 256
    d = np.abs(np.asarray(a, np.float64) - ref.astype(np.float64))[big]
    return float((d / np.spacing(np.abs(ref[big])).astype(np.float64)).max())


def _fused_pipeline(w, rounds, heads, bf16=False, stash=True, Ts=None, log=None):
    """Run `rounds` fused verify rounds of workload w on the GPU and the matching
    scan/replay chain on the oracle (sampled heads); compare every round.  With
    `log` (a list), append (round, max |d| state, max ulp state, max |d| o,
    max ulp o) per round."""
    js = synth.accepts(w.seed, max(rounds, 1), w.T - 1)
    snap = torch.zeros(w.L, w.H, D, D, device="cuda")
    ref = np.zeros((w.L, len(heads), D, D), np.float32)
    prev = None
    for r in range(rounds):
        T = Ts[r] if Ts else w.T
        rw = synth.rows_bf16(w.seed, r, w.L, T, w.H) if bf16 else synth.rows(w.seed, r, w.L, T, w.H)
        cur = rows_dev(rw)
        o = torch.empty(w.L, T, w.H, D, device="cuda")
        e = torch.empty(w.L, T, w.H, D, device="cuda")
        nxt = torch.empty_like(snap)
        if prev is None:
            kda.kda_verify_round(snap, nxt, None, 0, *cur, o, e=e)
        else:
            p_rows, p_e, keep = prev
            kda.kda_verify_round(snap, nxt, _prev(p_rows, p_e, stash), keep, *cur, o, e=e)
        snap = nxt
        sub = [x[:, :, heads] for x in rows_np(rw)]
        _, o_ref = oracle.scan_rows(ref, *sub, threads=oracle.max_threads())
        got_s, got_o = host(snap)[:, heads], host(o)[:, :, heads]
        if log is not None:
            log.append((r, maxerr(got_s, ref), max_ulp(got_s, ref), maxerr(got_o, o_ref),
                        max_ulp(got_o, o_ref)))
        assert maxerr(got_s, ref) <= TOL, f"round {r} snapshot"
        assert maxerr(got_o, o_ref) <= TOL, f"round {r} outputs"
        keep = int(js[r] % T) + 1
        ref = oracle.replay(ref, *sub, keep=keep, threads=oracle.max_threads())
        prev = (cur, e, keep)
    return ref


def test_fused_pipeline_tiny_vs_oracle():
    _fused_pipeline(synth.WORKLOADS["tiny"], 4, [0])


def test_fused_pipeline_verify_k14_sampled_vs_oracle():
    _fused_pipeline(synth.WORKLOADS["verify_k14"], 3, SAMPLE_HEADS)


def test_long_chain_drift_verify_k14_all_rounds():
    # all 32 rounds of the headline workload, 480 rows per chain: the error
    # against the oracle is logged per round so a drift over long chains shows
    w = synth.WORKLOADS["verify_k14"]
    log = []
    _fused_pipeline(w, w.rounds, SAMPLE_HEADS, log=log)
    print("\nround  max|d| state  max ulp state  max|d| o  max ulp o   (ulp over |ref| >= max/256)")
    for r, ds, us, do, uo in log:
        print(f"{r:5d}  {ds:12.3e}  {us:13.1f}  {do:8.3e}  {uo:9.1f}")
    # a steady error, not one that grows with the chain: the last 8 rounds may
    # not be worse than 4x the first 8
    first = max(x[1] for x in log[:8])
    last = max(x[1] for x in log[-8:])
    assert last <= 4 * first + 1e-7, f"state error grows along the chain: {first} -> {last}"


def test_very_long_chain_small_shape_drift():
    # 300 fused rounds of 15 rows on 2 layers x 4 heads (4,500 rows per chain),
    # every chain against the oracle each round: the error stays at rounding
    # level and does not grow with the chain
    w = synth.Workload("long_small", L=2, H=4, T=15, rounds=300, seed=5)
    log = []
    _fused_pipeline(w, w.rounds, list(range(w.H)), log=log)
    worst = max(x[1] for x in log)
    print(f"\n300 rounds: worst max|d| state {worst:.3e}, worst max ulp state "
          f"{max(x[2] for x in log):.1f}, worst max|d| o {max(x[3] for x in log):.3e}")
    first = max(x[1] for x in log[:50])
    last = max(x[1] for x in log[-50:])
    assert last <= 4 * first + 1e-7, f"state error grows along the chain: {first} -> {last}"


def test_fused_pipeline_serving_mix_bf16_sampled_vs_oracle():
    w = synth.WORKLOADS["serving_mix_bf16"]
    Ks = synth.serving_ks(w.seed, 3)
    _fused_pipeline(w, 3, SAMPLE_HEADS, bf16=True, stash=False, Ts=[int(k) + 1 for k in Ks])


# ----------------------------------------------------------------- tilings

def _per_layers(fn, L, chunk):
    """Run fn(l0, l1) on layer chunks [l0, l1) and return the pieces in order."""
    return [fn(l0, min(l0 + chunk, L)) for l0 in range(0, L, chunk)]


@pytest.mark.parametrize("chunk,bf16,L,H", [(1, False, 34, 64), (4, False, 34, 64),
                                            (8, False, 34, 64), (1, True, 34, 64),
                                            (4, True, 34, 64), (1, False, 17, 64),
                                            (8, False, 24, 64), (17, False, 68, 64),
                                            (1, False, 34, 8), (17, True, 34, 8),
                                            (5, False, 25, 12), (17, False, 34, 16),
                                            (4, False, 28, 16), (6, True, 40, 6),
                                            (100, False, 300, 1), (3, False, 41, 7)])
def test_layer_chunked_launches_match_the_full_launch_bit_for_bit(chunk, bf16, L, H):
    # 1 layer = 64 chains (4 workgroups per head), 4 layers = 256 chains
    # (2 per head), 8 layers = 512 chains (1 per head): every tiling must
    # give the bits of the full launch, for the scan, both replays and the
    # fused round.  The full launch itself ends in a split tail: at 34 layers
    # its last 128 chains run 2 workgroups per head, at 17 layers its last 64
    # chains 4 per head.  24 layers (1,536 chains) and 68 layers (4,352
    # chains, 17-layer pieces of 1,088) end in tails too large to split.
    # 34 x 8 = 272 and 25 x 12 = 300 chains run whole heads on 256 chains and
    # quarter heads on the rest, against pieces of 8 to 136 chains; 34 x 16 =
    # 544 chains two rounds of whole heads and 32 chains at 4 per head
    # (pieces of 272), 28 x 16 = 448 chains whole heads only (pieces of 64),
    # 40 x 6 = 240 chains half heads (pieces of 36, quarter heads); one head
    # per layer (300 x 1) and an odd head count (41 x 7 = 287) in split tails.
    T = 15
    r = rand_rows(91, L, T, H, bf16=bf16)
    rows = rows_dev(r)
    s0 = dev(rand_state(92, L, H, 0.5))
    s_full, o_full = scan(s0, rows)
    e_full = torch.empty(L, T, H, D, device="cuda")
    kda.kda_scan_rows_stash(s0, torch.empty_like(s0), *rows, torch.empty_like(o_full), e_full)
    rep_full = torch.empty_like(s0)
    kda.kda_replay(s0, rep_full, *rows, keep=6)
    reps_full = torch.empty_like(s0)
    kda.kda_replay_stash(s0, reps_full, rows[1], rows[3], e_full, keep=9)
    snap_full, o2_full = torch.empty_like(s0), torch.empty_like(o_full)
    kda.kda_verify_round(s0, snap_full, (rows[1], None, rows[3], None, e_full), 11, *rows, o2_full)
    torch.cuda.synchronize()

    def lay(x, l0, l1):
        return x[l0:l1].contiguous()

    def piece(l0, l1):
        rr = [lay(x, l0, l1) for x in rows]
        si = lay(s0, l0, l1)
        so, oo = scan(si, rr)
        rp = torch.empty_like(si)
        kda.kda_replay(si, rp, *rr, keep=6)
        el = lay(e_full, l0, l1)
        rps = torch.empty_like(si)
        kda.kda_replay_stash(si, rps, rr[1], rr[3], el, keep=9)
        sn, o2 = torch.empty_like(si), torch.empty_like(oo)
        kda.kda_verify_round(si, sn, (rr[1], None, rr[3], None, el), 11, *rr, o2)
        return so, oo, rp, rps, sn, o2

    parts = _per_layers(piece, L, chunk)
    torch.cuda.synchronize()
    got = [torch.cat([p[i] for p in parts]) for i in range(6)]
    for name, a, b in zip(("state", "o", "replay", "stash replay", "round snap", "round o"),
                          got, (s_full, o_full, rep_full, reps_full, snap_full, o2_full)):
        assert bits_equal(a, b), f"{name} differs at chunk {chunk}"


# ----------------------------------------------------------------- multi-round replay

@pytest.mark.parametrize("L,keeps,store,stash,bf16", [
    (2, [], True, True, False),              # no earlier round: a plain scan from snap_base
    (2, [5], True, True, False),             # one round, two stage areas
    (2, [3, 0, 8], False, True, False),      # a round with nothing kept is skipped
    (2, [2, 7], True, False, True),          # recomputed replay, bf16
    (3, [5, 9], True, True, False),          # 192 chains: 2 workgroups per head, one stage area
    (12, [4, 1, 12, 9], True, True, False),  # 768 chains, one workgroup per head
    (12, [6, 6], False, False, False),
    (17, [3, 8], True, True, True),          # 1,088 chains: the last 64 split 4 ways
    (34, [9, 2, 5], False, False, False),    # 2,176 chains: the last 128 split 2 ways
])
def test_verify_round_multi_equals_replays_then_scan(L, keeps, store, stash, bf16):
    H, T = 64, 15
    s0 = dev(rand_state(71, L, H, 0.5))
    prevs, ref = [], s0.clone()
    for n, keep in enumerate(keeps):
        Tn = [15, 9, 12, 15][n]
        r = rows_dev(rand_rows(72 + n, L, Tn, H, bf16=bf16))
        e_n = torch.empty(L, Tn, H, D, device="cuda")
        kda.kda_scan_rows_stash(ref, torch.empty_like(ref), *r, None, e_n)
        if keep:
            nxt = torch.empty_like(ref)
            if stash:
                kda.kda_replay_stash(ref, nxt, r[1], r[3], e_n, keep=keep)
            else:
                kda.kda_replay(ref, nxt, *r, keep=keep)
            ref = nxt
        if stash:
            prevs.append((r[1], None, r[3], None, e_n, keep))
        else:
            prevs.append((r[1], r[2], r[3], r[4], None, keep))
    cur = rows_dev(rand_rows(80, L, T, H, bf16=bf16))
    _, o_ref, e_ref = scan_e(ref, cur)
    snap_out = torch.empty_like(s0) if store else None
    o = torch.empty(L, T, H, D, device="cuda")
    e = torch.empty(L, T, H, D, device="cuda")
    kda.kda_verify_round_multi(s0, snap_out, prevs, *cur, o, e=e)
    torch.cuda.synchronize()
    if store:
        assert bits_equal(snap_out, ref)
    assert bits_equal(o, o_ref) and bits_equal(e, e_ref)


def test_verify_round_multi_in_place_and_refusals():
    L, H, T = 2, 8, 6
    s0 = dev(rand_state(81, L, H, 0.5))
    r1 = rows_dev(rand_rows(82, L, 10, H))
    e1 = torch.empty(L, 10, H, D, device="cuda")
    kda.kda_scan_rows_stash(s0, torch.empty_like(s0), *r1, None, e1)
    cur = rows_dev(rand_rows(83, L, T, H))
    ref = torch.empty_like(s0)
    kda.kda_replay_stash(s0, ref, r1[1], r1[3], e1, keep=4)
    x = s0.clone()
    o = torch.empty(L, T, H, D, device="cuda")
    kda.kda_verify_round_multi(x, x, [(r1[1], None, r1[3], None, e1, 4)], *cur, o)
    torch.cuda.synchronize()
    assert bits_equal(x, ref)
    with pytest.raises(kda.KdaError, match="all or none"):
        kda.kda_verify_round_multi(s0, None, [(r1[1], None, r1[3], None, e1, 4),
                                              (r1[1], r1[2], r1[3], r1[4], None, 2)], *cur, o)
    with pytest.raises(ValueError, match="at most 4"):
        kda.kda_verify_round_multi(s0, None, [(r1[1], None, r1[3], None, e1, 1)] * 5, *cur, o)
