"""Speculative rounds against the never-drafted chain, bit for bit.

The plain decode chain runs one-row launches over the committed rows only.  A
speculative round scans all of its T draft rows, commits keep = j + 1 of them
and rolls the state back to the last committed row.  For every j, the round's
committed outputs, the rolled-back state, and a continuation of one-row steps
after it must carry exactly the bits of the plain chain (the accept-j gate of
glm5_spec_ppn_gate.rs, with the chained t = 1 program as the reference arm).
A multi-round session of fused rounds with drafted T and j drawn per round
must likewise reproduce the plain chain's outputs for every committed row.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_delta_rule_rows_amd as kda  # noqa: E402
from gated_delta_rule_rows_amd import synth  # noqa: E402

D = 128
NAMES = ("q", "k", "v", "g", "beta")


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def rows(seed, index, L, T, H, bf16=False):
    r = (synth.rows_bf16 if bf16 else synth.rows)(seed, index, L, T, H)
    return [dev(r[n]) for n in NAMES]


def part(rd, t0, t1):
    return [x[:, t0:t1].contiguous() for x in rd]


def same(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def step(s, rd):
    """One-row launch: the plain chain's step."""
    L, _, H = rd[0].shape[:3]
    s2 = torch.empty_like(s)
    o = torch.empty(L, 1, H, D, device="cuda")
    kda.kda_scan_rows(s, s2, *rd, o=o)
    return s2, o


@pytest.mark.parametrize("bf16", [False, True])
def test_accept_j_then_continue_equals_never_drafted_chain(bf16):
    L, H, T, n_cont = 2, 4, 8, 12
    draft = rows(80, 0, L, T, H, bf16)
    cont = rows(80, 1, L, n_cont, H, bf16)
    rng = np.random.default_rng(81)
    s0 = dev((0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32))

    # speculative scan of all T drafts, out of place: s0 stays as the snapshot
    s_all = torch.empty_like(s0)
    o_all = torch.empty(L, T, H, D, device="cuda")
    kda.kda_scan_rows(s0, s_all, *draft, o=o_all)

    for j in range(T):
        keep = j + 1
        # rollback: replay the kept rows from the snapshot (no work at full accept)
        if keep < T:
            s = torch.empty_like(s0)
            kda.kda_replay(s0, s, *draft, keep=keep)
        else:
            s = s_all
        # the never-drafted chain over the committed rows
        p = s0
        for t in range(keep):
            p, o1 = step(p, part(draft, t, t + 1))
            assert same(o1[:, 0], o_all[:, t]), f"j={j}: committed row {t} output"
        assert same(s, p), f"j={j}: rolled-back state"
        # continue both for n_cont one-row steps
        for c in range(n_cont):
            r1 = part(cont, c, c + 1)
            s, os_ = step(s, r1)
            p, op = step(p, r1)
            assert same(os_, op), f"j={j}: continuation step {c} output"
        assert same(s, p), f"j={j}: state after the continuation"
    # non-vacuity: a partial accept really differs from the full-accept state
    part_state = torch.empty_like(s0)
    kda.kda_replay(s0, part_state, *draft, keep=1)
    assert not same(part_state, s_all)


@pytest.mark.parametrize("stash", [False, True])
def test_fused_session_equals_never_drafted_chain(stash):
    """Eight fused rounds with T and j drawn per round; every committed row's
    output and the committed state match the plain chain of one-row steps."""
    L, H, rounds = 2, 3, 8
    rng = np.random.default_rng(82)
    Ts = [int(x) for x in rng.integers(1, 16, rounds)]
    js = [int(rng.integers(0, t)) for t in Ts]
    snap = dev((0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32))
    chain = snap.clone()
    prev = None
    for r, (T, j) in enumerate(zip(Ts, js)):
        rd = rows(83, r, L, T, H)
        e = torch.empty(L, T, H, D, device="cuda")
        o = torch.empty(L, T, H, D, device="cuda")
        nxt = torch.empty_like(snap)
        if prev is None:
            kda.kda_verify_round(snap, nxt, None, 0, *rd, o, e=e)
        else:
            p_rd, p_e, p_keep = prev
            p = (p_rd[1], None, p_rd[3], None, p_e) if stash else \
                (p_rd[1], p_rd[2], p_rd[3], p_rd[4], None)
            kda.kda_verify_round(snap, nxt, p, p_keep, *rd, o, e=e)
        snap = nxt   # the state after the previous round's committed rows
        assert same(snap, chain), f"round {r}: committed state entering the round"
        keep = j + 1
        for t in range(keep):
            chain, o1 = step(chain, part(rd, t, t + 1))
            assert same(o1[:, 0], o[:, t]), f"round {r}: committed row {t} output"
        prev = (rd, e, keep)
    # the last round's commit, by a plain replay
    p_rd, _, p_keep = prev
    last = torch.empty_like(snap)
    kda.kda_replay(snap, last, *p_rd, keep=p_keep)
    assert same(last, chain)
