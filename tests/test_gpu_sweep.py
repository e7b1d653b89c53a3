"""A seeded sweep of launch shapes against the oracle.

Each case draws layers L, heads H (so 1 to ~600 chains: every tiling, and
fused rounds on both sides of the two-stage-area threshold), T and keep from
their full ranges, f32 or bf16 rows, and the stash plane or not.  It runs a
fused round from a random committed state and the split pipeline beside it,
and checks both against the oracle (1e-4) and against each other (bit for bit).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth
import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-4
D = 128
N_CASES = 24


def _cases():
    rng = np.random.default_rng(2024)
    out = []
    for i in range(N_CASES):
        H = int(rng.choice([1, 2, 3, 5, 8, 16, 64]))
        L = int(rng.integers(1, max(2, 600 // H) + 1))
        T = int(rng.integers(1, 16))
        T_prev = int(rng.integers(1, 16))
        keep = int(rng.integers(0, T_prev + 1))
        out.append((i, L, H, T, T_prev, keep, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


def _dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"c{c[0]}-L{c[1]}H{c[2]}T{c[3]}"
                         f"p{c[4]}k{c[5]}{'bf16' if c[6] else 'f32'}{'-stash' if c[7] else ''}")
def test_sweep_fused_and_split_vs_oracle(case):
    i, L, H, T, T_prev, keep, bf16, stash = case
    names = ("q", "k", "v", "g", "beta")
    gen = synth.rows_bf16 if bf16 else synth.rows
    prev_np = gen(500 + i, 0, L, T_prev, H)
    cur_np = gen(500 + i, 1, L, T, H)
    prev = [_dev(prev_np[n]) for n in names]
    cur = [_dev(cur_np[n]) for n in names]
    rng = np.random.default_rng(600 + i)
    S0 = (0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32)
    s0 = _dev(S0)

    # the previous round's stash plane, from its own scan
    e_prev = torch.empty(L, T_prev, H, D, device="cuda")
    kda.kda_scan_rows_stash(s0, torch.empty_like(s0), *prev, None, e_prev)

    # fused round
    snap = torch.empty_like(s0)
    o = torch.empty(L, T, H, D, device="cuda")
    e = torch.empty(L, T, H, D, device="cuda")
    p = (prev[1], None, prev[3], None, e_prev) if stash else (prev[1], prev[2], prev[3], prev[4], None)
    kda.kda_verify_round(s0, snap, p if keep else None, keep, *cur, o, e=e)

    # split pipeline: replay, then an out-of-place scan
    rep = torch.empty_like(s0)
    if keep:
        if stash:
            kda.kda_replay_stash(s0, rep, prev[1], prev[3], e_prev, keep=keep)
        else:
            kda.kda_replay(s0, rep, *prev, keep=keep)
    else:
        rep.copy_(s0)
    s_after = torch.empty_like(s0)
    o2 = torch.empty_like(o)
    kda.kda_scan_rows(rep, s_after, *cur, o=o2)
    torch.cuda.synchronize()

    assert np.array_equal(_bits(snap), _bits(rep)), "fused snapshot != replay"
    assert np.array_equal(_bits(o), _bits(o2)), "fused o != split o"

    # oracle on a sample of chains (all of them when few)
    heads = sorted(set([0, H - 1, H // 2]))
    sub = lambda r: [r[n][:, :, heads] for n in names]
    S_ref = S0[:, heads]
    if keep:
        S_ref = oracle.replay(S_ref, *sub(prev_np), keep=keep, threads=oracle.max_threads())
    S_end, o_ref = oracle.scan_rows(S_ref, *sub(cur_np), threads=oracle.max_threads())
    assert float(np.abs(snap.cpu().numpy()[:, heads] - S_ref).max()) <= TOL
    assert float(np.abs(o.cpu().numpy()[:, :, heads] - o_ref).max()) <= TOL
    assert float(np.abs(s_after.cpu().numpy()[:, heads] - S_end).max()) <= TOL
