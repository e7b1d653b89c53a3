"""Pre-scan row ops on the GPU against the oracle.

kda_row_ops computes in f32 (a fixed fmaf chain for the conv, the hardware
exp for SiLU, softplus and sigmoid); the oracle in f64.  Outputs are O(1)
(q, k unit rows; v, g in [-5, 0], beta in (0, 1)), so an absolute 1e-5 bound
leaves room for a few f32 roundings and catches any wrong term.  The conv
ring after the round must match bit for bit (it is moved, not computed).
End to end, row ops feeding kda_scan_rows must match the oracle's row ops
feeding the oracle's scan within the scan's 1e-4.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth
import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _run(inp, L, T, H, bf16=False):
    dev = {}
    for n in ("x", "a", "b"):
        if bf16:
            bits = synth.to_bf16_bits(inp[n])
            dev[n] = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            dev[n] = torch.from_numpy(inp[n]).cuda()
    w = torch.from_numpy(inp["w"]).cuda()
    ring = torch.from_numpy(inp["ring"]).cuda()
    out = {n: torch.full((L, T, H, 128), 9.0, device="cuda") for n in ("q", "k", "v", "g")}
    out["beta"] = torch.full((L, T, H), 9.0, device="cuda")
    ring_out = torch.full_like(ring, 9.0)
    kda.kda_row_ops(dev["x"], dev["a"], dev["b"], w, ring, out["q"], out["k"], out["v"],
                    out["g"], out["beta"], ring_out=ring_out)
    torch.cuda.synchronize()
    res = {n: t.cpu().numpy() for n, t in out.items()}
    res["ring"] = ring_out.cpu().numpy()
    return res, dev


def _ref(inp, H, bf16=False):
    if bf16:
        xs = [synth.to_bf16_bits(inp[n]) for n in ("x", "a", "b")]
    else:
        xs = [inp[n] for n in ("x", "a", "b")]
    return oracle.row_ops(*xs, inp["w"], inp["ring"], H)


def _close(got, ref):
    for n in ("q", "k", "v", "g", "beta"):
        err = float(np.abs(got[n] - ref[n]).max())
        assert err <= TOL, f"{n}: max abs err {err}"
    np.testing.assert_array_equal(got["ring"], ref["ring"])


@pytest.mark.parametrize("L,T,H", [(1, 8, 1), (1, 1, 1), (1, 8, 64), (2, 5, 3), (34, 15, 64)])
def test_row_ops_match_oracle_f32(L, T, H):
    inp = synth.row_op_inputs(5, L * 100 + T, L, T, H)
    got, _ = _run(inp, L, T, H)
    _close(got, _ref(inp, H))


@pytest.mark.parametrize("L,T,H", [(1, 8, 64), (34, 15, 64)])
def test_row_ops_match_oracle_bf16(L, T, H):
    inp = synth.row_op_inputs(6, L * 100 + T, L, T, H)
    got, _ = _run(inp, L, T, H, bf16=True)
    _close(got, _ref(inp, H, bf16=True))


@pytest.mark.parametrize("L,T,H", [(1, 8, 64), (34, 15, 64)])
def test_row_ops_small_rows_where_the_norm_epsilon_dominates(L, T, H):
    # raw projections and ring scaled by 1e-4: the conv outputs are ~3e-5, so
    # sum y^2 over a head (~1e-7) sits well below the norm's 1e-6 and q, k are
    # y / sqrt(sum y^2 + 1e-6), far from unit rows.  A kernel whose epsilon
    # differed from the oracle's (1e-7, 1e-8, 0) would miss the 1e-5 gate by
    # orders of magnitude.
    inp = synth.row_op_inputs(8, L * 100 + T, L, T, H)
    inp["x"] *= np.float32(1e-4)
    inp["ring"] *= np.float32(1e-4)
    ref = _ref(inp, H)
    for n in ("q", "k"):
        sq = (ref[n].astype(np.float64) ** 2).sum(-1)   # = sum y^2 / (sum y^2 + eps)
        assert sq.max() < 0.5, f"{n}: epsilon does not dominate this input"
    got, _ = _run(inp, L, T, H)
    _close(got, ref)


@pytest.mark.parametrize("T", [1, 2, 3, 7])
def test_row_ops_ring_is_the_full_accept_reroll(T):
    # the ring after all T rows (written by the last row's workgroup, from ring
    # rows when T < 3) is the re-roll of the snapshot at keep = T
    L, H = 2, 4
    inp = synth.row_op_inputs(7, T, L, T, H)
    got, dev = _run(inp, L, T, H)
    _close(got, _ref(inp, H))
    snap = torch.from_numpy(inp["ring"]).cuda()
    out = torch.empty_like(snap)
    kda.kda_conv_reroll(snap, dev["x"], T, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), got["ring"])
    # rows run in parallel, so an in-place ring is refused
    q = torch.empty(L, T, H, 128, device="cuda")
    beta = torch.empty(L, T, H, device="cuda")
    with pytest.raises(kda.KdaError, match="ring_out overlaps ring_in"):
        kda.kda_row_ops(dev["x"], dev["a"], dev["b"], torch.from_numpy(inp["w"]).cuda(), snap,
                        q, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), beta,
                        ring_out=snap)


def test_row_ops_feed_the_scan_end_to_end():
    # projections -> row ops -> scan, against the oracle's row ops -> oracle scan
    L, T, H = 2, 15, 8
    inp = synth.row_op_inputs(8, 0, L, T, H)
    got, _ = _run(inp, L, T, H)
    ref = _ref(inp, H)
    s0 = synth.warmup_rows(8, 1, L, H)   # any state: warm it with one oracle row
    S0, _ = oracle.scan_rows(np.zeros((L, H, 128, 128), np.float32),
                             *[s0[n] for n in ("q", "k", "v", "g", "beta")])
    s_in = torch.from_numpy(S0).cuda()
    s_out = torch.empty_like(s_in)
    o = torch.empty(L, T, H, 128, device="cuda")
    rows = [torch.from_numpy(got[n]).cuda() for n in ("q", "k", "v", "g", "beta")]
    kda.kda_scan_rows(s_in, s_out, *rows, o=o)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.scan_rows(S0, *[ref[n] for n in ("q", "k", "v", "g", "beta")])
    assert float(np.abs(o.cpu().numpy() - o_ref).max()) <= 1e-4
    assert float(np.abs(s_out.cpu().numpy() - S_ref).max()) <= 1e-4
