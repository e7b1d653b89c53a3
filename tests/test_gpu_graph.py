"""Per-layer launches captured in a HIP graph replay to the eager bits.

A model issues the scan one layer at a time; a serving loop captures those
launches once and replays them.  The library enqueues on the caller's stream
and never allocates or synchronizes, so its launches can be captured.  The
graph is replayed several times with eager work between the replays, and every
replay must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth

pytestmark = pytest.mark.gpu

D = 128


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def test_per_layer_round_graph_replays_match_eager():
    L, T, H, keep = 3, 15, 64, 6
    r = synth.rows(31, 0, L, T, H)
    rows = [torch.from_numpy(r[n]).cuda() for n in ("q", "k", "v", "g", "beta")]
    rng = np.random.default_rng(32)
    snap = torch.from_numpy((0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32)).cuda()
    e_prev = torch.from_numpy((0.1 * rng.standard_normal((L, T, H, D))).astype(np.float32)).cuda()
    nxt = torch.empty_like(snap)
    o = torch.empty(L, T, H, D, device="cuda")
    e = torch.empty_like(o)

    def layer_loop():
        for l in range(L):
            sl = slice(l, l + 1)
            rr = [x[sl] for x in rows]
            kda.kda_verify_round(snap[sl], nxt[sl], (rr[1], None, rr[3], None, e_prev[sl]), keep,
                                 *rr, o[sl], e=e[sl])

    layer_loop()
    torch.cuda.synchronize()
    want = [_bits(x) for x in (nxt, o, e)]

    s = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        layer_loop()
    s.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer_loop()
    for rep in range(4):
        for x in (nxt, o, e):
            x.fill_(float(rep + 1))       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, w in zip(("snap_out", "o", "e"), (nxt, o, e), want):
            assert np.array_equal(_bits(x), w), f"replay {rep}: {name} differs"
