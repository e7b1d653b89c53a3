"""The verify loop end to end: projections -> row ops -> fused verify round ->
greedy accept on the device -> conv-ring rollback -> next round.

Each GPU round feeds the next through the library only: the accepted-draft
count that sets `keep` comes from kda_accept_greedy, and the committed conv
ring from kda_conv_reroll.  The same chain is composed from the oracle's
functions (row ops, scan, accept, replay, ring roll).  Outputs and states must
agree within 1e-4, the accept decisions and the rings exactly.
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


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_verify_loop_rounds_match_the_oracle_chain():
    L, H, T, V, rounds = 2, 4, 8, 1000, 4
    C = 3 * H * D
    js_planted = [3, 7, 0, 5]          # j per round: partial, full, none, partial
    w = synth.row_op_inputs(40, 0, L, T, H)["w"]
    ring_ref = synth.row_op_inputs(40, 0, L, T, H)["ring"]
    S_ref = np.zeros((L, H, D, D), np.float32)

    ring = _dev(ring_ref)
    w_d = _dev(w)
    snap = torch.zeros(L, H, D, D, device="cuda")
    work = kda.accept_workspace()
    prev = None                         # (k, g, e, keep) of the previous round on the GPU
    prev_ref = None                     # (rows, keep) of the previous round, oracle side

    for r in range(rounds):
        p = synth.row_op_inputs(41, r, L, T, H)
        # ---- GPU: projections -> scan inputs
        q, k, v, g = (torch.empty(L, T, H, D, device="cuda") for _ in range(4))
        beta = torch.empty(L, T, H, device="cuda")
        x_d = _dev(p["x"])
        kda.kda_row_ops(x_d, _dev(p["a"]), _dev(p["b"]), w_d, ring, q, k, v, g, beta)
        # ---- GPU: fused round (replay of the previous round's kept rows, then scan)
        nxt = torch.empty_like(snap)
        o = torch.empty(L, T, H, D, device="cuda")
        e = torch.empty(L, T, H, D, device="cuda")
        if prev is None:
            kda.kda_verify_round(snap, nxt, None, 0, q, k, v, g, beta, o, e=e)
        else:
            pk, pg, pe, keep_prev = prev
            kda.kda_verify_round(snap, nxt, (pk, None, pg, None, pe), keep_prev,
                                 q, k, v, g, beta, o, e=e)
        snap = nxt
        # ---- GPU: greedy accept decides keep
        logits, drafts, planted = synth.accept_round(42, r, T, V, js_planted[r])
        vam = torch.empty(T, dtype=torch.int32, device="cuda")
        out2 = torch.empty(2, dtype=torch.int32, device="cuda")
        kda.kda_accept_greedy(_dev(logits), _dev(drafts.view(np.int32)), vam, out2, work)
        j = int(out2[0].item())
        keep = j + 1
        # ---- GPU: committed conv ring for the next round
        ring_next = torch.empty_like(ring)
        kda.kda_conv_reroll(ring, x_d, keep, ring_next)
        ring = ring_next
        prev = (k, g, e, keep)

        # ---- oracle chain
        ops = oracle.row_ops(p["x"], p["a"], p["b"], w, ring_ref, H)
        rows_ref = [ops[n] for n in ("q", "k", "v", "g", "beta")]
        if prev_ref is not None:
            S_ref = oracle.replay(S_ref, *prev_ref[0], keep=prev_ref[1])
        _, o_ref = oracle.scan_rows(S_ref, *rows_ref)
        vam_ref, j_ref, bonus_ref = oracle.accept_greedy(logits, drafts)
        ring_ref = oracle.conv_reroll(ring_ref, p["x"], j_ref + 1)
        prev_ref = (rows_ref, j_ref + 1)

        torch.cuda.synchronize()
        assert (j, int(out2[1].item())) == (j_ref, int(bonus_ref)) == (js_planted[r],
                                                                       int(planted[j_ref]))
        np.testing.assert_array_equal(vam.cpu().numpy().view(np.uint32), vam_ref)
        assert float(np.abs(snap.cpu().numpy() - S_ref).max()) <= TOL, f"round {r} snapshot"
        assert float(np.abs(o.cpu().numpy() - o_ref).max()) <= TOL, f"round {r} outputs"
        np.testing.assert_array_equal(ring.cpu().numpy(), ring_ref)
