"""Rollback with the accepted-draft count left on the device.

kda_verify_round_dev and kda_conv_reroll_dev read j (kda_accept_greedy's
out2[0]) in the kernels and commit keep = min(j, T - 1) + 1 rows.  For every j
they must give the bits of the host-keep calls with that keep, on every tiling;
and a verify loop that never reads j back between the accept and the rollback
must reproduce the loop that does.
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
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rows(seed, index, L, T, H):
    r = synth.rows(seed, index, L, T, H)
    return [dev(r[n]) for n in NAMES]


def same(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("L,H,stash", [(1, 64, True), (4, 64, False), (34, 64, True),
                                       (2, 3, False), (34, 8, True)])
def test_verify_round_dev_equals_host_keep(L, H, stash):
    print(f"devkeep round L={L} H={H} stash={stash}", flush=True)
    T_prev, T = 12, 15
    prev = rows(90, 0, L, T_prev, H)
    cur = rows(90, 1, L, T, H)
    rng = np.random.default_rng(91)
    s0 = dev((0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32))
    e_prev = torch.empty(L, T_prev, H, D, device="cuda")
    kda.kda_scan_rows_stash(s0, torch.empty_like(s0), *prev, None, e_prev)
    p = (prev[1], None, prev[3], None, e_prev) if stash else \
        (prev[1], prev[2], prev[3], prev[4], None)
    js = [0, 1, 5, T_prev - 1, T_prev, 1000, 0xFFFFFFFF] if L * H <= 256 else [0, 7, T_prev - 1,
                                                                                 50]
    for j in js:
        keep = min(j, T_prev - 1) + 1
        # element 0 carries j's 32 bits (0xFFFFFFFF as int32 -1); element 1 is noise
        jd = torch.tensor([j if j <= 0x7FFFFFFF else j - (1 << 32), 123], dtype=torch.int32,
                          device="cuda")
        outs = []
        for k_arg in (keep, jd):
            snap = torch.empty_like(s0)
            o = torch.empty(L, T, H, D, device="cuda")
            e = torch.empty(L, T, H, D, device="cuda")
            kda.kda_verify_round(s0, snap, p, k_arg, *cur, o, e=e)
            outs.append((snap, o, e))
        torch.cuda.synchronize()
        for name, a, b in zip(("snapshot", "o", "e"), *outs):
            assert same(a, b), f"j={j}: {name}"


@pytest.mark.parametrize("bf16", [False, True])
def test_conv_reroll_dev_equals_host_keep(bf16):
    L, T, C = 3, 9, 3 * 5 * D
    rng = np.random.default_rng(92)
    ring = dev(rng.standard_normal((L, 3, C)).astype(np.float32))
    raw = dev(rng.standard_normal((L, T, C)).astype(np.float32))
    if bf16:
        raw = raw.to(torch.bfloat16)
    for j in (0, 1, 2, 3, T - 1, T, 77):
        keep = min(j, T - 1) + 1
        a = torch.empty_like(ring)
        b = torch.empty_like(ring)
        kda.kda_conv_reroll(ring, raw, keep, a)
        kda.kda_conv_reroll(ring, raw, torch.tensor([j], dtype=torch.int32, device="cuda"), b)
        torch.cuda.synchronize()
        assert same(a, b), f"j={j}"


def test_loop_without_readback_equals_loop_with_it():
    """Row ops -> round -> accept -> re-roll for 5 rounds, once reading j back
    to the host each round and once leaving it on the device."""
    L, H, T, V, rounds = 2, 4, 8, 1000, 5
    js_planted = [3, 7, 0, 5, 2]
    base = synth.row_op_inputs(93, 0, L, T, H)
    w = dev(base["w"])

    def run(device_keep):
        ring = dev(base["ring"])
        snap = torch.zeros(L, H, D, D, device="cuda")
        work = kda.accept_workspace()
        prev = None
        outs = []
        for r in range(rounds):
            p_ = synth.row_op_inputs(94, r, L, T, H)
            x = dev(p_["x"])
            q, k, v, g = (torch.empty(L, T, H, D, device="cuda") for _ in range(4))
            beta = torch.empty(L, T, H, device="cuda")
            kda.kda_row_ops(x, dev(p_["a"]), dev(p_["b"]), w, ring, q, k, v, g, beta)
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
            logits, drafts, _ = synth.accept_round(95, r, T, V, js_planted[r])
            vam = torch.empty(T, dtype=torch.int32, device="cuda")
            out2 = torch.empty(2, dtype=torch.int32, device="cuda")
            kda.kda_accept_greedy(dev(logits), dev(drafts.view(np.int32)), vam, out2, work)
            keep = out2 if device_keep else int(out2[0].item()) + 1
            ring_next = torch.empty_like(ring)
            kda.kda_conv_reroll(ring, x, keep, ring_next)
            ring = ring_next
            prev = (k, g, e, keep)
            outs.append((o, snap, ring, out2))
        torch.cuda.synchronize()
        return outs

    host, devk = run(False), run(True)
    for r, (a, b) in enumerate(zip(host, devk)):
        for name, x, y in zip(("o", "snapshot", "ring", "accept"), a, b):
            assert same(x, y), f"round {r}: {name}"
    assert [int(h[3][0]) for h in host] == js_planted


def test_captured_loop_replays_equal_the_eager_loop():
    """The device-keep loop, captured as HIP graphs (one per buffer parity), replayed
    round after round with eager work and synchronizations between the replays:
    every replay's outputs equal the eager loop's round for round."""
    L, H, T, V, rounds = 2, 4, 8, 1000, 6
    js_planted = [3, 7, 0, 5, 2, 6]
    base = synth.row_op_inputs(96, 0, L, T, H)
    w = dev(base["w"])
    proj = [synth.row_op_inputs(97, r, L, T, H) for r in range(2)]
    xs = [dev(p_["x"]) for p_ in proj]
    as_ = [dev(p_["a"]) for p_ in proj]
    bs = [dev(p_["b"]) for p_ in proj]
    acc = [synth.accept_round(98, r, T, V, js_planted[r]) for r in range(rounds)]
    logits = [dev(a[0]) for a in acc]
    drafts = [dev(a[1].view(np.int32)) for a in acc]
    lg_buf = torch.empty_like(logits[0])
    dr_buf = torch.empty_like(drafts[0])
    work = kda.accept_workspace()
    sets = [[torch.empty(L, T, H, D, device="cuda") for _ in range(4)]
            + [torch.empty(L, T, H, device="cuda"), torch.empty(L, T, H, D, device="cuda")]
            for _ in range(2)]
    st = [torch.zeros(L, H, D, D, device="cuda") for _ in range(2)]
    rings = [dev(base["ring"]), torch.empty(L, 3, 3 * H * D, device="cuda")]
    o = torch.empty(L, T, H, D, device="cuda")
    vam = torch.empty(T, dtype=torch.int32, device="cuda")
    out2 = [torch.zeros(2, dtype=torch.int32, device="cuda") for _ in range(2)]

    def round_(i, first=False):
        cur, prv = sets[i % 2], sets[(i + 1) % 2]
        x = xs[i % 2]
        kda.kda_row_ops(x, as_[i % 2], bs[i % 2], w, rings[i % 2], *cur[:5])
        if first:
            kda.kda_verify_round(st[i % 2], st[(i + 1) % 2], None, 0, *cur[:5], o, e=cur[5])
        else:
            kda.kda_verify_round(st[i % 2], st[(i + 1) % 2], (prv[1], None, prv[3], None, prv[5]),
                                 out2[(i + 1) % 2], *cur[:5], o, e=cur[5])
        kda.kda_accept_greedy(lg_buf, dr_buf, vam, out2[i % 2], work)
        kda.kda_conv_reroll(rings[i % 2], x, out2[i % 2], rings[(i + 1) % 2])

    def snap_out(i):
        return [t.clone() for t in (o, st[(i + 1) % 2], rings[(i + 1) % 2], out2[i % 2])]

    def reset():
        st[0].zero_()
        rings[0].copy_(dev(base["ring"]))
        torch.cuda.synchronize()

    # eager reference
    reset()
    ref = []
    for i in range(rounds):
        lg_buf.copy_(logits[i]); dr_buf.copy_(drafts[i])
        round_(i, first=(i == 0))
        ref.append(snap_out(i))
    torch.cuda.synchronize()

    # round 0 eagerly, then capture one graph per parity
    reset()
    lg_buf.copy_(logits[0]); dr_buf.copy_(drafts[0])
    round_(0, first=True)
    torch.cuda.synchronize()
    got = [snap_out(0)]
    saved = [t.clone() for t in (st[1], rings[1], out2[0])]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the capture path
        round_(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for par in (1, 0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            round_(par)
        graphs.append(g)
    # undo what the warm-up and the captures touched: restore the state after round 0
    st[1].copy_(saved[0]); rings[1].copy_(saved[1]); out2[0].copy_(saved[2])
    torch.cuda.synchronize()
    for i in range(1, rounds):
        lg_buf.copy_(logits[i]); dr_buf.copy_(drafts[i])   # eager work between replays
        graphs[0 if i % 2 == 1 else 1].replay()
        torch.cuda.synchronize()
        got.append(snap_out(i))
    for i, (a, b) in enumerate(zip(ref, got)):
        for name, x, y in zip(("o", "snapshot", "ring", "accept"), a, b):
            assert same(x, y), f"round {i}: {name}"
    assert [int(r[3][0]) for r in ref] == js_planted
