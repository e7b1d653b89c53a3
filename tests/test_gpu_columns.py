"""The per-row state-column variant (kda_scan_rows_columns) against the replay arm.

Column t must carry the bits of kda_replay(keep = t + 1) and of a scan over
rows 0..t; its outputs and stash plane must equal kda_scan_rows'; a round that
continues from column keep - 1 must give the bits of the fused round that
replays keep rows instead.  The oracle checks the columns within 1e-4.  The
shapes cover every tiling: 4, 2 and 1 workgroups per head, and whole-head
launches that end in a split tail of 2 and 4 workgroups per head.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import gated_delta_rule_rows_amd as kda  # noqa: E402
from gated_delta_rule_rows_amd import synth  # noqa: E402
import oracle  # noqa: E402

TOL = 1e-4
D = 128
NAMES = ("q", "k", "v", "g", "beta")


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def rows(seed, index, L, T, H, bf16):
    r = (synth.rows_bf16 if bf16 else synth.rows)(seed, index, L, T, H)
    return r, [dev(r[n]) for n in NAMES]


def state(seed, L, H):
    rng = np.random.default_rng(seed)
    return (0.5 * rng.standard_normal((L, H, D, D))).astype(np.float32)


@pytest.mark.parametrize("L,H,T,bf16", [
    (1, 1, 8, False),      # 1 chain: 4 workgroups per head
    (3, 5, 15, True),
    (4, 64, 15, False),    # 256 chains: 2 per head
    (34, 8, 15, False),    # 272 chains: 256 whole heads, the last 16 at 4 per head
    (8, 64, 12, False),    # 512 chains: whole heads, one fill
    (17, 64, 15, True),    # 1,088 chains: whole heads, tail split 4 ways
    (34, 64, 15, False),   # 2,176 chains: whole heads, tail split 2 ways
])
def test_columns_equal_replays_and_the_scan(L, H, T, bf16):
    print(f"columns L={L} H={H} T={T} bf16={bf16}", flush=True)
    r_np, rd = rows(70, 0, L, T, H, bf16)
    S0 = state(71, L, H)
    s0 = dev(S0)
    s0_copy = s0.clone()
    cols = torch.empty(T, L, H, D, D, device="cuda")
    o = torch.empty(L, T, H, D, device="cuda")
    e = torch.empty(L, T, H, D, device="cuda")
    kda.kda_scan_rows_columns(s0, cols, *rd, o, e=e)

    s_out = torch.empty_like(s0)
    o_ref = torch.empty_like(o)
    e_ref = torch.empty_like(e)
    kda.kda_scan_rows_stash(s0, s_out, *rd, o_ref, e_ref)
    torch.cuda.synchronize()
    assert same_bits(s0, s0_copy), "s_in changed"
    assert same_bits(o, o_ref), "o differs from kda_scan_rows"
    assert same_bits(e, e_ref), "e differs from kda_scan_rows"
    assert same_bits(cols[T - 1], s_out), "last column != scan state"
    rep = torch.empty_like(s0)
    for t in range(T):
        kda.kda_replay(s0, rep, *rd, keep=t + 1)
        torch.cuda.synchronize()
        assert same_bits(cols[t], rep), f"column {t} != replay(keep={t + 1})"

    # the oracle, on a sample of chains, one row at a time
    heads = sorted({0, H // 3, H - 1})
    layers = sorted({0, L // 2, L - 1})
    sub = lambda t: [r_np[n][layers][:, t:t + 1][:, :, heads] for n in NAMES]
    S_ref = S0[layers][:, heads]
    cols_h = cols.cpu().numpy()[:, layers][:, :, heads]
    o_h = o.cpu().numpy()[layers][:, :, heads]
    for t in range(T):
        S_ref, o_t = oracle.scan_rows(S_ref, *sub(t), threads=oracle.max_threads())
        assert float(np.abs(cols_h[t] - S_ref).max()) <= TOL, f"column {t} vs oracle"
        assert float(np.abs(o_h[:, t:t + 1] - o_t).max()) <= TOL, f"o row {t} vs oracle"


@pytest.mark.parametrize("stash", [False, True])
def test_next_round_from_a_column_equals_the_fused_round(stash):
    """A round continued from column keep-1 by pointer gives the fused round's bits."""
    L, H, T = 2, 8, 15
    _, prev = rows(72, 0, L, T, H, False)
    _, cur = rows(72, 1, L, T, H, False)
    s0 = dev(state(73, L, H))
    cols = torch.empty(T, L, H, D, D, device="cuda")
    o_prev = torch.empty(L, T, H, D, device="cuda")
    e_prev = torch.empty(L, T, H, D, device="cuda")
    kda.kda_scan_rows_columns(s0, cols, *prev, o_prev, e=e_prev)
    for keep in (1, 6, T):
        # columns arm: the committed state is a view, the next round scans from it
        s_next = torch.empty_like(s0)
        o_cols = torch.empty(L, T, H, D, device="cuda")
        kda.kda_scan_rows(cols[keep - 1], s_next, *cur, o=o_cols)
        # replay arm: the fused round rebuilds it from the snapshot
        snap = torch.empty_like(s0)
        o_fused = torch.empty_like(o_cols)
        p = (prev[1], None, prev[3], None, e_prev) if stash else \
            (prev[1], prev[2], prev[3], prev[4], None)
        kda.kda_verify_round(s0, snap, p, keep, *cur, o_fused)
        torch.cuda.synchronize()
        assert same_bits(snap, cols[keep - 1]), f"keep={keep}: committed state"
        assert same_bits(o_cols, o_fused), f"keep={keep}: next round's outputs"


def test_columns_binding_refusals():
    L, H, T = 1, 2, 4
    _, rd = rows(74, 0, L, T, H, False)
    s0 = torch.zeros(L, H, D, D, device="cuda")
    o = torch.empty(L, T, H, D, device="cuda")
    with pytest.raises(ValueError, match="s_cols"):
        kda.kda_scan_rows_columns(s0, torch.empty(T - 1, L, H, D, D, device="cuda"), *rd, o)
    with pytest.raises(ValueError, match="o is required"):
        kda.kda_scan_rows_columns(s0, torch.empty(T, L, H, D, D, device="cuda"), *rd, None)
    # a column buffer that holds the input state is refused by the library;
    # the columns right after it are not an overlap
    big = torch.zeros(T + 1, L, H, D, D, device="cuda")
    with pytest.raises(kda.KdaError, match="s_cols overlaps s_in"):
        kda.kda_scan_rows_columns(big[0], big[:T], *rd, o)
    with pytest.raises(kda.KdaError, match="s_cols overlaps s_in"):
        kda.kda_scan_rows_columns(big[T - 1], big[:T], *rd, o)
    kda.kda_scan_rows_columns(big[0], big[1:], *rd, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(big[0]) == 0
