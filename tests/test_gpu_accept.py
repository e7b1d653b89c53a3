"""Greedy accept on the GPU: kda_accept_greedy against the oracle, bit for bit.

Every case compares the per-row argmaxes, j and the bonus token with the
CPU oracle (the argmax is an integer decided by f32 comparisons on both
sides, so the match must be exact), and where the inputs plant a unique
maximum per row also with the planted tokens.  Sizes run from one logit to
the pages' 150,000-entry vocabulary at t = 15 (K = 14) and past the point
where a workgroup loops over several chunks of a row.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def work():
    return kda.accept_workspace()


def _drafts_dev(drafts):
    if drafts.size == 0:
        return None
    return torch.from_numpy(np.ascontiguousarray(drafts, np.uint32).view(np.int32)).cuda()


def _gpu(logits_dev, drafts, work):
    t = logits_dev.shape[0]
    vam = torch.full((t,), 7, dtype=torch.int32, device="cuda")
    out2 = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    kda.kda_accept_greedy(logits_dev, _drafts_dev(drafts), vam, out2, work)
    torch.cuda.synchronize()
    o2 = out2.cpu().numpy().view(np.uint32)
    return vam.cpu().numpy().view(np.uint32), int(o2[0]), int(o2[1])


def _f32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _same(gpu, ref):
    vam, j, bonus = gpu
    rvam, rj, rbonus = ref
    np.testing.assert_array_equal(vam, rvam)
    assert (j, bonus) == (rj, rbonus)


CASES = [(1, 1, 0), (2, 1, 1), (4, 3, 2), (4, 32, 0), (8, 1000, 5), (15, 4095, 14),
         (15, 4096, 3), (15, 4097, 9), (4, 150_000, 3), (15, 150_000, 7), (15, 150_000, 14),
         (2, 300_001, 0)]


@pytest.mark.parametrize("t,V,j", CASES)
def test_accept_planted_f32(t, V, j, work):
    logits, drafts, planted = synth.accept_round(10, t * 1000 + j, t, V, j)
    got = _gpu(_f32_dev(logits), drafts, work)
    np.testing.assert_array_equal(got[0], planted)
    assert got[1:] == (j, int(planted[j]))
    _same(got, oracle.accept_greedy(logits, drafts))


@pytest.mark.parametrize("t,V,j", [(1, 5, 0), (4, 150_000, 1), (15, 150_000, 11), (7, 4099, 6)])
def test_accept_planted_bf16(t, V, j, work):
    logits, drafts, planted = synth.accept_round(11, t * 1000 + j, t, V, j)
    bits = synth.to_bf16_bits(logits)
    got = _gpu(_bf16_dev(bits), drafts, work)
    np.testing.assert_array_equal(got[0], planted)
    _same(got, oracle.accept_greedy(bits, drafts))


@pytest.mark.parametrize("V", [1000, 4097, 150_000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accept_ties_take_the_lowest_index(V, dtype, work):
    # small integer logits: every row's maximum occurs many times
    rng = np.random.default_rng(V)
    t = 15
    logits = np.round(rng.standard_normal((t, V)) * 1.5).astype(np.float32)
    first = np.argmax(logits, axis=1).astype(np.uint32)   # numpy: first occurrence
    drafts = first[: t - 1].copy()
    drafts[9] ^= 1
    if dtype == "f32":
        got = _gpu(_f32_dev(logits), drafts, work)
        ref = oracle.accept_greedy(logits, drafts)
    else:
        bits = synth.to_bf16_bits(logits)    # small integers are exact in bf16
        got = _gpu(_bf16_dev(bits), drafts, work)
        ref = oracle.accept_greedy(bits, drafts)
    np.testing.assert_array_equal(got[0], first)
    assert got[1:] == (9, int(first[9]))
    _same(got, ref)


def test_accept_special_values(work):
    V = 9000
    t = 10
    rng = np.random.default_rng(5)
    x = rng.standard_normal((t, V)).astype(np.float32)
    x[0, :] = -np.inf                          # all -inf: index 0
    x[1, :] = 0.0
    x[1, ::2] = -0.0                           # -0 == +0: index 0
    x[2, 4096] = np.inf                        # +inf on a chunk boundary
    x[3, [17, 8999]] = np.inf                  # two +inf: the first
    x[4, 0] = np.nan                           # NaN first
    x[5, V - 1] = np.nan                       # NaN last
    x[6, 4095] = np.nan                        # NaN at a chunk's end
    x[6, 10] = np.inf
    x[7, :] = np.nan                           # all NaN
    x[8, V - 1] = 50.0                         # maximum at the last index
    x[9, :] = -np.inf
    x[9, V - 1] = -1e38                        # the only finite value, last
    drafts = np.zeros(t - 1, np.uint32)
    got = _gpu(_f32_dev(x), drafts, work)
    ref = oracle.accept_greedy(x, drafts)
    _same(got, ref)
    nt = kda.NO_TOKEN
    np.testing.assert_array_equal(
        got[0], np.array([0, 0, 4096, 17, nt, nt, nt, nt, V - 1, V - 1], np.uint32))


def test_accept_walk_stops_at_a_nan_row(work):
    t, V = 6, 2000
    logits, drafts, planted = synth.accept_round(12, 0, t, V, t - 1)
    logits[3, 77] = np.nan
    got = _gpu(_f32_dev(logits), drafts, work)
    assert got[0][3] == kda.NO_TOKEN
    assert got[1:] == (3, kda.NO_TOKEN)
    _same(got, oracle.accept_greedy(logits, drafts))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ld_extra,off", [(0, 1), (3, 0), (5, 3), (4, 2), (1, 0)])
def test_accept_row_stride_and_offset(dtype, ld_extra, off, work):
    # rows inside a wider buffer: odd strides and offsets take the scalar-load
    # kernel, a padded stride of a multiple of 4 from an aligned base the vector one
    t, V = 15, 10_007
    logits, drafts, planted = synth.accept_round(13, ld_extra * 10 + off, t, V, 4)
    ld = V + ld_extra
    if dtype == "f32":
        big = np.full((t, ld + off), -7.0, np.float32)
        big[:, off:off + V] = logits
        dev = _f32_dev(big.reshape(-1))
        ref = oracle.accept_greedy(logits, drafts)
        esz = 4
    else:
        bits = synth.to_bf16_bits(logits)
        big = np.full((t, ld + off), synth.to_bf16_bits(np.float32([-7.0]))[0], np.uint16)
        big[:, off:off + V] = bits
        dev = _bf16_dev(big.reshape(-1))
        ref = oracle.accept_greedy(bits, drafts)
        esz = 2
    view = torch.as_strided(dev, (t, V), (ld + off, 1), off)
    assert view.data_ptr() % 16 == (off * esz) % 16
    got = _gpu(view, drafts, work)
    np.testing.assert_array_equal(got[0], planted)
    _same(got, ref)


def test_accept_workspace_contents_do_not_matter(work):
    # V sets the workgroups per row (1, 37, 64 and a looping 64); the
    # workspace is refilled with arbitrary bytes before every call
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    for i, (t, V) in enumerate([(3, 10), (15, 150_000), (15, 262_144), (5, 600_000), (1, 1),
                                (15, 150_000), (2, 4097)]):
        work.copy_(torch.randint(0, 256, work.shape, dtype=torch.uint8, device="cuda",
                                 generator=g))
        j = i % t
        logits, drafts, planted = synth.accept_round(14, i, t, V, j)
        got = _gpu(_f32_dev(logits), drafts, work)
        np.testing.assert_array_equal(got[0], planted)
        assert got[1:] == (j, int(planted[j]))


def test_accept_streams_and_binding_checks(work):
    t, V = 4, 5000
    logits, drafts, planted = synth.accept_round(15, 0, t, V, 2)
    s = torch.cuda.Stream()
    dev = _f32_dev(logits)
    vam = torch.empty(t, dtype=torch.int32, device="cuda")
    out2 = torch.empty(2, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        kda.kda_accept_greedy(dev, _drafts_dev(drafts), vam, out2, work)
    s.synchronize()
    np.testing.assert_array_equal(vam.cpu().numpy().view(np.uint32), planted)
    assert out2.cpu().tolist() == [2, int(planted[2])]
    with pytest.raises(TypeError):
        kda.kda_accept_greedy(dev.double(), _drafts_dev(drafts), vam, out2, work)
    with pytest.raises(ValueError):
        kda.kda_accept_greedy(dev, _drafts_dev(drafts), vam[:3], out2, work)
    with pytest.raises(ValueError):
        kda.kda_accept_greedy(dev.t(), None, vam, out2, work)
