"""Conv-ring rollback and the batched copy on the GPU, bit for bit.

kda_conv_reroll is compared element by element with the oracle's roll-per-row
definition at the pages' ring size (3 rows x 3 * 64 * 128 q/k/v channels per
layer, 34 layers, T = 15), for f32 and bf16 raw rows, on the vector kernel and
on the element-aligned kernel (odd channel counts, offset buffers).
kda_copy_batch must reproduce its sources exactly.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth
import oracle

pytestmark = pytest.mark.gpu

C_QKV = 3 * 64 * 128   # raw q/k/v channels of one layer


def _case(seed, L, T, C):
    rng = np.random.default_rng(seed)
    snap = rng.standard_normal((L, 3, C)).astype(np.float32)
    raw = rng.standard_normal((L, T, C)).astype(np.float32)
    return snap, raw


def _dev_at(x, offset_elems=0, dtype=torch.float32):
    """x on the device, starting offset_elems elements into a larger buffer."""
    x = np.ascontiguousarray(x)
    if dtype == torch.bfloat16:
        flat = torch.from_numpy(x.view(np.int16).reshape(-1))
        big = torch.zeros(flat.numel() + offset_elems, dtype=torch.int16, device="cuda")
    else:
        flat = torch.from_numpy(x.reshape(-1))
        big = torch.zeros(flat.numel() + offset_elems, dtype=torch.float32, device="cuda")
    big[offset_elems:] = flat.cuda()
    t = big[offset_elems:].view(x.shape)
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t


@pytest.mark.parametrize("keep", [1, 2, 3, 8, 15])
def test_reroll_full_size_f32(keep):
    L, T = 34, 15
    snap, raw = _case(keep, L, T, C_QKV)
    out = torch.full((L, 3, C_QKV), 7.0, device="cuda")
    kda.kda_conv_reroll(_dev_at(snap), _dev_at(raw), keep, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.conv_reroll(snap, raw, keep))


@pytest.mark.parametrize("keep", [1, 4, 15])
def test_reroll_bf16_rows(keep):
    L, T = 34, 15
    snap, raw = _case(20 + keep, L, T, C_QKV)
    bits = synth.to_bf16_bits(raw)
    out = torch.empty((L, 3, C_QKV), device="cuda")
    kda.kda_conv_reroll(_dev_at(snap), _dev_at(bits, 0, torch.bfloat16), keep, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.conv_reroll(snap, bits, keep))


@pytest.mark.parametrize("C,off,dtype", [(1001, 0, "f32"), (1001, 1, "bf16"), (4096, 1, "f32"),
                                         (4096, 3, "bf16"), (5, 0, "f32"), (1, 0, "f32")])
def test_reroll_unaligned_and_ragged(C, off, dtype):
    L, T, keep = 3, 6, 2
    snap, raw = _case(C + off, L, T, C)
    out = torch.zeros(L * 3 * C + off, device="cuda")[off:].view(L, 3, C)
    if dtype == "f32":
        raw_d = _dev_at(raw, off)
        ref = oracle.conv_reroll(snap, raw, keep)
    else:
        bits = synth.to_bf16_bits(raw)
        raw_d = _dev_at(bits, off, torch.bfloat16)
        ref = oracle.conv_reroll(snap, bits, keep)
    kda.kda_conv_reroll(_dev_at(snap, off), raw_d, keep, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_reroll_keeps_the_snapshot_and_rows_untouched():
    L, T = 2, 5
    snap, raw = _case(40, L, T, 256)
    s_d, r_d = _dev_at(snap), _dev_at(raw)
    out = torch.empty((L, 3, 256), device="cuda")
    for keep in range(1, T + 1):
        kda.kda_conv_reroll(s_d, r_d, keep, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.conv_reroll(snap, raw, keep))
    np.testing.assert_array_equal(s_d.cpu().numpy(), snap)
    np.testing.assert_array_equal(r_d.cpu().numpy(), raw)


def test_copy_batch_states_exact():
    # 34 per-layer 4 MiB states in separate allocations, one launch
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    srcs = [torch.randn(64, 128, 128, device="cuda", generator=g) for _ in range(34)]
    dsts = [torch.full_like(s, 3.0) for s in srcs]
    table = kda.copy_table(srcs, dsts)
    kda.kda_copy_batch(table, 34, 64 * 128 * 128)
    torch.cuda.synchronize()
    for s, d in zip(srcs, dsts):
        assert torch.equal(s, d)


@pytest.mark.parametrize("words,offs", [(1, (0, 0)), (7, (1, 2)), (4096, (1, 0)),
                                        (100_003, (0, 3)), (1 << 20, (0, 0))])
def test_copy_batch_alignments_and_sizes(words, offs):
    # pairs with and without 16-byte alignment in one table
    n = 3
    base_s = [torch.randn(words + 4, device="cuda") for _ in range(n)]
    base_d = [torch.zeros(words + 4, device="cuda") for _ in range(n)]
    srcs = [b[offs[0] if i % 2 else 0:][:words] for i, b in enumerate(base_s)]
    dsts = [b[offs[1] if i % 2 else 0:][:words] for i, b in enumerate(base_d)]
    table = kda.copy_table(srcs, dsts)
    kda.kda_copy_batch(table, n, words)
    torch.cuda.synchronize()
    for i, (s, d, bd) in enumerate(zip(srcs, dsts, base_d)):
        assert torch.equal(s, d)
        o = offs[1] if i % 2 else 0
        # nothing outside the destination window was written
        assert torch.count_nonzero(bd[:o]) == 0
        assert torch.count_nonzero(bd[o + words:]) == 0
