"""Pins of the fragment-tiled MXFP4 storage order (oracle side).

The layout is a storage convention, not part of the method; what pins it is
its definition, checked here slot by slot with plain index arithmetic, and
the product the scaled 16 x 16 x 128 matrix-core instruction forms from two
records, emulated lane by lane from the instruction's operand description
(lane l: row l % 16 and the 32 positions of group l // 16; one scale byte
per lane), which must equal the fp64 product of the row-layout operands."""
import numpy as np
import pytest

import oracle as O

GROUP = 32


def _random_operand(rng, rows, K):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(118, 136, (rows, K // GROUP), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("rows,K", [(1, 128), (16, 128), (37, 384), (64, 256)])
def test_slots_by_definition(rows, K):
    rng = np.random.default_rng(rows * 1000 + K)
    codes, scales = _random_operand(rng, rows, K)
    tc, ts = O.tile_mxfp4(codes, scales)
    nk = K // 128
    rt = (rows + 15) // 16
    assert tc.shape == (rt * nk * 1024,) and ts.shape == (rt * nk * 64,)
    seen = np.zeros(rt * nk * 64, bool)
    for row in range(rt * 16):
        for g in range(K // GROUP):
            record = (row // 16) * nk + g // 4
            slot = (g % 4) * 16 + row % 16
            got_c = tc[record * 1024 + slot * 16: record * 1024 + slot * 16 + 16]
            got_s = ts[record * 64 + slot]
            if row < rows:
                assert np.array_equal(got_c, codes[row, 16 * g: 16 * g + 16]), (row, g)
                assert got_s == scales[row, g], (row, g)
            else:
                assert not got_c.any() and got_s == 0, (row, g)
            seen[record * 64 + slot] = True
    assert seen.all()


@pytest.mark.parametrize("rows,K", [(5, 128), (33, 512)])
def test_round_trip(rows, K):
    rng = np.random.default_rng(7 + rows)
    codes, scales = _random_operand(rng, rows, K)
    c2, s2 = O.untile_mxfp4(*O.tile_mxfp4(codes, scales), rows, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        O.tile_mxfp4(np.zeros((2, 32), np.uint8), np.zeros((2, 2), np.uint8))


def _lane_values(code_record, scale_record, lane):
    """The 32 values lane `lane` feeds the instruction: its 16 code bytes,
    low nibble first, times 2^(scale - 127)."""
    b = code_record[16 * lane: 16 * lane + 16]
    nib = np.stack([b & 15, b >> 4], axis=1).reshape(-1)
    return O.code_value(nib) * 2.0 ** (int(scale_record[lane]) - 127)


def test_instruction_emulation_gives_the_product():
    rng = np.random.default_rng(11)
    M, N, K = 20, 35, 256
    a = _random_operand(rng, M, K)
    b = _random_operand(rng, N, K)
    ta, tsa = O.tile_mxfp4(*a)
    tb, tsb = O.tile_mxfp4(*b)
    nk = K // 128
    y = np.zeros((16 * ((M + 15) // 16), 16 * ((N + 15) // 16)))
    for tm in range((M + 15) // 16):
        for tn in range((N + 15) // 16):
            for s in range(nk):
                ra, rb = tm * nk + s, tn * nk + s
                ca, sa = ta[ra * 1024:(ra + 1) * 1024], tsa[ra * 64:(ra + 1) * 64]
                cb, sb = tb[rb * 1024:(rb + 1) * 1024], tsb[rb * 64:(rb + 1) * 64]
                for i in range(16):
                    for j in range(16):
                        acc = 0.0
                        for q in range(4):  # the four groups of the 128 positions
                            acc += float(_lane_values(ca, sa, i + 16 * q) @ _lane_values(cb, sb, j + 16 * q))
                        y[16 * tm + i, 16 * tn + j] += acc
    ref, _ = O.gemm_mxfp4(*a, *b)
    assert np.allclose(y[:M, :N], ref, rtol=1e-12, atol=0.0)
