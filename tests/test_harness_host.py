"""The parity tests' own comparison helpers, checked on the CPU: the fp4
indexer-record comparison accepts the oracle's encoding, accepts a neighbouring
code only where the value sits on a rounding boundary, and rejects a flipped
code anywhere else; the query-fragility test flags values on a boundary."""
import numpy as np

import oracle as O
from harness import FP4_T_MARGIN, compare_fp4_rows, fp4_fragile


def _rows(seed=0, n=40):
    return np.random.default_rng(seed).standard_normal((n, 128))


def test_fp4_compare_accepts_the_oracle_encoding():
    x = _rows()
    compare_fp4_rows(O.fp4_encode_rows(x), x, "self")


def test_fp4_compare_rejects_a_flipped_code():
    x = _rows(1)
    rec = O.fp4_encode_rows(x)
    for byte, bit in ((0, 0), (17, 4), (63, 5)):
        bad = rec.copy()
        bad[7, byte] ^= 1 << bit
        try:
            compare_fp4_rows(bad, x, "planted")
        except AssertionError:
            continue
        raise AssertionError(f"flip of byte {byte} bit {bit} not caught")


def test_fp4_compare_rejects_a_wrong_scale():
    x = _rows(2)
    rec = O.fp4_encode_rows(x)
    bad = rec.copy()
    bad[3, 65] += 1
    try:
        compare_fp4_rows(bad, x, "planted scale")
    except AssertionError:
        return
    raise AssertionError("scale byte change not caught")


def test_fp4_compare_allows_a_flip_on_a_boundary():
    x = _rows(3, 1)
    # put channel 5 of block 0 exactly between grid points 1.0 and 1.5 of its
    # block scale (the block max stays where it is)
    blk = np.abs(x[0, :32])
    e = int(np.floor(np.log2(blk.max()))) - 2
    if blk[5] == blk.max():
        x[0, 5] = -x[0, 5]
        x[0, 6] = blk.max()
    x[0, 5] = 1.25 * 2.0 ** e
    assert fp4_fragile(x)[0, 5]
    rec = O.fp4_encode_rows(x)
    code = (rec[0, 2] >> 4) & 15            # channel 5: high nibble of byte 2
    assert code in (2, 3)
    other = rec.copy()
    other[0, 2] = (other[0, 2] & 0x0F) | ((5 - code) << 4)   # the other neighbour (2 <-> 3)
    compare_fp4_rows(other, x, "boundary")


def test_fp4_fragile_margin():
    x = np.zeros((1, 128))
    x[0, 0] = 5.9            # block max 5.9: scale 2^0
    x[0, 1] = 0.75 + FP4_T_MARGIN / 2
    x[0, 2] = 0.75 + 4 * FP4_T_MARGIN
    f = fp4_fragile(x)
    assert f[0, 1] and not f[0, 2]
