"""Test-side encoder of canonical expert blocks from known integer codes.

Canonical block (the format the synthetic generator writes and both the oracle
and the GPU packer read): gate_q [f][d], up_q [f][d], down_q [d][f] packed
codes (int4: two's-complement nibbles, element 2i in the low nibble of byte i;
int8: one two's-complement byte per element), then float32 scales gate_s
[f][d/G], up_s [f][d/G], down_s [d][f/G] (G == 0: one scale per row).
"""
import numpy as np


def pack_codes(codes, wbits):
    codes = np.asarray(codes, np.int64)
    rows, cols = codes.shape
    if wbits == 8:
        assert codes.min() >= -128 and codes.max() <= 127
        return (codes & 0xFF).astype(np.uint8).reshape(rows, cols)
    assert codes.min() >= -8 and codes.max() <= 7 and cols % 2 == 0
    nib = (codes & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def make_block(gate_codes, up_codes, down_codes, gate_s, up_s, down_s, wbits):
    parts = [pack_codes(gate_codes, wbits).ravel(), pack_codes(up_codes, wbits).ravel(),
             pack_codes(down_codes, wbits).ravel()]
    for s in (gate_s, up_s, down_s):
        parts.append(np.ascontiguousarray(s, np.float32).ravel().view(np.uint8))
    return np.concatenate(parts)


def scales_shape(rows, cols, group):
    return (rows, cols // group) if group else (rows, 1)
