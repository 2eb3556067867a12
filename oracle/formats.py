"""Decoding of the packed expert block, float64.  (Oracle: test infrastructure only.)

The pages quantise experts to 4 bits with a per-block scale: Q4_0 style
"32 weights share a 2-byte scale" on the explainer page ("The bus problem"),
and NVFP4 (e2m1 values with FP8 E4M3 block scales) on the 95 GiB-on-32 GiB
page ("Decode") and the NVMe-streaming page ("Workflow").  The byte layout
itself is this project's (the pages give none):

block = gate [I x H] | up [I x H] | down [H x I]; each matrix with R rows and
C reduction columns is

* fp32:           R*C float32 row-major;
* int4 group 32:  nibbles [R, C/2] (element 2j low nibble of byte j, 2j+1
                  high), then scales [R, C/32] float16 LE; w = (q - 8) * s;
* e2m1 group 16:  nibbles as above holding e2m1 codes, then scales [R, C/16]
                  OCP E4M3 bytes; w = e4m3(s) * e2m1(q).

The number formats follow their public definitions (OCP 8-bit floating point
spec for E4M3 "fn": bias 7, no infinities, S.1111.111 is NaN, subnormals
m * 2^-9; OCP MX spec for e2m1: bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6).
"""
import numpy as np

F32, INT4_G32, E2M1_G16 = 0, 1, 2


def e2m1_value(code):
    """Value of a 4-bit e2m1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:                      # subnormal: 0 or 0.5
        mag = man * 0.5
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return sign * mag


def e4m3_value(code):
    """Value of an OCP E4M3 byte: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = man * 2.0 ** -9          # (man / 8) * 2^(1 - 7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def matrix_bytes(quant, rows, cols):
    n = rows * cols
    if quant == F32:
        return 4 * n
    if quant == INT4_G32:
        return n // 2 + 2 * (n // 32)
    if quant == E2M1_G16:
        return n // 2 + n // 16
    raise ValueError(quant)


def expert_bytes(quant, hidden, inter):
    return 2 * matrix_bytes(quant, inter, hidden) + matrix_bytes(quant, hidden, inter)


def _nibbles(plane, rows, cols):
    """Unpack [rows, cols/2] bytes into [rows, cols] codes (low nibble first)."""
    b = plane.reshape(rows, cols // 2)
    out = np.empty((rows, cols), dtype=np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def decode_matrix(quant, raw, rows, cols):
    """raw: uint8 bytes of one matrix -> float64 [rows, cols]."""
    raw = np.asarray(raw, dtype=np.uint8)
    assert raw.size == matrix_bytes(quant, rows, cols)
    if quant == F32:
        return raw.view("<f4").astype(np.float64).reshape(rows, cols)
    nib_len = rows * cols // 2
    q = _nibbles(raw[:nib_len], rows, cols)
    if quant == INT4_G32:
        s = raw[nib_len:].view("<f2").astype(np.float64).reshape(rows, cols // 32)
        return (q.astype(np.float64) - 8.0) * np.repeat(s, 32, axis=1)
    s = E4M3_TABLE[raw[nib_len:]].reshape(rows, cols // 16)
    return E2M1_TABLE[q] * np.repeat(s, 16, axis=1)


def decode_expert(quant, block, hidden, inter):
    """Packed block -> (W_gate [I,H], W_up [I,H], W_down [H,I]) in float64."""
    block = np.asarray(block, dtype=np.uint8)
    assert block.size == expert_bytes(quant, hidden, inter), (block.size, expert_bytes(quant, hidden, inter))
    out, off = [], 0
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        n = matrix_bytes(quant, rows, cols)
        out.append(decode_matrix(quant, block[off:off + n], rows, cols))
        off += n
    return tuple(out)
