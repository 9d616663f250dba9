"""Storage-format decoders, written from the format definitions (test infrastructure only).

bf16: the upper 16 bits of an IEEE-754 binary32; decoding shifts the pattern into the top half.
E4M3FN (OCP 8-bit floating point, "FN" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 encodes subnormals m * 2^-9; no infinities; codes 0x7F and 0xFF are NaN;
largest finite magnitude 448.  The pages name FP8 storage for the indexer path ([P1] §4, [P3] §3.3)
without fixing the flavour; E4M3FN is this library's reading.
E8M0 (the shared scale of the OCP Microscaling formats, which [P1] §4 and [P3] §3.3 name as MXFP8
for the indexer): an unsigned 8-bit biased exponent with no sign and no mantissa, value
2^(e - 127) for e in 0..254; e = 255 is NaN.
"""
import numpy as np


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def e4m3_table() -> np.ndarray:
    """Value of every one of the 256 E4M3FN codes, as float64."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            tab[code] = np.nan
        elif exp == 0:
            tab[code] = sign * man * 2.0 ** -9
        else:
            tab[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return tab


_E4M3 = e4m3_table()


def e4m3_codes_to_f64(u8: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(u8, dtype=np.uint8)]


def e8m0_to_f64(u8: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(e - 127), NaN for 255."""
    e = np.asarray(u8, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, e - 127).astype(np.float64)
    out[e == 255] = np.nan
    return out
