"""Exact decoding of the two stored weight formats (oracle; test infrastructure).

* BF16: the upper 16 bits of an IEEE binary32; value = binary32 with the low
  16 bits zero.  Decoded exactly into float64.
* E4M3FN (OCP 8-bit float, the FP8 weight format named in [OSDI] section 4.1:
  1 sign, 4 exponent, 3 mantissa bits, exponent bias 7, no infinities,
  maximum 448; S.1111.111 is NaN).  Normal codes: (-1)^s 2^(e-7) (1 + m/8);
  e = 0: (-1)^s 2^-6 (m/8).  Decoded from that definition into float64.
* Block-scaled FP8 matrix: one float32 scale per 128 x 128 tile of the
  [out, in] matrix; the weight is code value x scale of its tile ([OSDI]
  section 4.2 applies a shared per-block scale; the tile shape is 128 x 128).
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    tab = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            tab[c] = np.nan
        elif e == 0:
            tab[c] = s * 2.0 ** -6 * (m / 8.0)
        else:
            tab[c] = s * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return tab


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def dequant_b128(codes, scales, block: int = 128) -> np.ndarray:
    """[R, Cc] codes with [R/b, Cc/b] float32 scales -> float64 weights:
    element (r, c) is the code's value times the scale of tile (r//b, c//b).

    The table lookup and the product run as torch CPU ops (multi-threaded;
    numpy's gather takes seconds per expert matrix at full size); each
    element is still the one float64 product of the exact code value and its
    tile's scale, so the result is bit for bit the same as numpy's."""
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    R, Cc = c.shape
    v = torch.from_numpy(E4M3_VALUES)[c.long()]
    s = torch.from_numpy(np.asarray(scales, dtype=np.float32).astype(np.float64))
    return (v.view(R // block, block, Cc // block, block) * s[:, None, :, None]).reshape(R, Cc).numpy()
