"""Container for a packed block-quantized weight and the byte layout it follows.

Layout (the same for every tensor of a format; W is N x K, row-major, and the
quantization blocks run along K inside a row; ``batch`` stacks experts):

* ``codes``    uint8 [batch][N][K/2]  -- 4-bit codes, element k = 2j in bits 0-3
                                        of byte j, element 2j+1 in bits 4-7.
                                        (Q6_K: the low 4 bits of each 6-bit code.)
* ``codes_hi`` uint8 [batch][N][K/4]  -- Q6_K only: the 2 high bits, element
                                        k = 4j+i in bits 2i..2i+1 of byte j.
* ``scales``   affine4_g64: float16 [batch][N][K/64][2] = (scale, bias) pairs
               mxfp4:       uint8   [batch][N][K/32]    E8M0 block scale
               nvfp4:       uint8   [batch][N][K/16]    E4M3 block scale
               q6_k:        int8    [batch][N][K/16]    sub-block scale
* ``scales2``  q6_k: float16 [batch][N][K/256] super-block scale d; else None
* ``tensor_scale`` nvfp4: float32 [batch] per-tensor multiplier; else None

This module only describes storage; it computes nothing.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

AFFINE4_G64 = 1
MXFP4 = 2
NVFP4 = 3
Q6_K = 4

NAMES = {AFFINE4_G64: "affine4_g64", MXFP4: "mxfp4", NVFP4: "nvfp4", Q6_K: "q6_k"}
BY_NAME = {v: k for k, v in NAMES.items()}

#: elements per scale block along K
BLOCK = {AFFINE4_G64: 64, MXFP4: 32, NVFP4: 16, Q6_K: 256}


@dataclass
class Packed:
    fmt: int
    n: int
    k: int
    batch: int
    codes: np.ndarray
    scales: np.ndarray
    codes_hi: np.ndarray | None = None
    scales2: np.ndarray | None = None
    tensor_scale: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def name(self) -> str:
        return NAMES[self.fmt]

    def planes(self):
        """(name, array) for every stored array, in ABI order."""
        out = [("codes", self.codes)]
        if self.codes_hi is not None:
            out.append(("codes_hi", self.codes_hi))
        out.append(("scales", self.scales))
        if self.scales2 is not None:
            out.append(("scales2", self.scales2))
        if self.tensor_scale is not None:
            out.append(("tensor_scale", self.tensor_scale))
        return out

    def nbytes(self) -> int:
        """Bytes of weight storage (codes + all scales)."""
        return int(sum(a.nbytes for _, a in self.planes()))

    def expert(self, e: int) -> "Packed":
        """View of one matrix of a batch."""
        sl = slice(e, e + 1)
        return Packed(self.fmt, self.n, self.k, 1, self.codes[sl], self.scales[sl],
                      None if self.codes_hi is None else self.codes_hi[sl],
                      None if self.scales2 is None else self.scales2[sl],
                      None if self.tensor_scale is None else self.tensor_scale[sl])

    def rows(self, r0: int, r1: int) -> "Packed":
        """View of rows r0..r1 of every matrix of the batch."""
        s = slice(r0, r1)
        return Packed(self.fmt, r1 - r0, self.k, self.batch, self.codes[:, s],
                      self.scales[:, s],
                      None if self.codes_hi is None else self.codes_hi[:, s],
                      None if self.scales2 is None else self.scales2[:, s],
                      self.tensor_scale)


def empty(fmt: int, n: int, k: int, batch: int = 1) -> Packed:
    """Zero-filled storage of the right shapes."""
    if k % BLOCK[fmt]:
        raise ValueError(f"K={k} is not a multiple of the {NAMES[fmt]} block {BLOCK[fmt]}")
    codes = np.zeros((batch, n, k // 2), np.uint8)
    hi = s2 = ts = None
    if fmt == AFFINE4_G64:
        sc = np.zeros((batch, n, k // 64, 2), np.float16)
    elif fmt == MXFP4:
        sc = np.zeros((batch, n, k // 32), np.uint8)
    elif fmt == NVFP4:
        sc = np.zeros((batch, n, k // 16), np.uint8)
        ts = np.ones((batch,), np.float32)
    elif fmt == Q6_K:
        hi = np.zeros((batch, n, k // 4), np.uint8)
        sc = np.zeros((batch, n, k // 16), np.int8)
        s2 = np.zeros((batch, n, k // 256), np.float16)
    else:
        raise ValueError(f"unknown format {fmt}")
    return Packed(fmt, n, k, batch, codes, sc, hi, s2, ts)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """uint8 codes 0..15 [..., K] -> bytes [..., K/2] (even k in the low nibble)."""
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def pack_crumbs(h: np.ndarray) -> np.ndarray:
    """uint8 values 0..3 [..., K] -> bytes [..., K/4] (k = 4j+i at bits 2i)."""
    h = h.astype(np.uint8)
    return (h[..., 0::4] | (h[..., 1::4] << 2) | (h[..., 2::4] << 4) | (h[..., 3::4] << 6)).astype(np.uint8)
