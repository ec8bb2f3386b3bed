"""TEST INFRASTRUCTURE ONLY: a second, pure-Python statement of the EXQ1 bit layout.

It is written from the layout description (not from ``exq_oracle.c``) and in a
different shape: instead of computing a code's position, it walks each dword
of a column's group block and lists which (code, code bit) every bit holds,
the way a decoder consumes them:

  * a plane-0 dword of width p0 holds 8/p0 "units" t; unit t carries the four
    consecutive codes 4u..4u+3 (u = dword*8/p0 + t) at bit offsets
    p0*t + 0, +16, +8, +24 (codes 4u, 4u+1, 4u+2, 4u+3);
  * a plane-1 dword of width p1 serves R = p0/p1 consecutive plane-0 dwords;
    for the delta-th of them, the high field of the code at plane-0 offset
    p0*t + 16*e1 + 8*e2 sits at p0*t + 16*e1 + p1*delta + 8*e2.

Columns of a group block interleave at 16-byte word granularity: word j of
column n is at byte 16*(N*P_g + j*N + n).  Only meant for small layers.
"""
from __future__ import annotations

import numpy as np

PLANES = {2: (2,), 3: (2, 1), 4: (4,), 5: (4, 1), 6: (4, 2), 8: (8,)}


def dword_map(b: int):
    """For a width-b group: list over the column's 4*b dwords of 32 entries
    (code index, bit of that code)."""
    planes = PLANES[b]
    p0 = planes[0]
    per = 8 // p0
    lo = []
    for d in range(4 * p0):
        slots = [None] * 32
        for t in range(per):
            u = d * per + t
            for e, off in enumerate((0, 16, 8, 24)):
                for i in range(p0):
                    slots[p0 * t + off + i] = (4 * u + e, i)
        lo.append(slots)
    if len(planes) == 1:
        return lo
    p1 = planes[1]
    R = p0 // p1
    hi = []
    for h in range(4 * p1):
        slots = [None] * 32
        for delta in range(R):
            d = h * R + delta
            for t in range(per):
                u = d * per + t
                for e in range(4):
                    e1, e2 = e % 2, e // 2
                    pos = p0 * t + 16 * e1 + p1 * delta + 8 * e2
                    for i in range(p1):
                        slots[pos + i] = (4 * u + e, p0 + i)
        hi.append(slots)
    return lo + hi


def _dword_addr(N: int, Pg: int, n: int, m: int) -> int:
    return 16 * (N * Pg + (m // 4) * N + n) + 4 * (m % 4)


def pack(codes: np.ndarray, widths) -> np.ndarray:
    """codes uint8 [N][K] -> EXQ1 bytes."""
    N, K = codes.shape
    G = K // 128
    total = sum(int(b) * 16 * N for b in widths)
    out = bytearray(total)
    Pg = 0
    for g in range(G):
        b = int(widths[g])
        dmap = dword_map(b)
        for n in range(N):
            col = [int(c) for c in codes[n, 128 * g:128 * (g + 1)]]
            for m, slots in enumerate(dmap):
                word = 0
                for pos, (k, i) in enumerate(slots):
                    word |= ((col[k] >> i) & 1) << pos
                a = _dword_addr(N, Pg, n, m)
                out[a:a + 4] = word.to_bytes(4, "little")
        Pg += b
    return np.frombuffer(bytes(out), dtype=np.uint8)


def unpack(qweight: np.ndarray, K: int, N: int, widths) -> np.ndarray:
    G = K // 128
    codes = np.zeros((N, K), dtype=np.uint8)
    buf = bytes(np.asarray(qweight, dtype=np.uint8))
    Pg = 0
    for g in range(G):
        b = int(widths[g])
        dmap = dword_map(b)
        for n in range(N):
            col = [0] * 128
            for m, slots in enumerate(dmap):
                a = _dword_addr(N, Pg, n, m)
                word = int.from_bytes(buf[a:a + 4], "little")
                for pos, (k, i) in enumerate(slots):
                    col[k] |= ((word >> pos) & 1) << i
            codes[n, 128 * g:128 * (g + 1)] = col
        Pg += b
    return codes
