"""A host-side decoder of the packed expert blob, written from the layout's
definition (not from the packer's code), to check what the packer writes.

Layout of one packed matrix of R rows (R a multiple of 128) over a reduction
of C columns (a multiple of 32): slab s (rows 128 s .. 128 s + 127 in slab
row order), block b (columns 32 b .. 32 b + 31) is one 1280-byte record at
byte (s * C/32 + b) * 1280:

- 1024 code bytes, [64 lanes][4 dwords]: dword p of lane l holds the codes of
  slab rows A = 16 (2p) + l % 16 and B = 16 (2p + 1) + l % 16 at columns
  32 b + 8 (l // 16) + k, k = 0..7.  In that dword, byte 0 holds row A's
  codes k = 0, 2, 4, 6 and byte 1 row B's, at bit pairs 0, 2, 4, 6 of the
  byte; bytes 2 and 3 hold k = 1, 3, 5, 7 of rows A and B the same way.
- 256 scale bytes, fp16 [16][4][2]: entry (r, p, h) is the scale of slab row
  16 (2p + h) + r for block b.

Slab rows map to matrix rows: in the gate/up matrix, slab s row m < 64 is
gate row 64 s + m and row m >= 64 is up row 64 s + m - 64 (the canonical
array puts the gate rows first, then the up rows); in the down matrix slab
row m is row 128 s + m.
"""
import numpy as np

RECORD = 1280


def decode_matrix(blob: np.ndarray, R: int, C: int):
    """(codes uint8 [R][C], scales uint16 [R][C/32]) in slab row order."""
    nslab, nblk = R // 128, C // 32
    rec = np.asarray(blob, np.uint8)[: nslab * nblk * RECORD].reshape(nslab, nblk, RECORD)
    code_bytes = rec[:, :, :1024].reshape(nslab, nblk, 64, 4, 4)  # [s][b][lane][p][byte]
    codes = np.zeros((nslab, 128, nblk, 32), np.uint8)             # [s][slab row][b][column in block]
    for lane in range(64):
        r, kg = lane % 16, lane // 16
        for p in range(4):
            for byte in range(4):
                row = 16 * (2 * p + (byte & 1)) + r
                parity = byte >> 1
                v = code_bytes[:, :, lane, p, byte]
                for j in range(4):
                    k = 2 * j + parity
                    codes[:, row, :, 8 * kg + k] = (v >> (2 * j)) & 3
    scale_words = rec[:, :, 1024:].copy().view(np.uint16).reshape(nslab, nblk, 16, 4, 2)  # [s][b][r][p][h]
    scales = np.zeros((nslab, 128, nblk), np.uint16)
    for r in range(16):
        for p in range(4):
            for h in range(2):
                scales[:, 16 * (2 * p + h) + r, :] = scale_words[:, :, r, p, h]
    return codes.reshape(R, C), scales.reshape(R, nblk)


def gate_up_rows(I: int) -> np.ndarray:
    """Canonical row of each slab row of the gate/up matrix (2I rows)."""
    m = np.arange(2 * I)
    s, r = m // 128, m % 128
    return np.where(r < 64, 64 * s + r, I + 64 * s + r - 64)


def decode_expert(gate_up_blob: np.ndarray, down_blob: np.ndarray, H: int, I: int):
    """Canonical (codes_gu [2I][H], scales_gu, codes_d [H][I], scales_d) of one expert."""
    cg, sg = decode_matrix(gate_up_blob, 2 * I, H)
    rows = gate_up_rows(I)
    codes_gu = np.empty_like(cg)
    scales_gu = np.empty_like(sg)
    codes_gu[rows] = cg
    scales_gu[rows] = sg
    cd, sd = decode_matrix(down_blob, H, I)
    return codes_gu, scales_gu, cd, sd
