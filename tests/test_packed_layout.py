"""The host decoder of the packed layout on hand-made records (CPU): single
codes and scales placed by the layout's definition land where it says."""
import numpy as np

import packed_layout as PL


def _blob(R, C):
    return np.zeros((R // 128) * (C // 32) * PL.RECORD, np.uint8)


def test_one_code_lands_on_its_row_and_column():
    R, C = 128, 64
    blob = _blob(R, C)
    # slab 0, block 1, lane 17 (row 1 of its fragment, k group 1), dword 2, byte 3
    # (row B of fragments 4/5, odd k), bits 6-7 (j = 3): code 1 at row 16*5 + 1, k = 7
    off = 1 * PL.RECORD + (17 * 4 + 2) * 4 + 3
    blob[off] = 1 << 6
    codes, scales = PL.decode_matrix(blob, R, C)
    assert codes[81, 32 + 8 + 7] == 1
    assert np.count_nonzero(codes) == 1 and np.count_nonzero(scales) == 0


def test_every_bit_pair_is_one_code():
    R, C = 256, 32  # two slabs, one block
    blob = _blob(R, C)
    blob[PL.RECORD: PL.RECORD + 1024] = 0xFF  # slab 1: every code 3
    codes, _ = PL.decode_matrix(blob, R, C)
    assert np.all(codes[128:] == 3) and np.all(codes[:128] == 0)


def test_one_scale_lands_on_its_row():
    R, C = 128, 96
    blob = _blob(R, C)
    # block 2, scale entry (r = 5, p = 3, h = 1): slab row 16 * 7 + 5
    off = 2 * PL.RECORD + 1024 + ((5 * 4 + 3) * 2 + 1) * 2
    blob[off:off + 2] = np.frombuffer(np.uint16(0x3C00).tobytes(), np.uint8)
    _, scales = PL.decode_matrix(blob, R, C)
    assert scales[117, 2] == 0x3C00 and np.count_nonzero(scales) == 1


def test_gate_up_rows_interleave_64_gate_then_64_up():
    rows = PL.gate_up_rows(192)  # I = 192: 3 slabs
    assert list(rows[:64]) == list(range(64)) and list(rows[64:128]) == list(range(192, 256))
    assert list(rows[128:192]) == list(range(64, 128)) and sorted(rows) == list(range(384))
