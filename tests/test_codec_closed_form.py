"""The density-field carry of DF-SSD reads each value's ones count in closed form instead of running
the sigma-delta cell by cell: with U = e + 127 in [0, 254] at a value's first cell, c cells of target
t leave (U + c t) div 255 ones and U' = (U + c t) mod 255 ([DF-SSM] §3.4 steps 2-3, App. D). These
CPU tests tie that identity to the oracle's cell-by-cell definition: exhaustively over (U, t) for the
cell counts the supported d_state values give, and per value over whole rows of the oracle encoder."""
import numpy as np

from oracle import dfssm_oracle as O


def _cell_by_cell(U, t, c):
    e, ones = U - 127, 0
    for _ in range(c):
        v = e + t
        b = 1 if v >= 128 else 0
        e = v - 255 * b
        ones += b
    return ones, e + 127


def test_closed_form_equals_cell_by_cell_exhaustive():
    counts = set()
    for N in (16, 32, 64, 128, 256):
        cells = O.codec_cells(N)
        counts.update(int(cells[i + 1] - cells[i]) for i in range(N))
    assert counts and max(counts) < 32
    for c in sorted(counts):
        for U in range(255):
            for t in range(256):
                ones, U2 = _cell_by_cell(U, t, c)
                assert ones == (U + c * t) // 255 and U2 == (U + c * t) % 255, (U, t, c)


def test_closed_form_counts_match_oracle_rows():
    rng = np.random.default_rng(7)
    for N in (16, 64, 128, 256):
        cells = O.codec_cells(N)
        for k in range(20):
            row = (rng.standard_normal(N) * (0.1 if k % 2 else 3.0)).astype(np.float32)
            if k == 3:
                row[rng.integers(N)] = 40.0   # a spike: most codes at 0
            bits, mu, sigma = O.state_codec_encode_row(row)
            lo = np.float32(mu - np.float32(np.float32(3) * sigma))
            span = np.float32(np.float32(6) * sigma)
            x = np.clip(((row - lo).astype(np.float32) / span).astype(np.float32), np.float32(0), np.float32(1))
            t = np.rint((x * np.float32(255)).astype(np.float32)).astype(np.int64)
            U = 127
            for i in range(N):
                c = int(cells[i + 1] - cells[i])
                s = U + c * int(t[i])
                assert s // 255 == int(bits[cells[i]:cells[i + 1]].sum()), (N, k, i)
                U = s % 255
