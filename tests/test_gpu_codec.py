"""GPU parity of the density field state codec (dfssm_state_encode / dfssm_state_decode) against the
oracle ([DF-SSM] §3.4, App. D):
  - mu and sigma bit-equal to the oracle's fp32 element-order sums (same operations, correctly
    rounded division and square root on both sides);
  - every field bit equal to the oracle's encoding of the row with those mu and sigma (the 8-bit
    code t is decided in fp32 on both sides);
  - the readout of the GPU's field within 1e-6 of (|mu| + 6 sigma) of the oracle's fp64 readout of
    the same bits.
Rows: Gaussian, heavy-tailed (values past 3 sigma are clamped), constant (sigma = 0), one spike,
tiny sigma around a large mean; every supported d_state, ragged row counts, and the 1.3B state at
batch 64 on sampled rows."""
import dataclasses

import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
from test_gpu_decode import _lib, say

pytestmark = pytest.mark.gpu


def _dims(d_state: int):
    t = gen.DIMS["tiny"]
    nat = 2 * t.d_inner + 2 * t.ngroups * d_state + t.nheads
    return dataclasses.replace(t, d_state=d_state, n_in_proj=nat)


def _states(dims, batch: int, seed: int) -> np.ndarray:
    """[batch][H][P][N] fp32 with a mix of row kinds."""
    rng = np.random.default_rng(seed)
    shape = (batch, dims.nheads, dims.headdim, dims.d_state)
    S = (rng.standard_normal(shape) * 0.1).astype(np.float32)
    flat = S.reshape(-1, dims.d_state)
    n = flat.shape[0]
    kind = rng.integers(0, 6, n)
    for r in np.flatnonzero(kind == 1):                      # heavy tails
        flat[r] = (rng.standard_t(2, dims.d_state) * 0.05).astype(np.float32)
    for r in np.flatnonzero(kind == 2):                      # constant row
        flat[r] = np.float32(rng.choice([0.0, 0.375, -1.25]))
    for r in np.flatnonzero(kind == 3):                      # one spike
        flat[r] = 0.0
        flat[r, rng.integers(dims.d_state)] = np.float32(rng.standard_normal() * 3)
    for r in np.flatnonzero(kind == 4):                      # tiny spread around a large mean
        flat[r] = (50.0 + rng.standard_normal(dims.d_state) * 1e-4).astype(np.float32)
    return S


def _run(dims, S: np.ndarray):
    L, Dv = _lib()
    B = S.shape[0]
    ssm = torch.from_numpy(S).cuda()
    fields, stats = Dv.state_encode(dims, ssm, B)
    back = torch.full_like(ssm, float("nan"))
    Dv.state_decode(dims, fields, stats, B, back)
    torch.cuda.synchronize()
    f = fields.cpu().numpy().view(np.uint32)
    return f, stats.cpu().numpy(), back.cpu().numpy().reshape(-1, dims.d_state)


def _unpack(words: np.ndarray, K2: int) -> np.ndarray:
    bits = (words[:, None] >> np.arange(32, dtype=np.uint32)[None, :]) & 1
    return bits.reshape(-1)[:K2].astype(np.uint8)


def _check_rows(dims, S, f, st, back, rows, what):
    N = dims.d_state
    K2 = O.codec_field_side(N) ** 2
    flat = S.reshape(-1, N)
    assert f.shape[1] == (K2 + 31) // 32
    for r in rows:
        mu, sigma = O.state_codec_stats(flat[r])
        assert np.float32(st[r, 0]) == mu and np.float32(st[r, 1]) == sigma, \
            f"{what} row {r}: stats {st[r]} vs oracle ({mu}, {sigma})"
        bits = _unpack(f[r], K2)
        ref, _, _ = O.state_codec_encode_row(flat[r], mu, sigma)
        bad = np.flatnonzero(bits != ref)
        assert bad.size == 0, f"{what} row {r}: {bad.size} field bits differ, first cells {bad[:8]}"
        # unused bits of the last word stay zero
        tail = f[r, -1] >> (K2 % 32) if K2 % 32 else np.uint32(0)
        assert tail == 0, f"{what} row {r}: bits past cell {K2} set"
        dec = O.state_codec_decode_row(bits, mu, sigma, N)
        tol = 1e-6 * (abs(float(mu)) + 6 * float(sigma)) + 1e-30
        d = np.abs(back[r].astype(np.float64) - dec).max()
        assert d <= tol, f"{what} row {r}: readout off by {d} (tol {tol})"


@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("B", [1, 3])
def test_codec_every_row_small(N, B):
    dims = _dims(N)
    say(f"case: state codec, d_state {N}, batch {B} ({B * dims.nheads * dims.headdim} rows)")
    S = _states(dims, B, seed=N + B)
    f, st, back = _run(dims, S)
    rows = range(S.size // N) if N <= 64 else range(0, S.size // N, 3)
    _check_rows(dims, S, f, st, back, rows, f"N={N} B={B}")


def test_codec_1p3b_batch64_sampled():
    dims = gen.DIMS["1p3b"]
    B = 64
    say(f"case: state codec, 1.3B state at batch {B} (262144 rows of 128), 600 sampled rows")
    S = _states(dims, B, seed=7)
    f, st, back = _run(dims, S)
    n = S.size // dims.d_state
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 63, 64, n - 65, n - 1], rng.integers(0, n, 595)]))
    _check_rows(dims, S, f, st, back, rows, "1p3b B=64")
    # every constant row reads back exactly as its value
    flat = S.reshape(-1, dims.d_state)
    const = np.flatnonzero((flat == flat[:, :1]).all(axis=1))
    assert const.size > 0
    assert (back[const] == flat[const]).all()
    assert (f[const] == 0).all() and (st[const, 1] == 0).all()


def test_codec_reconstruction_error_bound():
    """Quantisation + density error of the values inside mu +- 3 sigma: each read-back value lies within
    6 sigma * (1/(2*255) + 1/cells) of the original (8-bit code, then a density over >= cells bits
    whose running error stays within one code step)."""
    dims = _dims(128)
    rng = np.random.default_rng(5)
    S = np.clip(rng.standard_normal((2, dims.nheads, dims.headdim, 128)), -2.5, 2.5).astype(np.float32)
    say("case: state codec error bound, d_state 128, batch 2")
    f, st, back = _run(dims, S)
    flat = S.reshape(-1, 128)
    cells = np.diff(O.codec_cells(128))
    bound = 6 * st[:, 1:2].astype(np.float64) * (0.5 / 255 + 1.0 / cells[None, :]) * (1 + 1e-5)
    err = np.abs(back.astype(np.float64) - flat)
    lo = st[:, :1].astype(np.float64) - 3 * st[:, 1:2]
    hi = st[:, :1].astype(np.float64) + 3 * st[:, 1:2]
    inside = (flat >= lo) & (flat <= hi)
    assert inside.mean() > 0.99
    assert (err[inside] <= bound[inside]).all(), float((err / bound)[inside].max())
