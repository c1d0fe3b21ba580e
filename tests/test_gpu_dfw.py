"""GPU parity of the 17-level scaffold projection (dfssm_dfw_project, [DF-SSM] §3.1 Eq. (1), §3.2
Eq. (3)) against the oracle: the int8 codes and scales of the quantizer bit-exact, the scaffold sums
acc and the LoRA-down sums t exact, y within 1e-3 (element-wise bound). Shapes: ragged row counts
and token groups, non-power-of-two chunk counts, the 1.3B in_proj and out_proj, n_in 8192."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say

pytestmark = pytest.mark.gpu


def _run(P, xs):
    L, Dv = _lib()
    dp = Dv.DeviceDfwProj(P)
    B = xs.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(xs, np.float32)).cuda()
    y = torch.full((B, P.n_out), float("nan"), device="cuda")
    taps = dict(q=torch.empty((B, P.n_in), dtype=torch.int8, device="cuda"), s=torch.empty(B, device="cuda"),
                acc=torch.empty((B, P.n_out), dtype=torch.int32, device="cuda"),
                t=torch.empty((B, P.rank), dtype=torch.int32, device="cuda"))
    Dv.dfw_project(dp, x, y, taps=taps)
    torch.cuda.synchronize()
    return y.cpu().numpy(), {k: v.cpu().numpy() for k, v in taps.items()}


def _check(P, xs, y, taps, what, levels=None):
    k = O.dfw_unpack_planes(P.planes, P.n_in) if levels is None else levels
    for b in range(xs.shape[0]):
        q, s = O.quantize_token(xs[b])
        assert (taps["q"][b] == q).all() and np.float32(taps["s"][b]) == s, f"{what} token {b}: codes"
        yo, acc, t = O.project_dfw(q, s, P, k=k)
        assert (taps["t"][b].astype(np.int64) == t).all(), f"{what} token {b}: LoRA-down sums"
        bad = np.flatnonzero(taps["acc"][b].astype(np.int64) != acc)
        assert bad.size == 0, f"{what} token {b}: {bad.size} scaffold sums differ, e.g. rows {bad[:5]}"
        e = PY.err(y[b], yo)
        assert e < PY.TOL_LAYER, (what, b, e)


@pytest.mark.parametrize("n_out,n_in,rank,B", [(72, 256, 8, 1), (72, 256, 8, 3), (200, 384, 5, 5),
                                               (33, 128, 1, 2), (130, 1024, 64, 9)])
def test_dfw_small_shapes(n_out, n_in, rank, B):
    P = gen.dfw_proj(n_out, n_in, rank, seed=n_out + B)
    xs = np.random.default_rng(B).standard_normal((B, n_in)).astype(np.float32)
    say(f"case: 17-level projection {n_out} x {n_in}, rank {rank}, batch {B}")
    y, taps = _run(P, xs)
    _check(P, xs, y, taps, f"{n_out}x{n_in} B={B}")


@pytest.mark.parametrize("name,n_out,n_in,B", [("in_proj", 8512, 2048, 1), ("in_proj", 8512, 2048, 4),
                                               ("out_proj", 2048, 4096, 1), ("out_proj", 2048, 4096, 2)])
def test_dfw_1p3b_projections(name, n_out, n_in, B):
    P = gen.dfw_proj(n_out, n_in, 32, seed=1)
    xs = np.random.default_rng(2).standard_normal((B, n_in)).astype(np.float32)
    say(f"case: 17-level {name} of the 1.3B layer ({n_out} x {n_in}), batch {B}")
    y, taps = _run(P, xs)
    _check(P, xs, y, taps, f"{name} B={B}")


def test_dfw_wide_input_and_latent_weights_through_eq1():
    # latent weights through Eq. (1) (the oracle's quantizer), then the GPU projection of the result
    rng = np.random.default_rng(9)
    w = rng.normal(0.0, 0.6, size=(96, 8192))
    _, k = O.dfw_quantize(w)
    P = gen.dfw_proj(96, 8192, 16, seed=9, levels=k)
    xs = rng.standard_normal((3, 8192)).astype(np.float32)
    xs[1] = 0.0                                    # a zero token: q = 0, s = 0, y = 0
    say("case: 17-level projection 96 x 8192 from Eq. (1) levels, batch 3 with a zero token")
    y, taps = _run(P, xs)
    _check(P, xs, y, taps, "eq1 8192", levels=k)
    assert (y[1] == 0).all() and taps["s"][1] == 0
