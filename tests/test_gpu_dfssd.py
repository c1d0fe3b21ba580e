"""GPU parity of DF-SSD, the density field codec at the chunk boundaries of the prefill scan
(dfssm_layer_prefill_ex with state_codec; [DF-SSM] §3.4, App. D), against the oracle:
  - the state entering chunk 0 is the initial state, untouched;
  - at every later boundary the state the chunk uses equals the oracle's codec applied to the GPU's
    own state before the codec, to 1e-6 of (|mu| + 6 sigma) per row (one field bit apart would be
    at least 6 sigma / 5 apart, so this holds the codec's decisions exact);
  - with the GPU's codes and its coded states forced in, the oracle's layer (DF-SSD, sequential)
    matches the outputs, the final conv/SSM states and the pre-codec states of every boundary to
    1e-3 (P2), and the codes are exact against the oracle quantizer of the GPU's own u (P1)."""
import dataclasses

import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say

pytestmark = pytest.mark.gpu


def run_dfssd(dims, lw, xs, conv0, ssm0, chunk, bf16=False):
    L, Dv = _lib()
    B, T = xs.shape[:2]
    nch = (T + chunk - 1) // chunk
    dev = Dv.DeviceLayer(lw)
    st = Dv.DeviceState(conv0, ssm0)
    x = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
    if bf16:
        x = x.to(torch.bfloat16)
        assert (x.float().cpu().numpy() == xs).all()
    y = torch.empty((B, T, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_LAYER_PREFILL, B, T)
    tp = Dv.Taps(dims, B * T)
    shp = (nch, B, dims.nheads, dims.headdim, dims.d_state)
    pre = torch.full(shp, float("nan"), device="cuda")
    ent = torch.full(shp, float("nan"), device="cuda")
    Dv.layer_prefill(dims, dev, st, x, y, chunk, ws, tp, state_codec=True, chunk_state_pre=pre, chunk_state_in=ent)
    torch.cuda.synchronize()
    tps = {k: v.reshape(B, T, *v.shape[1:]) for k, v in tp.numpy().items()}
    return (y.cpu().numpy(), tps, (st.conv.cpu().numpy(), st.ssm.cpu().numpy()), pre.cpu().numpy(),
            ent.cpu().numpy())


def check_codec_boundaries(pre, ent, ssm0, rows_per_boundary=None, seed=0):
    nch, B = pre.shape[:2]
    N = pre.shape[-1]
    assert np.array_equal(pre[0], ssm0) and np.array_equal(ent[0], ssm0)
    rng = np.random.default_rng(seed)
    for c in range(1, nch):
        P = pre[c].reshape(-1, N)
        Q = ent[c].reshape(-1, N)
        rows = range(P.shape[0]) if rows_per_boundary is None else rng.choice(P.shape[0], rows_per_boundary, False)
        for r in rows:
            bits, mu, sigma = O.state_codec_encode_row(P[r])
            ref = O.state_codec_decode_row(bits, mu, sigma, N)
            tol = 1e-6 * (abs(float(mu)) + 6 * float(sigma)) + 1e-30
            d = np.abs(Q[r].astype(np.float64) - ref).max()
            assert d <= tol, f"boundary {c} row {r}: coded state off by {d} (tol {tol})"


def check_forced(lw, xs, conv0, ssm0, out, tps, final, pre, ent, chunk, what):
    T = xs.shape[0]
    for t in range(T):
        PY.assert_codes_exact(tps["in_u"][t], tps["in_q"][t], tps["in_s"][t][0], f"{what} t={t} in")
        PY.assert_codes_exact(tps["out_u"][t], tps["out_q"][t], tps["out_s"][t][0], f"{what} t={t} out")
    force = dict(in_q=tps["in_q"], in_s=tps["in_s"][:, 0], out_q=tps["out_q"], out_s=tps["out_s"][:, 0],
                 state_in=ent)
    o, cs, ss, otp = O.layer_tokens(xs, lw, conv0, ssm0, force=force, codec_chunk=chunk)
    assert (tps["in_acc"].astype(np.int64)[:, :otp["in_acc"].shape[1]] == otp["in_acc"]).all(), what
    assert (tps["out_acc"].astype(np.int64) == otp["out_acc"]).all(), what
    errs = dict(out=max(PY.err(out[t], o[t]) for t in range(T)), conv=PY.err(final[0], cs), ssm=PY.err(final[1], ss),
                out_u=max(PY.err(tps["out_u"][t], otp["out_u"][t]) for t in range(T)),
                pre=max([PY.err(pre[c], otp["state_pre"][c]) for c in range(1, pre.shape[0])] or [0.0]))
    say(f"{what}: {errs}")
    for k, v in errs.items():
        assert v < PY.TOL_LAYER, (what, k, errs)


@pytest.mark.parametrize("chunk", [16, 64])
def test_dfssd_tiny_ragged_two_sequences(chunk):
    dims = gen.DIMS["tiny"]
    lw = gen.layer_weights(dims, 0, seed=21, random_norms=True, per_channel_lora=True)
    B, T = 2, 150
    xs = gen.token_inputs(dims, (B, T), 21, tag=3)
    conv0, ssm0 = gen.initial_states(dims, B, 0, 21, std=0.1)
    say(f"case: DF-SSD tiny layer, batch {B}, {T} tokens, chunk {chunk}")
    out, tps, final, pre, ent = run_dfssd(dims, lw, xs, conv0, ssm0, chunk)
    for b in range(B):
        check_codec_boundaries(pre[:, b:b + 1], ent[:, b:b + 1], ssm0[b:b + 1])
        check_forced(lw, xs[b], conv0[b], ssm0[b], out[b], {k: v[b] for k, v in tps.items()},
                     (final[0][b], final[1][b]), pre[:, b], ent[:, b], chunk, f"tiny chunk {chunk} b{b}")


@pytest.mark.parametrize("d_state", [32, 64, 256])
def test_dfssd_every_carry_geometry(d_state):
    """The carry codes rows one lane per row below d_state 64 and splits each row over d_state / 32
    lanes from 64 up (sums passed lane to lane, the sigma-delta start from a prefix): tiny layers
    widened to those d_state, 3 chunks of 64 with a ragged last one, non-zero entering states."""
    t = gen.DIMS["tiny"]
    dims = dataclasses.replace(t, d_state=d_state, n_in_proj=2 * t.d_inner + 2 * t.ngroups * d_state + t.nheads)
    lw = gen.layer_weights(dims, 0, seed=23, random_norms=True, per_channel_lora=True)
    B, T, chunk = 2, 150, 64
    xs = gen.token_inputs(dims, (B, T), 23, tag=5)
    conv0, ssm0 = gen.initial_states(dims, B, 0, 23, std=0.2)
    say(f"case: DF-SSD tiny layer d_state {d_state}, batch {B}, {T} tokens, chunk {chunk}")
    out, tps, final, pre, ent = run_dfssd(dims, lw, xs, conv0, ssm0, chunk)
    for b in range(B):
        check_codec_boundaries(pre[:, b:b + 1], ent[:, b:b + 1], ssm0[b:b + 1])
        check_forced(lw, xs[b], conv0[b], ssm0[b], out[b], {k: v[b] for k, v in tps.items()},
                     (final[0][b], final[1][b]), pre[:, b], ent[:, b], chunk, f"d_state {d_state} b{b}")


def test_dfssd_single_chunk_is_the_plain_prefill():
    """One chunk covers the sequence: no boundary, so DF-SSD must give the plain prefill's outputs and
    conv state bit for bit, and its final SSM state up to the rounding of the last carry (the codec
    carry forms exp(Lam) S + S_loc with two roundings, the plain scan may fuse them)."""
    L, Dv = _lib()
    dims = gen.DIMS["tiny"]
    lw = gen.layer_weights(dims, 0, seed=22)
    xs = gen.token_inputs(dims, (1, 40), 22, tag=4)
    conv0, ssm0 = gen.initial_states(dims, 1, 0, 22, std=0.1)
    say("case: DF-SSD with one chunk against the plain prefill")
    out, _, final, pre, ent = run_dfssd(dims, lw, xs, conv0, ssm0, 64)
    from test_gpu_prefill import run_prefill
    out2, _, final2 = run_prefill(dims, lw, xs, conv0, ssm0, 64)
    assert np.array_equal(out, out2) and np.array_equal(final[0], final2[0])
    assert np.abs(final[1] - final2[1]).max() <= 1e-6 * np.abs(final2[1]).max()


def test_dfssd_1p3b_layer_2048_tokens_bf16():
    dims = gen.DIMS["1p3b"]
    lw = gen.layer_weights(dims, 0, seed=0)
    xs = gen.token_inputs(dims, (1, 2048), 0, tag=5, bf16=True)
    conv0, ssm0 = gen.initial_states(dims, 1, 0, 0, std=0.1)
    say("case: DF-SSD 1.3B layer, 2048 bf16 tokens, chunk 256 (7 coded boundaries)")
    out, tps, final, pre, ent = run_dfssd(dims, lw, xs, conv0, ssm0, 256, bf16=True)
    check_codec_boundaries(pre, ent, ssm0, rows_per_boundary=48, seed=1)
    check_forced(lw, xs[0], conv0[0], ssm0[0], out[0], {k: v[0] for k, v in tps.items()}, (final[0][0], final[1][0]),
                 pre[:, 0], ent[:, 0], 256, "1p3b")


def test_dfssd_stack_prefill_equals_the_layer_calls():
    """dfssm_stack_prefill_ex with state_codec: the same bits as DF-SSD layer prefills one after the
    other plus the library's final norm (the same kernels), and every layer's coded boundaries hold
    the codec's decisions (checked through the layer calls' taps)."""
    L, Dv = _lib()
    dims = gen.DIMS["tiny"]
    nL, B, T, Q = 3, 2, 130, 32
    layers = gen.stack_weights(dims, nL, seed=23)
    states0 = [gen.initial_states(dims, B, l, 23, std=0.1) for l in range(nL)]
    xs = gen.token_inputs(dims, (B, T), 23, tag=6)
    fw = np.random.default_rng(23).uniform(0.5, 1.5, dims.d_model).astype(np.float32)
    say(f"case: DF-SSD tiny stack prefill, {nL} layers, batch {B}, {T} tokens, chunk {Q}")
    devs = [Dv.DeviceLayer(w) for w in layers]
    sts = [Dv.DeviceState(c, s) for c, s in states0]
    x = torch.from_numpy(xs).cuda()
    y = torch.empty((B, T, dims.d_model), device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_PREFILL, B, T, nL)
    Dv.stack_prefill(dims, devs, sts, torch.from_numpy(fw).cuda(), x, y, Q, ws, state_codec=True)
    torch.cuda.synchronize()
    ys = y.cpu().numpy()
    finals = [(s.ssm.cpu().numpy(), s.conv.cpu().numpy()) for s in sts]
    h = xs
    for l in range(nL):
        out, _, final, pre, ent = run_dfssd(dims, layers[l], h, states0[l][0], states0[l][1], Q)
        check_codec_boundaries(pre, ent, states0[l][1])
        assert np.array_equal(final[1], finals[l][0]) and np.array_equal(final[0], finals[l][1]), l
        h = out
    assert np.abs(O.rmsnorm(h, fw, dims.eps) - ys).max() < 1e-5
