"""GPU parity of dfssm_layer_prefill against the CPU oracle.

Prefill is defined as sequential decode steps (quantization is per token); the kernels evaluate
the projections as int8 MFMA GEMMs over all tokens and the recurrence as a chunked scan. Every
case checks the P1/P2 protocol of dfssm_parity per token: codes exact against the oracle
quantizer of the GPU's own u, integer sums exact, and the oracle run with the GPU's codes forced
in within 1e-3 on outputs and on the final conv/SSM states."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say, run_layer

pytestmark = pytest.mark.gpu

TINY = gen.DIMS["tiny"]
BIG = gen.DIMS["1p3b"]


def run_prefill(dims, lw, xs, conv0, ssm0, chunk, bf16=False, taps=True):
    """xs [B][L][D] fp32 (bf16-representable when bf16) -> (out [B][L][D], taps [B][L][...], states)."""
    L, Dv = _lib()
    B, T = xs.shape[:2]
    dev = Dv.DeviceLayer(lw)
    st = Dv.DeviceState(conv0, ssm0)
    x = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
    if bf16:
        x = x.to(torch.bfloat16)
        assert (x.float().cpu().numpy() == xs).all(), "inputs must be bf16-representable"
    y = torch.empty((B, T, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_LAYER_PREFILL, B, T)
    tp = Dv.Taps(dims, B * T) if taps else None
    Dv.layer_prefill(dims, dev, st, x, y, chunk, ws, tp)
    torch.cuda.synchronize()
    tps = None
    if taps:
        tps = {k: v.reshape(B, T, *v.shape[1:]) for k, v in tp.numpy().items()}
    return y.cpu().numpy(), tps, (st.conv.cpu().numpy(), st.ssm.cpu().numpy())


def check_sequence(lw, xs, conv0, ssm0, out, tps, final, dense=None, tol=PY.TOL_LAYER, what="", final_w=None):
    """P1 + P2 over one sequence (batch row): xs [T][D], tps dict of [T][...]. With final_w, `out`
    is the stack's output RMSNorm(h) * final_w of this (last) layer's residual h."""
    T = xs.shape[0]
    assert (tps["h_in"] == xs).all(), f"{what}: h_in tap is not the layer input"
    for t in range(T):
        PY.assert_codes_exact(tps["in_u"][t], tps["in_q"][t], tps["in_s"][t][0], f"{what} t={t} in")
        PY.assert_codes_exact(tps["out_u"][t], tps["out_q"][t], tps["out_s"][t][0], f"{what} t={t} out")
    force = dict(in_q=tps["in_q"], in_s=tps["in_s"][:, 0], out_q=tps["out_q"], out_s=tps["out_s"][:, 0])
    o, cs, ss, otp = O.layer_tokens(xs, lw, conv0, ssm0, force=force, dense=dense)
    # the oracle's integer sums of the GPU's codes (P1)
    assert (tps["in_acc"].astype(np.int64)[:, :otp["in_acc"].shape[1]] == otp["in_acc"]).all(), f"{what}: in acc"
    assert (tps["in_t"].astype(np.int64) == otp["in_t"]).all(), f"{what}: in t"
    assert (tps["out_acc"].astype(np.int64) == otp["out_acc"]).all(), f"{what}: out acc"
    assert (tps["out_t"].astype(np.int64) == otp["out_t"]).all(), f"{what}: out t"
    e_in = max(PY.err(tps["in_u"][t], otp["in_u"][t]) for t in range(T))
    e_ou = max(PY.err(tps["out_u"][t], otp["out_u"][t]) for t in range(T))
    if final_w is not None:
        o = O.rmsnorm(o, final_w, lw.dims.eps)
    e_o = max(PY.err(out[t], o[t]) for t in range(T))
    e_c, e_s = PY.err(final[0], cs), PY.err(final[1], ss)
    errs = dict(in_u=e_in, out_u=e_ou, out=e_o, conv=e_c, ssm=e_s)
    assert e_in < 1e-5, f"{what}: {errs}"
    for k in ("out_u", "out", "conv", "ssm"):
        assert errs[k] < tol, f"{what}: {k} {errs}"
    return errs


def free_running_sequence(lw, xs, conv0, ssm0, out, tps, dense=None, what=""):
    """The oracle on its own codes. In-codes depend only on the inputs, so every in-code flip must
    sit at a rounding tie; out-codes and outputs are compared up to the first in-code flip."""
    o, _, _, otp = O.layer_tokens(xs, lw, conv0, ssm0, dense=dense)
    T = xs.shape[0]
    first = T
    for t in range(T):
        f, ok = PY.flips_at_ties(otp["in_u"][t], otp["in_q"][t], tps["in_q"][t])
        if f:
            assert ok, f"{what} t={t}: an in-code flip away from a rounding tie"
            first = min(first, t)
    errs = []
    for t in range(first):
        f, ok = PY.flips_at_ties(otp["out_u"][t], otp["out_q"][t], tps["out_q"][t])
        if f:
            assert ok, f"{what} t={t}: an out-code flip away from a rounding tie"
            continue
        errs.append(PY.err(out[t], o[t]))
    if errs:
        assert max(errs) < PY.TOL_LAYER, f"{what}: {max(errs)}"
    return (max(errs) if errs else 0.0), first


@pytest.mark.parametrize("chunk", [16, 64, 256])
def test_prefill_tiny_ragged_nonzero_state(chunk):
    B, T = 2, 300      # 300 = ragged for every chunk length
    lw = gen.layer_weights(TINY, 5, 11, random_norms=True, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(TINY, B, 5, 11, std=0.3)
    xs = gen.token_inputs(TINY, (B, T), 11, tag=1)
    say(f"case: tiny prefill, batch {B}, seqlen {T}, chunk {chunk}, nonzero state, fp32 input")
    out, tps, final = run_prefill(TINY, lw, xs, conv0, ssm0, chunk)
    dense = O.dense_signs(lw)
    for b in range(B):
        tb = {k: v[b] for k, v in tps.items()}
        errs = check_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], tb, (final[0][b], final[1][b]), dense,
                              what=f"chunk {chunk} row {b}")
        fr, first = free_running_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], tb, dense, what=f"row {b}")
        say(f"chunk {chunk} row {b}: forced {errs}; free-running {fr:.2e} up to token {first}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 33])
def test_prefill_tiny_short_sequences_bf16(T):
    """Sequences shorter than the conv window (the new conv state still holds old entries) and
    than one chunk, with bf16 inputs."""
    B = 3
    lw = gen.layer_weights(TINY, 6, 12, random_norms=True)
    conv0, ssm0 = gen.initial_states(TINY, B, 6, 12, std=0.3)
    xs = gen.token_inputs(TINY, (B, T), 12, tag=2, bf16=True)
    say(f"case: tiny prefill, batch {B}, seqlen {T}, chunk 32, bf16 input")
    out, tps, final = run_prefill(TINY, lw, xs, conv0, ssm0, 32, bf16=True)
    dense = O.dense_signs(lw)
    for b in range(B):
        tb = {k: v[b] for k, v in tps.items()}
        check_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], tb, (final[0][b], final[1][b]), dense,
                       what=f"T={T} row {b}")


def test_prefill_then_decode_state_handoff():
    """prefill(L1) leaves the state that L2 decode steps continue from: the oracle runs all
    L1 + L2 tokens in one sequence with the GPU's codes forced in."""
    L1, L2 = 100, 6
    lw = gen.layer_weights(TINY, 7, 13, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(TINY, 1, 7, 13, std=0.2)
    xs = gen.token_inputs(TINY, (1, L1 + L2), 13, tag=3)
    say(f"case: tiny prefill {L1} tokens (chunk 32) then {L2} decode steps")
    out_p, tps_p, mid = run_prefill(TINY, lw, xs[:, :L1], conv0, ssm0, 32)
    xs_d = np.ascontiguousarray(np.transpose(xs[:, L1:], (1, 0, 2)))     # [L2][1][D]
    out_d, tps_d, final, _ = run_layer(TINY, lw, xs_d, mid[0], mid[1])
    tps = {k: np.concatenate([tps_p[k][0], np.stack([tp[k][0] for tp in tps_d])]) for k in tps_p}
    out = np.concatenate([out_p[0], out_d[:, 0]])
    errs = check_sequence(lw, xs[0], conv0[0], ssm0[0], out, tps, (final[0][0], final[1][0]), what="handoff")
    say(f"handoff: {errs}")


def test_prefill_degenerate_zero_tokens_and_dt_zero():
    """All-zero tokens take the a == 0 quantizer path; dt -> 0 leaves the SSM state unchanged."""
    lw = gen.layer_weights(TINY, 8, 14)
    conv0, ssm0 = gen.initial_states(TINY, 1, 8, 14, std=0.3)
    xs = gen.token_inputs(TINY, (1, 40), 14, tag=4)
    xs[0, 3] = 0
    xs[0, 17] = 0
    say("case: tiny prefill with all-zero tokens, chunk 16")
    out, tps, final = run_prefill(TINY, lw, xs, conv0, ssm0, 16)
    assert not tps["in_q"][0, 3].any() and tps["in_s"][0, 3, 0] == 0
    check_sequence(lw, xs[0], conv0[0], ssm0[0], out[0], {k: v[0] for k, v in tps.items()},
                   (final[0][0], final[1][0]), what="zero tokens")
    lw.dt_bias[:] = -100.0
    say("case: tiny prefill with dt -> 0, chunk 64")
    out, tps, final = run_prefill(TINY, lw, xs, conv0, ssm0, 64, taps=False)
    assert (final[1] == ssm0).all()


def test_prefill_1p3b_2048_tokens_bf16_chunk256():
    """One layer of the 2048-token bf16 prefill workload (1.3B shape, chunk 256): every token."""
    T = 2048
    lw = gen.layer_weights(BIG, 0, 0)
    conv0, ssm0 = gen.initial_states(BIG, 1)
    xs = gen.token_inputs(BIG, (1, T), 0, tag=5, bf16=True)
    say(f"case: 1.3B-shaped layer prefill, seqlen {T}, chunk 256, bf16 input")
    out, tps, final = run_prefill(BIG, lw, xs, conv0, ssm0, 256, bf16=True)
    dense = O.dense_signs(lw)
    tb = {k: v[0] for k, v in tps.items()}
    errs = check_sequence(lw, xs[0], conv0[0], ssm0[0], out[0], tb, (final[0][0], final[1][0]), dense,
                          what="1p3b prefill")
    fr, first = free_running_sequence(lw, xs[0], conv0[0], ssm0[0], out[0], tb, dense, what="1p3b")
    say(f"1p3b prefill: forced {errs}; free-running {fr:.2e} up to token {first}")


def test_prefill_1p3b_two_ragged_sequences_nonzero_state():
    """Two 1.3B-shaped sequences of 1,100 tokens (2,200 rows: the one-round in_proj GEMM with the
    B|C|dt blocks riding along; the second sequence starts inside a 128-row tile) with nonzero initial
    conv and SSM states, chunk 256, fp32 input: every token of both sequences and both final states."""
    B, T = 2, 1100
    lw = gen.layer_weights(BIG, 3, 7)
    conv0, ssm0 = gen.initial_states(BIG, B, 3, 7, std=0.3)
    xs = gen.token_inputs(BIG, (B, T), 7, tag=6)
    say(f"case: 1.3B-shaped layer prefill, batch {B}, seqlen {T}, chunk 256, nonzero state, fp32 input")
    out, tps, final = run_prefill(BIG, lw, xs, conv0, ssm0, 256)
    dense = O.dense_signs(lw)
    for b in range(B):
        tb = {k: v[b] for k, v in tps.items()}
        errs = check_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], tb, (final[0][b], final[1][b]), dense,
                              what=f"1p3b two sequences, row {b}")
        say(f"1p3b two sequences row {b}: forced {errs}")


def test_prefill_chunk_lengths_agree():
    """Every chunk length evaluates the same recurrence. The quantizer rounds half to even, so two
    correct evaluations that differ by rounding may pick different codes where u * 127 / max|u|
    sits at a .5 boundary: every code that differs from the chunk-256 run must sit at such a tie,
    and outputs (and, without a flip, the final states) agree within the layer tolerance up to the
    first token with a flip."""
    lw = gen.layer_weights(TINY, 9, 15)
    conv0, ssm0 = gen.initial_states(TINY, 1, 9, 15, std=0.2)
    T = 257
    xs = gen.token_inputs(TINY, (1, T), 15, tag=6)
    outs = {}
    for c in (16, 32, 64, 128, 256):
        say(f"case: tiny prefill seqlen {T} chunk {c}")
        outs[c] = run_prefill(TINY, lw, xs, conv0, ssm0, c)
    ref_out, ref_tp, ref_st = outs[256]
    for c in (16, 32, 64, 128):
        out, tp, st = outs[c]
        first = T
        for kq, ku in (("in_q", "in_u"), ("out_q", "out_u")):
            for t in range(T):
                if (tp[kq][0, t] != ref_tp[kq][0, t]).any():
                    n, ok = PY.flips_at_ties(ref_tp[ku][0, t], ref_tp[kq][0, t], tp[kq][0, t])
                    assert ok, f"chunk {c}: {kq} flip away from a rounding tie at token {t}"
                    first = min(first, t)
                    break
        e = max((PY.err(out[0, t], ref_out[0, t]) for t in range(first)), default=0.0)
        say(f"chunk {c}: max normwise difference {e:.2e} over {first} tokens (first code flip: {first < T})")
        assert e < PY.TOL_LAYER, (c, e)
        if first == T:
            assert PY.err(st[1], ref_st[1]) < PY.TOL_LAYER


def run_stack_prefill(dims, layers, xs, states0, chunk, final_w, bf16=False, taps=True):
    """dfssm_stack_prefill over xs [B][T][D]; returns (y, taps numpy per layer [L][B][T][...] as a
    function of the layer, final states, the device taps object)."""
    L, Dv = _lib()
    B, T = xs.shape[:2]
    nL = len(layers)
    devs = [Dv.DeviceLayer(lw) for lw in layers]
    sts = [Dv.DeviceState(c, s_) for c, s_ in states0]
    x = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
    if bf16:
        x = x.to(torch.bfloat16)
    fw = torch.from_numpy(final_w).cuda()
    y = torch.empty((B, T, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_PREFILL, B, T, nL)
    tp = Dv.Taps(dims, nL * B * T) if taps else None
    Dv.stack_prefill(dims, devs, sts, fw, x, y, chunk, ws, tp)
    torch.cuda.synchronize()

    def layer_taps(l):
        return {k: v[l * B * T:(l + 1) * B * T].cpu().numpy().reshape(B, T, -1) for k, v in tp.t.items()}

    return (y.cpu().numpy(), layer_taps if taps else None,
            [(s_.conv.cpu().numpy(), s_.ssm.cpu().numpy()) for s_ in sts], devs, sts)


def test_stack_prefill_tiny_per_layer_and_composition():
    """A 3-layer stack prefill (batch 2, 300 tokens, chunk 64, nonzero states, random final norm
    weight): every layer checked from its own GPU input (P1 + P2 per token, final states), the
    output against the oracle's final RMSNorm, and the whole against three dfssm_layer_prefill calls
    and the library's final norm (the same kernels: bit-identical)."""
    nL, B, T, Q = 3, 2, 300, 64
    layers = gen.stack_weights(TINY, nL, seed=16, random_norms=True, per_channel_lora=True)
    states0 = [gen.initial_states(TINY, B, l, 16, std=0.2) for l in range(nL)]
    xs = gen.token_inputs(TINY, (B, T), 16, tag=7)
    fw = np.random.default_rng(16).uniform(0.5, 1.5, TINY.d_model).astype(np.float32)
    say(f"case: tiny stack prefill, {nL} layers, batch {B}, seqlen {T}, chunk {Q}")
    y, lt, finals, _, _ = run_stack_prefill(TINY, layers, xs, states0, Q, fw)
    for l in range(nL):
        tl = lt(l)
        dense = O.dense_signs(layers[l])
        for b in range(B):
            tb = {k: v[b] for k, v in tl.items()}
            out = lt(l + 1)["h_in"][b] if l + 1 < nL else y[b]
            errs = check_sequence(layers[l], tb["h_in"], states0[l][0][b], states0[l][1][b], out, tb,
                                  (finals[l][0][b], finals[l][1][b]), dense, what=f"layer {l} row {b}",
                                  final_w=None if l + 1 < nL else fw)
            say(f"layer {l} row {b}: {errs}")
    # composition of single-layer prefills gives the same bits
    say("case: same stack as three dfssm_layer_prefill calls")
    h = xs
    st = [list(s_) for s_ in states0]
    for l in range(nL):
        h, _, fin = run_prefill(TINY, layers[l], h, st[l][0], st[l][1], Q, taps=False)
        assert (fin[0] == finals[l][0]).all() and (fin[1] == finals[l][1]).all(), l
    assert (O.rmsnorm(h, fw, TINY.eps) - y).__abs__().max() < 1e-5


def test_stack_prefill_1p3b_48_layers_2048_then_decode():
    """The prefill workload (48 layers, 2048 bf16 tokens, chunk 256, zero states) with its final
    states handed to 16 stack-decode steps fed the last position's output. Sampled layers are
    checked over every token from their own GPU input (codes and integer sums exact, floats and the
    final states against the oracle's sequential recurrence); the 16 decode steps are checked
    through all 48 layers with the GPU's codes forced into the oracle, which starts from the
    handed-off states and keeps its own float trajectory (P3)."""
    L, Dv = _lib()
    nL, T, Q, T2 = 48, 2048, 256, 16
    layers = gen.stack_weights(BIG, nL, seed=0)
    states0 = [gen.initial_states(BIG, 1, l) for l in range(nL)]
    xs = gen.token_inputs(BIG, (1, T), 0, tag=11, bf16=True)
    fw = np.ones(BIG.d_model, np.float32)
    say(f"case: 1.3B stack prefill, {nL} layers, seqlen {T}, chunk {Q}, bf16 input, with taps")
    y, lt, finals, devs, sts = run_stack_prefill(BIG, layers, xs, states0, Q, fw, bf16=True)
    assert np.isfinite(y).all()
    for l in (0, 1, 24, 47):
        tl = {k: v[0] for k, v in lt(l).items()}
        out = lt(l + 1)["h_in"][0] if l + 1 < nL else y[0]
        if l == 0:
            assert (tl["h_in"] == xs[0]).all()
        errs = check_sequence(layers[l], tl["h_in"], states0[l][0][0], states0[l][1][0], out, tl,
                              (finals[l][0][0], finals[l][1][0]), O.dense_signs(layers[l]), what=f"layer {l}",
                              final_w=None if l + 1 < nL else fw)
        say(f"prefill layer {l}: {errs}")
    # hand-off: decode 16 tokens from the prefill's final states, x0 = the last position's output
    say(f"case: {T2} stack-decode steps from the handed-off states")
    x0 = torch.from_numpy(np.ascontiguousarray(y[:, -1])).cuda()
    yd = torch.empty((T2, 1, BIG.d_model), dtype=torch.float32, device="cuda")
    wsd = Dv.workspace(BIG, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)
    tpd = Dv.Taps(BIG, T2 * nL)
    Dv.stack_decode(BIG, devs, sts, torch.from_numpy(fw).cuda(), x0, yd, T2, wsd, tpd)
    torch.cuda.synchronize()
    assert Dv.stack_status(wsd) == L.DFSSM_STATUS_OK
    yd = yd.cpu().numpy()
    taps = tpd.numpy()
    dense_all = [O.dense_signs(lw) for lw in layers]
    cs = [f[0][0].astype(np.float64) for f in finals]
    ss = [f[1][0].astype(np.float64) for f in finals]
    x = y[0, -1].astype(np.float64)
    errs = []
    for t in range(T2):
        h = x
        for l in range(nL):
            tap = PY.tap_record(taps, t * nL + l)
            PY.assert_codes_exact(tap["in_u"], tap["in_q"], tap["in_s"][0], f"decode t{t} l{l} in")
            PY.assert_codes_exact(tap["out_u"], tap["out_q"], tap["out_s"][0], f"decode t{t} l{l} out")
            PY.assert_products_exact(layers[l].in_proj, tap["in_q"], tap["in_acc"], tap["in_t"], dense_all[l]["in"])
            PY.assert_products_exact(layers[l].out_proj, tap["out_q"], tap["out_acc"], tap["out_t"],
                                     dense_all[l]["out"])
            force = dict(in_q=tap["in_q"], in_s=tap["in_s"][0], out_q=tap["out_q"], out_s=tap["out_s"][0])
            h, cs[l], ss[l], _ = O.layer_decode(h, layers[l], cs[l], ss[l], force=force, dense=dense_all[l])
        yo = O.rmsnorm(h, fw, BIG.eps)
        errs.append(PY.err(yd[t][0], yo))
        x = yo
    say(f"hand-off decode, code-forced through 48 layers: max err {max(errs):.2e}")
    assert max(errs) < PY.TOL_STACK
    for l in range(nL):
        assert PY.err(sts[l].conv.cpu().numpy()[0], cs[l]) < PY.TOL_STACK, l
        assert PY.err(sts[l].ssm.cpu().numpy()[0], ss[l]) < PY.TOL_STACK, l
