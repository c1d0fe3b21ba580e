"""GPU parity of batched decode (more than 4 tokens per step: the projections run as int8 MFMA
GEMMs) against the CPU oracle, for single layers and for the layer stack."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say, run_layer, run_stack, forced_chain

pytestmark = pytest.mark.gpu

TINY = gen.DIMS["tiny"]
BIG = gen.DIMS["1p3b"]


def p1_all_rows(lw, tps, dense=None):
    for t, tp in enumerate(tps):
        for b in range(tp["in_q"].shape[0]):
            r = PY.tap_record(tp, b)
            PY.assert_codes_exact(r["in_u"], r["in_q"], r["in_s"][0], f"t={t} b={b} in")
            PY.assert_codes_exact(r["out_u"], r["out_q"], r["out_s"][0], f"t={t} b={b} out")
        q = tp["in_q"]
        _, acc, tt = O.project_tokens(q, np.ones(q.shape[0], np.float32), lw.in_proj,
                                      None if dense is None else dense["in"])
        assert (tp["in_acc"].astype(np.int64)[:, :acc.shape[1]] == acc).all() and (tp["in_t"] == tt).all(), t
        q = tp["out_q"]
        _, acc, tt = O.project_tokens(q, np.ones(q.shape[0], np.float32), lw.out_proj,
                                      None if dense is None else dense["out"])
        assert (tp["out_acc"].astype(np.int64) == acc).all() and (tp["out_t"] == tt).all(), t


def test_layer_decode_tiny_batch64_mfma():
    B, T = 64, 4
    lw = gen.layer_weights(TINY, 10, 20, random_norms=True, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(TINY, B, 10, 20, std=0.3)
    xs = gen.token_inputs(TINY, (T, B), 20, tag=1)
    say(f"case: tiny layer decode, batch {B}, {T} steps (MFMA projections)")
    outs, tps, final, _ = run_layer(TINY, lw, xs, conv0, ssm0)
    dense = O.dense_signs(lw)
    p1_all_rows(lw, tps, dense)
    for b in (0, 5, 31, 63):
        worst, ec, es = forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)
        say(f"row {b}: forced max err {worst:.2e} conv {ec:.2e} ssm {es:.2e}")


@pytest.mark.parametrize("B", [5, 17, 33, 50, 130])
def test_layer_decode_tiny_ragged_batches_mfma(B):
    """Batches that leave a ragged 32-row block of the skinny GEMM (5, 17: one block; 33, 50: a
    partial second block) or a ragged 128-row tile of the tile GEMM (130)."""
    lw = gen.layer_weights(TINY, 11, 21)
    conv0, ssm0 = gen.initial_states(TINY, B, 11, 21, std=0.2)
    xs = gen.token_inputs(TINY, (2, B), 21, tag=2)
    say(f"case: tiny layer decode, batch {B}, 2 steps (MFMA projections)")
    outs, tps, final, _ = run_layer(TINY, lw, xs, conv0, ssm0)
    dense = O.dense_signs(lw)
    p1_all_rows(lw, tps, dense)
    for b in sorted({0, B // 2, B - 1}):
        forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)


# a tiny layer whose in_proj has 8200 rows (8 past a multiple of 64, 257 blocks of 32): the skinny
# GEMM takes two column blocks per workgroup and its last workgroup holds a partial first block
WIDE = gen.Dims(d_model=256, d_inner=512, d_state=16, headdim=64, ngroups=1, d_conv=4,
                n_in_proj=8200, rank_in=8, rank_out=8)


@pytest.mark.parametrize("B", [7, 64])
def test_layer_decode_wide_in_proj_two_column_blocks(B):
    lw = gen.layer_weights(WIDE, 13, 23)
    conv0, ssm0 = gen.initial_states(WIDE, B, 13, 23, std=0.2)
    xs = gen.token_inputs(WIDE, (2, B), 23, tag=3)
    say(f"case: tiny layer with 8200 in_proj rows, batch {B}, 2 steps (MFMA projections)")
    outs, tps, final, _ = run_layer(WIDE, lw, xs, conv0, ssm0)
    dense = O.dense_signs(lw)
    p1_all_rows(lw, tps, dense)
    for b in sorted({0, B - 1}):
        forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)


def test_layer_decode_mfma_and_gemv_paths_agree():
    """The same 4 tokens through the packed-sign GEMV (batch 4) and through the MFMA GEMM (the
    same rows twice, batch 8): codes equal except at rounding ties, outputs within 1e-3."""
    lw = gen.layer_weights(TINY, 12, 22, random_norms=True)
    conv0, ssm0 = gen.initial_states(TINY, 4, 12, 22, std=0.3)
    xs = gen.token_inputs(TINY, (3, 4), 22, tag=3)
    say("case: tiny layer decode batch 4 (GEMV) vs batch 8 (MFMA)")
    o4, t4, f4, _ = run_layer(TINY, lw, xs, conv0, ssm0)
    o8, t8, f8, _ = run_layer(TINY, lw, np.concatenate([xs, xs], 1), np.concatenate([conv0, conv0]),
                              np.concatenate([ssm0, ssm0]))
    for t in range(3):
        for b in range(4):
            for half in (0, 4):
                f, ok = PY.flips_at_ties(t4[t]["in_u"][b], t4[t]["in_q"][b], t8[t]["in_q"][b + half])
                assert ok, (t, b)
                assert PY.err(o8[t][b + half], o4[t][b]) < PY.TOL_LAYER
            # rows that saw the same inputs in the same launch are bit-identical
            assert (o8[t][b] == o8[t][b + 4]).all()
    assert PY.err(f8[1][:4], f4[1]) < PY.TOL_LAYER


def test_layer_decode_1p3b_batch64():
    B, T = 64, 2
    lw = gen.layer_weights(BIG, 0, 0)
    conv0, ssm0 = gen.initial_states(BIG, B, 0, 0, std=0.1)
    xs = gen.token_inputs(BIG, (T, B), 0, tag=4)
    say(f"case: 1.3B-shaped layer decode, batch {B}, {T} steps (MFMA projections)")
    outs, tps, final, _ = run_layer(BIG, lw, xs, conv0, ssm0)
    dense = O.dense_signs(lw)
    p1_all_rows(lw, tps, dense)
    for b in (0, 37, 63):
        worst, ec, es = forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)
        say(f"1p3b batch-64 row {b}: forced max err {worst:.2e} conv {ec:.2e} ssm {es:.2e}")


def test_stack_decode_tiny_batch64_forced():
    nL, T, B = 3, 3, 64
    layers = gen.stack_weights(TINY, nL, seed=6, random_norms=True, per_channel_lora=True)
    states0 = [gen.initial_states(TINY, B, l, 6, std=0.1) for l in range(nL)]
    x0 = gen.token_inputs(TINY, (B,), 6, tag=5)
    fw = np.random.default_rng(6).uniform(0.5, 1.5, TINY.d_model).astype(np.float32)
    say(f"case: tiny stack decode, {nL} layers, {T} steps, batch {B}, with taps")
    y, states, taps = run_stack(TINY, layers, x0, states0, T, taps=True, final_w=fw)
    dense = [O.dense_signs(lw) for lw in layers]
    for b in (0, 29, 63):
        cs = [s[0][b].astype(np.float64) for s in states0]
        ss = [s[1][b].astype(np.float64) for s in states0]
        for t in range(T):
            for l in range(nL):
                tap = PY.tap_record(taps, (t * nL + l) * B + b)
                if l == 0:
                    assert (tap["h_in"] == (x0[b] if t == 0 else y[t - 1][b])).all()
                PY.assert_codes_exact(tap["in_u"], tap["in_q"], tap["in_s"][0], f"t{t} l{l} b{b}")
                PY.assert_codes_exact(tap["out_u"], tap["out_q"], tap["out_s"][0], f"t{t} l{l} b{b}")
                PY.assert_products_exact(layers[l].in_proj, tap["in_q"], tap["in_acc"], tap["in_t"], dense[l]["in"])
                PY.assert_products_exact(layers[l].out_proj, tap["out_q"], tap["out_acc"], tap["out_t"],
                                         dense[l]["out"])
                force = dict(in_q=tap["in_q"], in_s=tap["in_s"][0], out_q=tap["out_q"], out_s=tap["out_s"][0])
                h, cs[l], ss[l], _ = O.layer_decode(tap["h_in"], layers[l], cs[l], ss[l], force=force,
                                                    dense=dense[l])
                if l + 1 < nL:
                    assert PY.err(PY.tap_record(taps, (t * nL + l + 1) * B + b)["h_in"], h) < PY.TOL_LAYER
                else:
                    assert PY.err(y[t][b], O.rmsnorm(h, fw, TINY.eps)) < PY.TOL_LAYER
        for l in range(nL):
            assert PY.err(states[l][0][b], cs[l]) < PY.TOL_LAYER
            assert PY.err(states[l][1][b], ss[l]) < PY.TOL_LAYER


def test_stack_decode_1p3b_48_layers_batch64_sampled():
    """The batch-64 decode workload (48 layers, 128 steps): deterministic across a split run, and
    the last step checked layer by layer, from the GPU's own state and input, on sampled rows."""
    nL, T, B = 48, 128, 64
    layers = gen.stack_weights(BIG, nL, seed=0)
    states0 = [gen.initial_states(BIG, B, l, 0, std=0.1) for l in range(nL)]
    x0 = gen.token_inputs(BIG, (B,), 0, tag=8)
    say(f"case: 1.3B stack decode, {nL} layers, {T} steps, batch {B}")
    y_full, _, _ = run_stack(BIG, layers, x0, states0, T)
    assert np.isfinite(y_full).all()
    say(f"case: same stack, {T - 1} steps then 1 tapped step")
    y_a, st_a, _ = run_stack(BIG, layers, x0, states0, T - 1)
    assert (y_full[:T - 1] == y_a).all(), "the decode is not deterministic across runs"
    y_b, st_b, taps = run_stack(BIG, layers, y_a[-1], st_a, 1, taps=True)
    assert (y_full[T - 1] == y_b[0]).all()
    worst = {}
    for l in range(nL):
        lw = layers[l]
        dense = O.dense_signs(lw)
        for b in (0, 63):
            tap = PY.tap_record(taps, l * B + b)
            out_gpu = PY.tap_record(taps, (l + 1) * B + b)["h_in"] if l + 1 < nL else None
            force = dict(in_q=tap["in_q"], in_s=tap["in_s"][0], out_q=tap["out_q"], out_s=tap["out_s"][0])
            PY.assert_codes_exact(tap["in_u"], tap["in_q"], tap["in_s"][0], f"layer {l} row {b} in")
            PY.assert_codes_exact(tap["out_u"], tap["out_q"], tap["out_s"][0], f"layer {l} row {b} out")
            PY.assert_products_exact(lw.in_proj, tap["in_q"], tap["in_acc"], tap["in_t"], dense["in"])
            PY.assert_products_exact(lw.out_proj, tap["out_q"], tap["out_acc"], tap["out_t"], dense["out"])
            h, cs, ss, _ = O.layer_decode(tap["h_in"], lw, st_a[l][0][b], st_a[l][1][b], force=force, dense=dense)
            errs = dict(conv=PY.err(st_b[l][0][b], cs), ssm=PY.err(st_b[l][1][b], ss))
            if out_gpu is not None:
                errs["out"] = PY.err(out_gpu, h)
            else:
                errs["out"] = PY.err(y_b[0][b], O.rmsnorm(h, np.ones(BIG.d_model), BIG.eps))
            for k, v in errs.items():
                assert v < PY.TOL_LAYER, (l, b, errs)
                worst[k] = max(worst.get(k, 0.0), v)
    say(f"1p3b batch-64 stack last step per-layer worst errors: {worst}")


def test_stack_decode_halves_match_single_stream():
    """From 32 sequences up a stack decode runs as two batch halves on two streams. At batch 41
    (halves of 20 and 21) the outputs, final states and every tap record equal, bit for bit, those of
    two separate decodes of the same 20 and 21 sequences, which run below the threshold on one stream."""
    nL, T, B, b0 = 3, 3, 41, 20
    layers = gen.stack_weights(TINY, nL, seed=7, random_norms=True, per_channel_lora=True)
    states0 = [gen.initial_states(TINY, B, l, 7, std=0.1) for l in range(nL)]
    x0 = gen.token_inputs(TINY, (B,), 7, tag=6)
    fw = np.random.default_rng(7).uniform(0.5, 1.5, TINY.d_model).astype(np.float32)
    say(f"case: tiny stack decode, {nL} layers, {T} steps, batch {B} (two halves) against {b0} + {B - b0}")
    y, states, taps = run_stack(TINY, layers, x0, states0, T, taps=True, final_w=fw)
    for lo, hi in ((0, b0), (b0, B)):
        part = [(c[lo:hi].copy(), s[lo:hi].copy()) for c, s in states0]
        yp, sp, tp = run_stack(TINY, layers, x0[lo:hi].copy(), part, T, taps=True, final_w=fw)
        assert (y[:, lo:hi] == yp).all(), (lo, hi)
        for l in range(nL):
            assert (states[l][0][lo:hi] == sp[l][0]).all() and (states[l][1][lo:hi] == sp[l][1]).all(), (lo, l)
        n = hi - lo
        for t in range(T):
            for l in range(nL):
                for k, v in taps.items():
                    full = v[(t * nL + l) * B + lo:(t * nL + l) * B + hi]
                    assert (full == tp[k][(t * nL + l) * n:(t * nL + l + 1) * n]).all(), (k, t, l, lo)
