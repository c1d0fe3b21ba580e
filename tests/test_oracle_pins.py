"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something the paper prints (fixtures under tests/golden/),
a closed form, an invariant, a library routine or a brute-force evaluation by a different route,
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, index or bit order,
a transposed operand) fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dfssm_oracle as O
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_dims(**kw):
    base = dict(d_model=64, d_inner=128, d_state=8, headdim=32, ngroups=1, d_conv=4,
                n_in_proj=2 * 128 + 2 * 8 + 4, rank_in=4, rank_out=4)
    base.update(kw)
    return gen.Dims(**base)


# ------------------------------------------------------------------ packing
def test_unpack_matches_pure_python_bit_extraction():
    rng = np.random.default_rng(1)
    packed = rng.integers(0, 256, size=(5, 4), dtype=np.uint8)
    dense = O.unpack_signs(packed, 32)
    for n in range(5):
        for k in range(32):
            bit = (int(packed[n, k // 8]) >> (k % 8)) & 1
            assert dense[n, k] == (1 if bit else -1)


def test_packing_is_64bit_little_endian_words():
    fx = _golden("avx512_packing.json")
    K = fx["row_elements"]
    assert K // fx["weights_per_load"] == fx["instructions_per_row"]
    rng = np.random.default_rng(2)
    words = rng.integers(0, 2**63, size=K // 64, dtype=np.uint64)
    row = words.astype("<u8").view(np.uint8)[None, :]          # bytes of LE 64-bit words
    assert row.shape[1] == (K // fx["weights_per_load"]) * fx["bytes_per_load"]
    dense = O.unpack_signs(row, K)[0]
    for k in range(0, K, 37):
        bit = (int(words[k // 64]) >> (k % 64)) & 1
        assert dense[k] == (1 if bit else -1)


# ------------------------------------------------------------------ Table 1 byte model
def test_table1_scaffold_and_lora_sizes():
    fx = _golden("table1_model_size.json")
    sh = _golden("model_shape_facts.json")
    d = gen.DIMS["1p3b"]
    assert d.d_model == sh["d_model"] and d.d_state == sh["d_state"]
    b = O.table1_bytes(d.d_model, d.d_inner, d.n_in_proj, fx["n_layers"], fx["lora_rank"])
    # 1 bit per scaffold weight reproduces the printed 155 MB
    assert round(b["scaffold"] / 1e6) == fx["scaffold_MB"]
    # the printed LoRA size is given to the MB
    assert abs(b["lora"] / 1e6 - fx["lora_MB"]) < 1.0
    # a 2-bit scaffold or a missing in_proj block does not
    assert round(2 * b["scaffold"] / 1e6) != fx["scaffold_MB"]
    b2 = O.table1_bytes(d.d_model, d.d_inner, 2 * d.d_inner, fx["n_layers"], fx["lora_rank"])
    assert round(b2["scaffold"] / 1e6) != fx["scaffold_MB"]
    # the fixed state: d_inner * d_state = 524,288 values ("524 KB")
    assert round(d.nheads * d.headdim * d.d_state / 1000) == sh["ssm_state_KB"]
    assert fx["scaffold_MB"] + fx["embedding_MB"] + fx["lora_MB"] + fx["other_MB"] == fx["total_MB"]


# ------------------------------------------------------------------ quantizer
def test_quantizer_ties_round_to_even_and_amax_maps_to_127():
    u = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, -126.5], np.float32)
    q, s = O.quantize_token(u)          # a = 127 -> inv = 1 exactly
    assert q.tolist() == [127, 0, 2, 2, 0, -2, 4, -126]
    assert s == np.float32(1.0)
    # Python's round() is also half-to-even: same codes by a different routine
    assert q.tolist() == [round(float(v)) for v in u]


def test_quantizer_zero_symmetry_and_error_bound():
    q, s = O.quantize_token(np.zeros(16, np.float32))
    assert not q.any() and s == 0
    rng = np.random.default_rng(3)
    for _ in range(20):
        u = (rng.standard_normal(257) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        q, s = O.quantize_token(u)
        qn, sn = O.quantize_token(-u)
        assert (qn == -q).all() and sn == s
        i = np.argmax(np.abs(u))
        assert abs(int(q[i])) == 127 and np.sign(q[i]) == np.sign(u[i])
        assert np.abs(q.astype(int)).max() <= 127
        # dequantized values are within half a step of the input
        err = np.abs(u.astype(np.float64) - float(s) * q.astype(np.float64))
        assert err.max() <= float(s) * (0.5 + 1e-4)


# ------------------------------------------------------------------ projection
def _proj(n_out, n_in, rank, seed, per_channel=True):
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 256, size=(n_out, n_in // 8), dtype=np.uint8)
    return gen.ProjWeights(
        sign=sign,
        row_scale=rng.uniform(0.01, 0.05, n_out).astype(np.float16),
        lora_dn=rng.integers(-127, 128, size=(rank, n_in)).astype(np.int8),
        dn_scale=(rng.uniform(0.5, 1.5, rank) * 1e-3).astype(np.float32) if per_channel else np.full(rank, 1e-3, np.float32),
        lora_up=rng.integers(-127, 128, size=(n_out, rank)).astype(np.int8),
        up_scale=(rng.uniform(0.5, 1.5, n_out) * 1e-3).astype(np.float32) if per_channel else np.full(n_out, 1e-3, np.float32),
    )


def test_project_brute_force_exact():
    P = _proj(6, 16, 3, seed=4)
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, 16).astype(np.int8)
    s = np.float32(0.0371)
    y, acc, t = O.project(q, s, P)
    for n in range(6):
        a = 0
        for k in range(16):
            bit = (int(P.sign[n, k // 8]) >> (k % 8)) & 1
            a += int(q[k]) if bit else -int(q[k])
        assert acc[n] == a
    tt = [sum(int(P.lora_dn[j, k]) * int(q[k]) for k in range(16)) for j in range(3)]
    assert t.tolist() == tt
    S = Fraction(float(s))
    for n in range(6):
        exact = S * Fraction(float(P.row_scale[n])) * acc[n]
        for j in range(3):
            exact += (Fraction(float(P.up_scale[n])) * int(P.lora_up[n, j])
                      * Fraction(float(P.dn_scale[j])) * S * tt[j])
        assert abs(float(exact) - y[n]) <= 1e-12 * max(1.0, abs(float(exact)))


def test_project_equals_dense_effective_matrix():
    # Eq. (3) as one dense matrix: W = diag(sc) sgn + diag(us) L_up diag(ds) L_dn, applied to s*q
    P = _proj(40, 64, 5, seed=6)
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, 64).astype(np.int8)
    s = np.float32(0.021)
    y, _, _ = O.project(q, s, P)
    bits = np.array([[(int(P.sign[n, k // 8]) >> (k % 8)) & 1 for k in range(64)] for n in range(40)])
    W = (P.row_scale.astype(np.float64)[:, None] * (2.0 * bits - 1.0)
         + (P.up_scale.astype(np.float64)[:, None] * P.lora_up.astype(np.float64))
         @ (P.dn_scale.astype(np.float64)[:, None] * P.lora_dn.astype(np.float64)))
    np.testing.assert_allclose(y, W @ (float(s) * q.astype(np.float64)), rtol=1e-12, atol=1e-12)


def test_project_complement_parity_and_bounds():
    P = _proj(8, 64, 2, seed=8)
    rng = np.random.default_rng(9)
    q = rng.integers(-127, 128, 64).astype(np.int8)
    _, acc, _ = O.project(q, np.float32(1), P)
    Pc = gen.ProjWeights(~P.sign, P.row_scale, P.lora_dn, P.dn_scale, P.lora_up, P.up_scale)
    _, accc, _ = O.project(q, np.float32(1), Pc)
    assert (accc == -acc).all()
    assert ((acc - int(q.astype(int).sum())) % 2 == 0).all()
    assert np.abs(acc).max() <= 64 * 127
    ones = gen.ProjWeights(np.full_like(P.sign, 255), P.row_scale, P.lora_dn, P.dn_scale, P.lora_up, P.up_scale)
    _, acc1, _ = O.project(q, np.float32(1), ones)
    assert (acc1 == int(q.astype(int).sum())).all()


# ------------------------------------------------------------------ conv
def test_conv_matches_numpy_convolve_and_first_step():
    rng = np.random.default_rng(10)
    C, T = 7, 12
    w = rng.uniform(-0.5, 0.5, (C, 4))
    b = rng.uniform(-0.5, 0.5, C)
    xs = rng.standard_normal((T, C))
    st = np.zeros((C, 3))
    outs = []
    for t in range(T):
        o, st = O.conv_step(st, xs[t], w, b)
        outs.append(o)
    outs = np.array(outs)
    for c in range(C):
        v = np.convolve(xs[:, c], w[c, ::-1])[:T] + b[c]
        np.testing.assert_allclose(outs[:, c], v / (1 + np.exp(-v)), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(st, xs[-3:].T)
    o0, _ = O.conv_step(np.zeros((C, 3)), xs[0], w, b)
    v0 = w[:, 3] * xs[0] + b
    np.testing.assert_allclose(o0, v0 / (1 + np.exp(-v0)), rtol=1e-14)


# ------------------------------------------------------------------ ssm
def _ssm_inputs(H=4, P=3, N=5, G=1, seed=11):
    rng = np.random.default_rng(seed)
    return dict(S=rng.standard_normal((H, P, N)) * 0.3, x=rng.standard_normal(H * P),
                Bm=rng.standard_normal((G, N)), Cm=rng.standard_normal((G, N)),
                dt=rng.uniform(1e-3, 0.1, H), A=-rng.uniform(1, 16, H), D=rng.standard_normal(H))


def test_ssm_closed_forms():
    d = _ssm_inputs()
    H, P, N = d["S"].shape
    # B = 0 from zero state: y = D x, state stays exactly zero
    y, S = O.ssm_step(np.zeros_like(d["S"]), d["x"], np.zeros_like(d["Bm"]), d["Cm"], d["dt"], d["A"], d["D"], 1)
    assert not S.any()
    np.testing.assert_array_equal(y, np.repeat(d["D"], P) * d["x"])
    # dt = 0: the state is unchanged bit for bit, y = C.S + D x
    y, S = O.ssm_step(d["S"], d["x"], d["Bm"], d["Cm"], np.zeros(H), d["A"], d["D"], 1)
    np.testing.assert_array_equal(S, d["S"])
    # one step from zero: y = dt (C.B) x + D x   (x is scaled by dt: App. B Table 12, row 1)
    y, S = O.ssm_step(np.zeros_like(d["S"]), d["x"], d["Bm"], d["Cm"], d["dt"], d["A"], d["D"], 1)
    cb = float(d["Cm"][0] @ d["Bm"][0])
    np.testing.assert_allclose(y, np.repeat(d["dt"], P) * cb * d["x"] + np.repeat(d["D"], P) * d["x"], rtol=1e-12)
    # A -> -inf: memoryless, the old state is forgotten
    y1, _ = O.ssm_step(d["S"], d["x"], d["Bm"], d["Cm"], d["dt"], np.full(H, -1e300), d["D"], 1)
    y2, _ = O.ssm_step(np.zeros_like(d["S"]), d["x"], d["Bm"], d["Cm"], d["dt"], np.full(H, -1e300), d["D"], 1)
    np.testing.assert_allclose(y1, y2, rtol=1e-12)


def test_ssm_group_mapping():
    d = _ssm_inputs(H=4, G=2)
    Bm = d["Bm"].copy()
    Bm[1] = 0.0                                   # heads 2 and 3 read group 1
    y, S = O.ssm_step(np.zeros_like(d["S"]), d["x"], Bm, d["Cm"], d["dt"], d["A"], d["D"], 2)
    P = d["S"].shape[1]
    assert not S[2:].any() and S[:2].any()
    np.testing.assert_array_equal(y[2 * P:], np.repeat(d["D"][2:], P) * d["x"][2 * P:])


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_chunked_equals_sequential(G):
    rng = np.random.default_rng(12)
    T, H, P, N = 100, 4, 3, 6
    xs = rng.standard_normal((T, H, P))
    dts = rng.uniform(1e-3, 0.2, (T, H))
    A = -rng.uniform(1, 16, H)
    Bs, Cs = rng.standard_normal((T, G, N)), rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    S0 = rng.standard_normal((H, P, N)) * 0.5
    ys, ST = O.ssm_scan_sequential(xs, dts, A, Bs, Cs, D, S0, G)
    for Q in (1, 3, 16, 64, 100, 256):
        yc, SC = O.ssd_chunked(xs, dts, A, Bs, Cs, D, S0, G, Q)
        np.testing.assert_allclose(yc, ys, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(SC, ST, rtol=1e-10, atol=1e-12)


def test_ssd_quadratic_form_equals_sequential():
    rng = np.random.default_rng(13)
    T, H, P, N, G = 40, 2, 3, 4, 1
    xs = rng.standard_normal((T, H, P))
    dts = rng.uniform(1e-3, 0.3, (T, H))
    A = -rng.uniform(1, 16, H)
    Bs, Cs = rng.standard_normal((T, G, N)), rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    ys, _ = O.ssm_scan_sequential(xs, dts, A, Bs, Cs, D, np.zeros((H, P, N)), G)
    yq = O.ssd_quadratic(xs, dts, A, Bs, Cs, D, G)
    np.testing.assert_allclose(yq, ys, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ norms
def test_gated_norm_order_and_rmsnorm_closed_form():
    rng = np.random.default_rng(14)
    y = rng.standard_normal(64)
    w = rng.uniform(0.5, 1.5, 64)
    z0 = 3.0
    c = z0 / (1 + np.exp(-z0))
    out, _ = O.gated_rmsnorm(y, np.full(64, z0), w, 1e-5)
    # gate first: a constant gate c only rescales eps, norm(c y) = norm_{eps/c^2}(y)
    np.testing.assert_allclose(out, O.rmsnorm(y, w, 1e-5 / c ** 2), rtol=1e-13)
    assert not np.allclose(out, c * O.rmsnorm(y, w, 1e-5), rtol=1e-3)
    h = np.full(32, 0.7)
    np.testing.assert_allclose(O.rmsnorm(h, np.ones(32), 1e-5), 0.7 / np.sqrt(0.49 + 1e-5), rtol=1e-14)


# ------------------------------------------------------------------ layer
def _zero_z_rows(W):
    E = W.dims.d_inner
    W.in_proj.row_scale[:E] = 0
    W.in_proj.up_scale[:E] = 0
    return W


def test_layer_zero_gate_is_identity():
    dm = _tiny_dims()
    W = _zero_z_rows(gen.layer_weights(dm, 0, 21, random_norms=True, per_channel_lora=True))
    cs, ss = gen.initial_states(dm, 1, 0, 21, std=0.3)
    h = gen.token_inputs(dm, (1,), 21)[0]
    h_out, _, ss2, tp = O.layer_decode(h, W, cs[0], ss[0])
    assert not tp.out_q.any() and tp.out_s == 0
    np.testing.assert_array_equal(h_out, h.astype(np.float64))


def test_layer_dt_to_zero_keeps_state():
    dm = _tiny_dims()
    W = gen.layer_weights(dm, 0, 22)
    W.dt_bias[:] = -100.0
    cs, ss = gen.initial_states(dm, 1, 0, 22, std=0.3)
    h = gen.token_inputs(dm, (1,), 22)[0]
    _, _, ss2, _ = O.layer_decode(h, W, cs[0], ss[0])
    np.testing.assert_array_equal(ss2, ss[0].astype(np.float64))


def test_layer_B_zero_gives_Dx_and_zero_state():
    dm = _tiny_dims()
    W = gen.layer_weights(dm, 0, 23)
    E, N = dm.d_inner, dm.d_state
    rows = slice(2 * E, 2 * E + N)             # B rows of in_proj: after z (E) and x (E)
    W.in_proj.row_scale[rows] = 0
    W.in_proj.up_scale[rows] = 0
    W.conv_b[E:E + N] = 0                       # conv channels of B
    cs, ss = gen.initial_states(dm, 1)
    h = gen.token_inputs(dm, (1,), 23)[0]
    _, _, ss2, _ = O.layer_decode(h, W, cs[0], ss[0])
    assert not ss2.any()


def test_layer_forced_codes_reproduce_free_run_and_state_handoff():
    dm = _tiny_dims()
    W = gen.layer_weights(dm, 0, 24, random_norms=True)
    cs, ss = gen.initial_states(dm, 1)
    xs = gen.token_inputs(dm, (9,), 24)
    o_all, cs_all, ss_all, taps = O.layer_decode_steps(xs, W, cs[0], ss[0])
    o_a, cs_a, ss_a, _ = O.layer_prefill(xs[:4], W, cs[0], ss[0])
    o_b, cs_b, ss_b, _ = O.layer_decode_steps(xs[4:], W, cs_a, ss_a)
    np.testing.assert_array_equal(np.concatenate([o_a, o_b]), o_all)
    np.testing.assert_array_equal(ss_b, ss_all)
    np.testing.assert_array_equal(cs_b, cs_all)
    # forcing the oracle's own codes changes nothing
    t0 = taps[0]
    o_f, _, _, _ = O.layer_decode(xs[0], W, cs[0], ss[0],
                                  force=dict(in_q=t0.in_q, in_s=t0.in_s, out_q=t0.out_q, out_s=t0.out_s))
    np.testing.assert_array_equal(o_f, o_all[0])


def test_stack_feedback_is_normalised():
    dm = _tiny_dims()
    layers = gen.stack_weights(dm, 2, seed=25)
    states = [gen.initial_states(dm, 1, l) for l in range(2)]
    x0 = gen.token_inputs(dm, (1,), 25)[0]
    ys, _, _ = O.stack_decode(x0, layers, [s[0][0] for s in states], [s[1][0] for s in states],
                              3, np.ones(dm.d_model), dm.eps)
    rms = np.sqrt(np.mean(ys ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-4)
    assert not np.allclose(ys[0], ys[1])


def test_project_tokens_equals_per_token_project():
    P = _proj(24, 64, 8, seed=30)
    rng = np.random.default_rng(31)
    q = rng.integers(-127, 128, size=(5, 64)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, 5).astype(np.float32)
    y, acc, t = O.project_tokens(q, s, P)
    for m in range(5):
        y1, a1, t1 = O.project(q[m], s[m], P)
        np.testing.assert_array_equal(acc[m], a1)
        np.testing.assert_array_equal(t[m], t1)
        np.testing.assert_allclose(y[m], y1, rtol=1e-13, atol=1e-13)


def test_layer_tokens_equals_sequential_decode():
    d = _tiny_dims()
    lw = gen.layer_weights(d, 2, 40, random_norms=True, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(d, 1, 2, 40, std=0.2)
    xs = gen.token_inputs(d, (9, 1), 40)[:, 0]
    o1, c1, s1, taps = O.layer_decode_steps(xs, lw, conv0[0], ssm0[0])
    o2, c2, s2, tp2 = O.layer_tokens(xs, lw, conv0[0], ssm0[0])
    for t in range(9):
        for k in ("in_q", "in_acc", "in_t", "out_q", "out_acc", "out_t"):
            np.testing.assert_array_equal(getattr(taps[t], k), tp2[k][t])
        assert taps[t].in_s == tp2["in_s"][t] and taps[t].out_s == tp2["out_s"][t]
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2, c1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-12)
    # forcing the codes it would choose anyway changes nothing
    f = dict(in_q=tp2["in_q"], in_s=tp2["in_s"], out_q=tp2["out_q"], out_s=tp2["out_s"])
    o3, _, _, _ = O.layer_tokens(xs, lw, conv0[0], ssm0[0], force=f)
    np.testing.assert_array_equal(o3, o2)


# ------------------------------------------------------------------ elementwise functions
def test_softplus_closed_forms_and_library():
    """softplus(v) = log(1 + e^v): ln 2 at 0, softplus(v) - softplus(-v) = v, numpy's logaddexp(0, v)
    (the same function by another route) everywhere, continuous across the v > 20 branch, e^v in
    the far-negative tail."""
    assert O.softplus(0.0) == pytest.approx(np.log(2.0), rel=1e-15)
    # above 20 the oracle returns v itself (the usual Mamba threshold): it drops log1p(e^-v) <= 2.1e-9
    v = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(O.softplus(v) - O.softplus(-v), v, rtol=0, atol=2.1e-9)
    inner = np.abs(v) <= 20.0
    np.testing.assert_allclose(O.softplus(v[inner]) - O.softplus(-v[inner]), v[inner], rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.softplus(v[inner]), np.logaddexp(0.0, v[inner]), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.softplus(v), np.logaddexp(0.0, v), rtol=1e-10, atol=0)
    lo, hi = O.softplus(np.nextafter(20.0, 0.0)), O.softplus(np.nextafter(20.0, 40.0))
    assert abs(float(hi) - float(lo)) < 1e-8
    np.testing.assert_allclose(O.softplus(np.array([-40.0, -60.0])), np.exp([-40.0, -60.0]), rtol=1e-12)
    assert (O.softplus(v) >= np.maximum(v, 0.0)).all()


def test_silu_closed_forms_and_library():
    """silu(v) = v * sigmoid(v): 0 at 0, silu(v) - silu(-v) = v, scipy's expit gives the sigmoid by
    another route, slope 1/2 at 0, -> v for large v and -> 0 for very negative v."""
    from scipy.special import expit
    assert O.silu(0.0) == 0.0
    v = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(O.silu(v) - O.silu(-v), v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)
    h = 1e-6
    assert (O.silu(h) - O.silu(-h)) / (2 * h) == pytest.approx(0.5, rel=1e-9)
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)
    assert O.silu(40.0) == pytest.approx(40.0, rel=1e-15) and abs(O.silu(-40.0)) < 1e-15


def test_stack_identity_layers_closed_form():
    """With every layer the identity (z rows zeroed, so the gate and the out-projection codes are 0),
    the stack's step t outputs RMSNorm applied t + 1 times with the final weight w: y[t] points along
    x0 * w^(t+1) and y[t] / w has mean square m / (m + eps), m the mean square of the step's input.
    Feeding back the un-normalised residual, or dropping w, breaks the direction or the scale."""
    dm = _tiny_dims()
    layers = [_zero_z_rows(gen.layer_weights(dm, l, 26, random_norms=True)) for l in range(2)]
    states = [gen.initial_states(dm, 1, l) for l in range(2)]
    x0 = gen.token_inputs(dm, (1,), 26)[0].astype(np.float64) * 3.0
    w = np.random.default_rng(26).uniform(0.5, 1.5, dm.d_model)
    T = 4
    ys, _, _ = O.stack_decode(x0, layers, [s[0][0] for s in states], [s[1][0] for s in states], T, w, dm.eps)
    x = x0
    for t in range(T):
        direction = x0 * w ** (t + 1)
        ratio = ys[t] / direction
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)          # parallel, same sign
        assert ratio[0] > 0
        m = sum(float(v) * float(v) for v in x) / x.size                  # mean square of the input
        got = sum(float(v) * float(v) for v in ys[t] / w) / x.size
        assert got == pytest.approx(m / (m + dm.eps), rel=1e-12)
        x = ys[t]


# ------------------------------------------------------------------ embedding + LM head
def test_embedding_size_matches_table1():
    fx = _golden("table1_model_size.json")
    d = gen.DIMS["1p3b"]
    b = O.table1_bytes(d.d_model, d.d_inner, d.n_in_proj, fx["n_layers"], fx["lora_rank"], vocab=gen.VOCAB_1P3B)
    # one byte per weight of the tied embedding/LM head reproduces the printed 103 MB
    assert round(b["embedding"] / 1e6) == fx["embedding_MB"]
    assert round(2 * b["embedding"] / 1e6) != fx["embedding_MB"]          # not fp16, not untied


def test_embed_rows_by_explicit_indexing():
    rng = np.random.default_rng(50)
    codes = rng.integers(-127, 128, size=(11, 6)).astype(np.int8)
    scale = rng.uniform(1e-4, 1e-3, 11).astype(np.float32)
    toks = np.array([3, 0, 10, 3], np.int32)
    x = O.embed(toks, codes, scale)
    for i, t in enumerate(toks):
        for k in range(6):
            assert x[i, k] == float(scale[t]) * int(codes[t, k])


def test_lm_head_brute_force_dense_and_argmax():
    rng = np.random.default_rng(51)
    V, D = 37, 24
    codes = rng.integers(-127, 128, size=(V, D)).astype(np.int8)
    scale = rng.uniform(1e-4, 1e-3, V).astype(np.float32)
    y = rng.standard_normal(D).astype(np.float32)
    logits, acc, q, s = O.lm_head(y, codes, scale, chunk_rows=5)
    qo, so = O.quantize_token(y)
    assert (q == qo).all() and s == so
    for v in range(V):
        assert acc[v] == sum(int(codes[v, k]) * int(q[k]) for k in range(D))
    # the same logits from the dequantised matrices by another route
    dense = (codes.astype(np.float64) * scale.astype(np.float64)[:, None]) @ (q.astype(np.float64) * float(s))
    np.testing.assert_allclose(logits, dense, rtol=1e-12, atol=1e-15)
    # a planted maximum wins; equal maxima resolve to the smallest index
    c2 = codes.copy()
    c2[17] = np.where(q >= 0, 127, -127)
    s2 = scale.copy()
    s2[17] = 2e-3
    l2, _, _, _ = O.lm_head(y, c2, s2)
    assert O.argmax_first(l2) == 17
    c2[30], s2[30] = c2[17], s2[17]
    l3, _, _, _ = O.lm_head(y, c2, s2)
    assert O.argmax_first(l3) == 17


# ------------------------------------------------------------------ density field state codec
def test_codec_field_sizes_from_appendix_d():
    # App. D: K = 23 (a 529-cell field) for d_state 128, and K^2 ~ 4 d_state in general
    assert O.codec_field_side(128) == 23 and O.codec_field_side(128) ** 2 == 529
    for n in (16, 32, 64, 128, 256):
        K = O.codec_field_side(n)
        assert abs(K * K - 4 * n) <= 2 * K + 1
        cells = O.codec_cells(n)
        assert cells[0] == 0 and cells[-1] == K * K and (np.diff(cells) >= 3).all()
        assert np.diff(cells).max() - np.diff(cells).min() <= 1          # cells spread evenly


def test_codec_constant_and_flat_rows():
    for n in (16, 128):
        # a constant row whose fp32 mean is exact: sigma = 0, read back exactly
        row = np.full(n, 0.375, np.float32)
        bits, mu, sigma = O.state_codec_encode_row(row)
        assert sigma == 0 and not bits.any()
        np.testing.assert_array_equal(O.state_codec_decode_row(bits, mu, sigma, n), np.float32(0.375))
        # any constant row reads back to within the rounding of its fp32 mean
        row = np.full(n, 0.37, np.float32)
        bits, mu, sigma = O.state_codec_encode_row(row)
        np.testing.assert_allclose(O.state_codec_decode_row(bits, mu, sigma, n), 0.37, rtol=2e-6)


def test_codec_sigma_delta_density_and_accumulator():
    """Every value's cell density is within one cell of its 8-bit target (the first-order error
    feedback carries the rest), the error accumulator fits 8 bits, and the density summed over the
    whole field is within one cell of the summed targets (no drift)."""
    rng = np.random.default_rng(60)
    n = 128
    cells = O.codec_cells(n)
    for trial in range(5):
        row = (rng.standard_normal(n) * rng.uniform(0.01, 3)).astype(np.float32)
        bits, mu, sigma = O.state_codec_encode_row(row)
        lo, span = np.float32(mu - np.float32(3) * sigma), np.float32(np.float32(6) * sigma)
        x = np.clip(((row - lo) / span).astype(np.float32), 0, 1)
        t = np.rint(x * np.float32(255)).astype(np.int64)
        # brute-force the accumulator path independently of the encoder's loop structure
        e, emin, emax, k = 0, 0, 0, 0
        for i in range(n):
            for _ in range(cells[i + 1] - cells[i]):
                v = e + t[i]
                assert bits[k] == (1 if v >= 128 else 0)
                e = v - 255 * bits[k]
                emin, emax = min(emin, e), max(emax, e)
                k += 1
        assert -128 <= emin and emax <= 127
        ncell = np.diff(cells)
        for i in range(n):
            dens = bits[cells[i]:cells[i + 1]].sum()
            assert abs(dens - t[i] * ncell[i] / 255) <= 1.0 + 1e-9 + 1, (i, dens, t[i])
        assert abs(bits.sum() - (t * ncell).sum() / 255) <= 1.0 + 1e-9
        # the readout lands within one cell's share of the [mu - 3 sigma, mu + 3 sigma] range, and
        # inside it, for values that were inside it
        dec = O.state_codec_decode_row(bits, mu, sigma, n)
        inside = (row >= lo) & (row <= lo + span)
        assert (dec >= lo - 1e-6).all() and (dec <= lo + span + 1e-6).all()
        assert np.mean(np.abs(dec - row)[inside]) < float(span) / 4


def test_codec_stats_are_the_row_mean_and_std():
    rng = np.random.default_rng(61)
    row = rng.standard_normal(128).astype(np.float32)
    mu, sigma = O.state_codec_stats(row)
    assert abs(float(mu) - float(np.mean(row.astype(np.float64)))) < 1e-6
    assert abs(float(sigma) - float(np.std(row.astype(np.float64)))) < 1e-6


def test_dfssd_codec_off_is_the_plain_scan_and_on_stays_close():
    rng = np.random.default_rng(62)
    T, H, P, N, G = 80, 2, 3, 16, 1
    xs = rng.standard_normal((T, H, P))
    dts = rng.uniform(1e-3, 0.2, (T, H))
    A = -rng.uniform(1, 16, H)
    Bs, Cs = rng.standard_normal((T, G, N)), rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    S0 = rng.standard_normal((H, P, N)) * 0.5
    y0, S_0 = O.ssd_chunked(xs, dts, A, Bs, Cs, D, S0, G, 16)
    y1, S_1 = O.ssd_chunked(xs, dts, A, Bs, Cs, D, S0, G, 16, codec=False)
    np.testing.assert_array_equal(y0, y1)
    yc, S_c = O.ssd_chunked(xs, dts, A, Bs, Cs, D, S0, G, 16, codec=True)
    # the first chunk never sees the codec
    np.testing.assert_array_equal(yc[:16], y0[:16])
    assert not np.array_equal(yc[16:], y0[16:])
    assert np.linalg.norm(yc - y0) / np.linalg.norm(y0) < 0.5


# ------------------------------------------------------------------ 17-level DFW scaffold
def test_dfw_levels_are_the_set_eq3_prints():
    # Eq. (3): W_scaffold in {-1, -14/16, ..., 0, ..., 14/16, 1}: 17 values, step 2/16
    w = np.linspace(-1.5, 1.5, 100001)
    wq, k = O.dfw_quantize(w)
    vals = sorted({Fraction(float(v)).limit_denominator(16) for v in wq})
    assert vals == [Fraction(2 * i, 16) - 1 for i in range(17)]
    assert set(k.tolist()) == set(range(17))
    # value and index agree: w_q = 2k/16 - 1 = (k - 8)/8
    assert np.array_equal(wq, (k - 8) / 8.0)


def test_dfw_end_points_zero_clamp_and_ties():
    wq, k = O.dfw_quantize([-1.0, 1.0, 0.0, -7.0, 3.5, 1.0 + 1e-9, -1.0 - 1e-9])
    assert wq.tolist() == [-1.0, 1.0, 0.0, -1.0, 1.0, 1.0, -1.0]
    assert k.tolist() == [0, 16, 8, 0, 16, 16, 0]
    # (w + 1)/2 * 16 = j + 1/2 exactly at w = (2j + 1)/16 - 1: round half to even picks the even j
    j = np.arange(16)
    wt = (2 * j + 1) / 16.0 - 1.0
    _, kt = O.dfw_quantize(wt)
    assert kt.tolist() == [int(x) + (int(x) % 2) for x in j]
    # just off the tie the nearer level wins
    _, kp = O.dfw_quantize(wt + 1e-9)
    assert kp.tolist() == (j + 1).tolist()


def test_dfw_idempotent_monotone_and_half_step_error():
    rng = np.random.default_rng(21)
    w = np.sort(rng.uniform(-1.2, 1.2, 20000))
    wq, _ = O.dfw_quantize(w)
    assert np.array_equal(O.dfw_quantize(wq)[0], wq)
    assert (np.diff(wq) >= 0).all()
    inside = np.abs(w) <= 1
    assert np.abs(wq - w)[inside].max() <= 1 / 16 + 1e-15


def test_dfw_planes_match_pure_python_bit_extraction():
    lv = gen.dfw_levels(3, 24, seed=2)
    assert lv.min() >= 0 and lv.max() <= 16
    planes = gen.pack_level_planes(lv)
    assert planes.shape == (5, 3, 3)
    k = O.dfw_unpack_planes(planes, 24)
    for n in range(3):
        for i in range(24):
            v = sum(((int(planes[b, n, i // 8]) >> (i % 8)) & 1) << b for b in range(5))
            assert k[n, i] == v == lv[n, i]


def test_dfw_levels_generator_covers_all_17():
    lv = gen.dfw_levels(64, 2048, seed=0)
    assert set(np.unique(lv).tolist()) == set(range(17))


def test_project_dfw_brute_force_exact():
    P = gen.dfw_proj(5, 24, 3, seed=4)
    rng = np.random.default_rng(6)
    q = rng.integers(-127, 128, 24).astype(np.int8)
    s = np.float32(0.0293)
    y, acc, t = O.project_dfw(q, s, P)
    S = Fraction(float(s))
    for n in range(5):
        a = Fraction(0)
        for i in range(24):
            k = sum(((int(P.planes[b, n, i // 8]) >> (i % 8)) & 1) << b for b in range(5))
            a += (Fraction(2 * k, 16) - 1) * int(q[i])          # Eq. (1)'s level value times the code
        assert acc[n] == 8 * a
        exact = S * Fraction(float(P.row_scale[n])) * a
        for j in range(3):
            tj = sum(int(P.lora_dn[j, i]) * int(q[i]) for i in range(24))
            assert t[j] == tj
            exact += Fraction(float(P.up_scale[n])) * int(P.lora_up[n, j]) * Fraction(float(P.dn_scale[j])) * S * tj
        assert abs(float(exact) - y[n]) <= 1e-12 * max(1.0, abs(float(exact)))


def test_project_dfw_end_levels_equal_the_one_bit_projection():
    # a 17-level scaffold that only uses levels 0 and 16 (-1 and +1) is the 1-bit scaffold
    P1 = _proj(12, 64, 4, seed=10)
    bits = np.unpackbits(P1.sign, axis=1, bitorder="little")[:, :64].astype(np.int64)
    Pd = gen.DfwProjWeights(gen.pack_level_planes(16 * bits), P1.row_scale, P1.lora_dn, P1.dn_scale,
                            P1.lora_up, P1.up_scale)
    rng = np.random.default_rng(11)
    q = rng.integers(-127, 128, 64).astype(np.int8)
    y1, acc1, t1 = O.project(q, np.float32(0.017), P1)
    yd, accd, td = O.project_dfw(q, np.float32(0.017), Pd)
    assert np.array_equal(accd, 8 * acc1) and np.array_equal(td, t1)
    np.testing.assert_allclose(yd, y1, rtol=1e-13, atol=1e-15)
    # and the middle level contributes nothing
    P0 = gen.DfwProjWeights(gen.pack_level_planes(np.full((12, 64), 8)), P1.row_scale, P1.lora_dn,
                            P1.dn_scale, P1.lora_up, P1.up_scale)
    y0, acc0, _ = O.project_dfw(q, np.float32(0.017), P0)
    assert (acc0 == 0).all()


def test_layer_dfssd_matches_chunked_codec_scan_and_reduces_to_plain():
    dm = _tiny_dims()
    W = gen.layer_weights(dm, 0, seed=12)
    rng = np.random.default_rng(13)
    T, Q = 11, 4
    xs = rng.standard_normal((T, dm.d_model))
    conv0 = rng.standard_normal((dm.conv_dim, dm.d_conv - 1)) * 0.1
    ssm0 = rng.standard_normal((dm.nheads, dm.headdim, dm.d_state)) * 0.1
    o, cs, ss, tp = O.layer_tokens(xs, W, conv0, ssm0, codec_chunk=Q)
    A = -np.exp(np.asarray(W.A_log, np.float64))
    ys, S = O.ssd_chunked(tp["x"].reshape(T, dm.nheads, dm.headdim), tp["dt"], A, tp["B"], tp["C"], W.D, ssm0,
                          dm.ngroups, Q, codec=True)
    np.testing.assert_allclose(ss, S, rtol=1e-9, atol=1e-12)
    assert tp["state_in"].shape[0] == tp["state_pre"].shape[0] == 3
    assert np.array_equal(tp["state_in"][0], ssm0) and not np.allclose(tp["state_in"][1], tp["state_pre"][1])
    # forcing the coded states with the oracle's own gives the same run
    o2, _, ss2, _ = O.layer_tokens(xs, W, conv0, ssm0, force={"state_in": tp["state_in"]}, codec_chunk=Q)
    assert np.array_equal(o2, o) and np.array_equal(ss2, ss)
    # one chunk over the whole sequence: no boundary, the plain layer
    o3, _, ss3, _ = O.layer_tokens(xs, W, conv0, ssm0, codec_chunk=T)
    o4, _, ss4, _ = O.layer_tokens(xs, W, conv0, ssm0)
    assert np.array_equal(o3, o4) and np.array_equal(ss3, ss4)
