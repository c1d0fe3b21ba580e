"""Every kind of shape the C ABI accepts, at small sizes, through each entry point: layer decode on
the packed-sign GEMV (batch 1) and on the int8 MFMA GEMMs (batch 8), the batch-1 stack decode (the
persistent kernel where the shape fits it, per-layer launches otherwise) and prefill. Each is held to
the same P1/P2 protocol as the workload shapes: codes and integer sums exact against the oracle,
floats within 1e-3 with the GPU's codes forced in."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say, run_layer, forced_chain, run_stack
from test_gpu_prefill import run_prefill, check_sequence

pytestmark = pytest.mark.gpu


def _dims(d_model=256, d_inner=512, d_state=16, ngroups=1, rank=8):
    H = d_inner // 64
    nat = 2 * d_inner + 2 * ngroups * d_state + H
    return gen.Dims(d_model=d_model, d_inner=d_inner, d_state=d_state, headdim=64, ngroups=ngroups, d_conv=4,
                    n_in_proj=(nat + 15) // 16 * 16, rank_in=rank, rank_out=rank)


SHAPES = {
    "ngroups2": _dims(ngroups=2),
    "ngroups4_state32": _dims(d_state=32, ngroups=4),
    "state32": _dims(d_state=32),
    "state64": _dims(d_state=64),
    "state256": _dims(d_state=256),
    "rank64": _dims(rank=64),
    "rank16": _dims(rank=16),
    "rank12": _dims(rank=12),
    "dmodel384": _dims(d_model=384, d_inner=768),
    "dmodel1024": _dims(d_model=1024, d_inner=2048),
    "dmodel4096": _dims(d_model=4096, d_inner=8192),
    "dinner_3x": _dims(d_model=256, d_inner=768),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_shape_layer_decode_gemv_and_mfma(name):
    dims = SHAPES[name]
    steps = 2 if dims.d_model >= 4096 else 3
    for B in (1, 8):
        lw = gen.layer_weights(dims, 1, 60, random_norms=True, per_channel_lora=True)
        conv0, ssm0 = gen.initial_states(dims, B, 1, 60, std=0.2)
        xs = gen.token_inputs(dims, (steps, B), 60, tag=1)
        say(f"case: {name} layer decode, batch {B}, {steps} steps")
        outs, tps, final, _ = run_layer(dims, lw, xs, conv0, ssm0)
        dense = O.dense_signs(lw)
        for b in sorted({0, B - 1}):
            worst, ec, es = forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)
            say(f"{name} batch {B} row {b}: out {worst:.2e} conv {ec:.2e} ssm {es:.2e}")


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_shape_stack_decode_batch1(name):
    L, Dv = _lib()
    dims = SHAPES[name]
    nL, T = 2, 3
    layers = gen.stack_weights(dims, nL, seed=61, random_norms=True, per_channel_lora=True)
    states0 = [gen.initial_states(dims, 1, l, 61, std=0.1) for l in range(nL)]
    x0 = gen.token_inputs(dims, (1,), 61, tag=2)
    fw = np.random.default_rng(61).uniform(0.5, 1.5, dims.d_model).astype(np.float32)
    # the persistent kernel where the shape fits it (the default), else per-layer launches
    path = L.DFSSM_PATH_FLOW
    ws_probe = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)
    devs = [Dv.DeviceLayer(lw) for lw in layers]
    sts = [Dv.DeviceState(c, s_) for c, s_ in states0]
    arr_w, arr_s = Dv._arrays(devs, sts)
    y_probe = torch.empty((1, 1, dims.d_model), device="cuda")
    x_probe = torch.from_numpy(x0).cuda()
    r = L.dfssm_stack_decode_ex(Dv.dims_struct(dims), arr_w, arr_s, nL, torch.from_numpy(fw).cuda().data_ptr(),
                                x_probe.data_ptr(), y_probe.data_ptr(), 1, 1, ws_probe.data_ptr(), ws_probe.numel(),
                                None, L.dfssm_stack_opts(L.DFSSM_PATH_FLOW, 0), Dv.stream_handle())
    torch.cuda.synchronize()
    if r == L.DFSSM_EUNSUPPORTED:
        path = L.DFSSM_PATH_PER_LAYER
    else:
        L.check(r, "probe")
    say(f"case: {name} stack decode, {nL} layers, {T} steps, batch 1, path {path}")
    y, states, taps = run_stack(dims, layers, x0, states0, T, taps=True, final_w=fw, path=path)
    dense = [O.dense_signs(lw) for lw in layers]
    cs = [s_[0][0].astype(np.float64) for s_ in states0]
    ss = [s_[1][0].astype(np.float64) for s_ in states0]
    x = x0[0].astype(np.float64)
    for t in range(T):
        h = x
        for l in range(nL):
            tap = PY.tap_record(taps, t * nL + l)
            PY.assert_codes_exact(tap["in_u"], tap["in_q"], tap["in_s"][0], f"{name} t{t} l{l} in")
            PY.assert_codes_exact(tap["out_u"], tap["out_q"], tap["out_s"][0], f"{name} t{t} l{l} out")
            PY.assert_products_exact(layers[l].in_proj, tap["in_q"], tap["in_acc"], tap["in_t"], dense[l]["in"])
            PY.assert_products_exact(layers[l].out_proj, tap["out_q"], tap["out_acc"], tap["out_t"], dense[l]["out"])
            force = dict(in_q=tap["in_q"], in_s=tap["in_s"][0], out_q=tap["out_q"], out_s=tap["out_s"][0])
            h, cs[l], ss[l], _ = O.layer_decode(h, layers[l], cs[l], ss[l], force=force, dense=dense[l])
        yo = O.rmsnorm(h, fw, dims.eps)
        e = PY.err(y[t][0], yo)
        assert e < PY.TOL_LAYER, (name, t, e)
        x = yo
    for l in range(nL):
        assert PY.err(states[l][0][0], cs[l]) < PY.TOL_LAYER and PY.err(states[l][1][0], ss[l]) < PY.TOL_LAYER, (name, l)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_shape_prefill(name):
    L, Dv = _lib()
    dims = SHAPES[name]
    B, T, Q = 2, 70, 32
    lw = gen.layer_weights(dims, 2, 62, random_norms=True, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(dims, B, 2, 62, std=0.2)
    xs = gen.token_inputs(dims, (B, T), 62, tag=3)
    if dims.rank_in % 8:
        # the prefill GEMM epilogue takes ranks in multiples of 8: the call must say so
        assert L.dfssm_workspace_bytes(Dv.dims_struct(dims), L.DFSSM_OP_LAYER_PREFILL, B, T) == 0
        return
    say(f"case: {name} prefill, batch {B}, seqlen {T}, chunk {Q}")
    out, tps, final = run_prefill(dims, lw, xs, conv0, ssm0, Q)
    dense = O.dense_signs(lw)
    for b in range(B):
        tb = {k: v[b] for k, v in tps.items()}
        errs = check_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], tb, (final[0][b], final[1][b]), dense,
                              what=f"{name} row {b}")
        say(f"{name} prefill row {b}: {errs}")
