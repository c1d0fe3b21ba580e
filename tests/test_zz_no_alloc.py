"""dfssm_layer_decode_noalloc (the entry point for callers that cannot allocate) against
dfssm_layer_decode: the same kernels over the same inputs, so outputs, states and taps must be
identical bit for bit. Two calls in a row share the library's fixed scratch array; the second
runs a smaller input, so stale contents from the first are present when it starts."""
import ctypes as C

import numpy as np
import pytest
import torch

from synth import gen

pytestmark = pytest.mark.gpu


def _lib():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm device"
    from bit_quantized_mamba_packed_amd import _lib as L, device as Dv
    L.load()
    return L, Dv


def _pair(dims, layer, seed, batch, steps, std):
    """Run `steps` decode steps through both entry points from the same state; return both runs."""
    L, Dv = _lib()
    lw = gen.layer_weights(dims, layer, seed, random_norms=True, per_channel_lora=True)
    conv0, ssm0 = gen.initial_states(dims, batch, layer, seed, std=std)
    xs = gen.token_inputs(dims, (steps, batch), seed, tag=5)
    dev = Dv.DeviceLayer(lw)
    st_a, st_b = Dv.DeviceState(conv0, ssm0), Dv.DeviceState(conv0, ssm0)
    ws = Dv.workspace(dims, L.DFSSM_OP_LAYER_DECODE, batch)
    d = Dv.dims_struct(dims)
    stream = Dv.stream_handle()
    out = {"a": [], "b": [], "ta": [], "tb": []}
    for t in range(steps):
        x = torch.from_numpy(xs[t]).cuda()
        ya, yb = torch.empty_like(x), torch.empty_like(x)
        ta, tb = Dv.Taps(dims, batch), Dv.Taps(dims, batch)
        L.check(L.dfssm_layer_decode(d, dev.struct, st_a.struct, x.data_ptr(), ya.data_ptr(), batch, ws.data_ptr(),
                                     ws.numel(), ta.struct, stream), "dfssm_layer_decode")
        L.check(L.dfssm_layer_decode_noalloc(d, dev.struct, st_b.struct, x.data_ptr(), yb.data_ptr(), batch, tb.struct,
                                             stream), "dfssm_layer_decode_noalloc")
        torch.cuda.synchronize()
        out["a"].append(ya.cpu().numpy())
        out["b"].append(yb.cpu().numpy())
        out["ta"].append(ta.numpy())
        out["tb"].append(tb.numpy())
    return out, (st_a, st_b)


def _same(out, states, what):
    for t in range(len(out["a"])):
        assert np.array_equal(out["a"][t], out["b"][t]), f"{what}: output of step {t} differs"
        for k in out["ta"][t]:
            np.testing.assert_array_equal(out["ta"][t][k], out["tb"][t][k], err_msg=f"{what}: tap {k} step {t}")
    a, b = states
    assert torch.equal(a.conv, b.conv) and torch.equal(a.ssm, b.ssm), f"{what}: states differ"
    assert np.isfinite(np.stack(out["a"])).all()


def test_noalloc_matches_layer_decode_two_calls_second_smaller():
    L, Dv = _lib()
    big = gen.DIMS["1p3b"]
    print("case: no-alloc layer decode, 1.3B layer, batch 48 (skinny MFMA GEMMs), 2 steps", flush=True)
    out, st = _pair(big, 0, 30, 48, 2, 0.1)
    _same(out, st, "1.3B batch 48")
    print("case: no-alloc layer decode, 1.3B layer, batch 4 (packed-sign GEMV), 3 steps", flush=True)
    out, st = _pair(big, 0, 31, 4, 3, 0.1)
    _same(out, st, "1.3B batch 4")
    print("case: no-alloc layer decode, tiny layer, batch 2, 2 steps (smaller, after the larger)", flush=True)
    out, st = _pair(gen.DIMS["tiny"], 1, 32, 2, 2, 0.2)
    _same(out, st, "tiny batch 2")
    print("case: no-alloc layer decode, tiny layer, batch 16 (MFMA projections)", flush=True)
    out, st = _pair(gen.DIMS["tiny"], 2, 33, 16, 2, 0.2)
    _same(out, st, "tiny batch 16")


def test_noalloc_rejects_what_exceeds_the_scratch():
    L, Dv = _lib()
    big = gen.DIMS["1p3b"]
    d = Dv.dims_struct(big)
    B = 512
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_DECODE, B) > L.DFSSM_NOALLOC_SCRATCH_BYTES
    lw = Dv.DeviceLayer(gen.layer_weights(big, 0, 0))
    conv = torch.zeros((B, big.conv_dim, big.d_conv - 1), device="cuda")
    ssm = torch.zeros((B, big.nheads, big.headdim, big.d_state), device="cuda")
    st = Dv.DeviceState.from_tensors(conv, ssm, big, B)
    x = torch.zeros((B, big.d_model), device="cuda")
    y = torch.empty_like(x)
    r = L.dfssm_layer_decode_noalloc(d, lw.struct, st.struct, x.data_ptr(), y.data_ptr(), B, None,
                                     Dv.stream_handle())
    assert r == L.DFSSM_EWORKSPACE, L.dfssm_strerror(r)
