"""The 48-layer 1.3B-shaped stack decode at the batch sizes of the pages' batched throughput table
(8, 32, 128, 512; batch 1 and 64 have their own tests): beyond 4 tokens the projections run as int8
MFMA GEMMs (the skinny kernel up to 64 rows, the tile kernel above). One step from zero states, then
one tapped step: the codes and integer sums of sampled rows are checked exact against the oracle,
and every layer of those rows in isolation from the GPU's own state and input (codes forced)."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say

pytestmark = pytest.mark.gpu

BIG = gen.DIMS["1p3b"]
NL = 48
_cache = {}


def _layers():
    if "layers" not in _cache:
        _cache["layers"] = gen.stack_weights(BIG, NL, seed=0)
        _cache["dense"] = [O.dense_signs(lw) for lw in _cache["layers"]]
    return _cache["layers"], _cache["dense"]


@pytest.mark.parametrize("B", [8, 32, 128, 512])
def test_stack_decode_1p3b_48_layers_batch_sweep(B):
    L, Dv = _lib()
    layers, dense = _layers()
    if "dev" not in _cache:
        _cache["dev"] = [Dv.DeviceLayer(lw) for lw in layers]
    devs = _cache["dev"]
    conv = torch.zeros((NL, B, BIG.conv_dim, BIG.d_conv - 1), device="cuda")
    ssm = torch.zeros((NL, B, BIG.nheads, BIG.headdim, BIG.d_state), device="cuda")
    sts = [Dv.DeviceState.from_tensors(conv[l], ssm[l], BIG, B) for l in range(NL)]
    fw = torch.ones(BIG.d_model, device="cuda")
    x0 = torch.from_numpy(gen.token_inputs(BIG, (B,), 0, tag=12)).cuda()
    ws = Dv.workspace(BIG, L.DFSSM_OP_STACK_DECODE, B, 0, NL)
    y1 = torch.empty((1, B, BIG.d_model), device="cuda")
    say(f"case: 1.3B stack decode, {NL} layers, batch {B}, one step from zero states")
    Dv.stack_decode(BIG, devs, sts, fw, x0, y1, 1, ws)
    torch.cuda.synchronize()
    assert Dv.stack_status(ws) == L.DFSSM_STATUS_OK
    assert torch.isfinite(y1).all()
    rows = sorted({0, B // 2, B - 1})
    before = [(conv[l][rows].cpu().numpy(), ssm[l][rows].cpu().numpy()) for l in range(NL)]
    y2 = torch.empty((1, B, BIG.d_model), device="cuda")
    taps = Dv.Taps(BIG, NL * B)
    say(f"case: same stack, batch {B}, one tapped step")
    x1 = y1[0].contiguous()
    Dv.stack_decode(BIG, devs, sts, fw, x1, y2, 1, ws, taps)
    torch.cuda.synchronize()
    assert Dv.stack_status(ws) == L.DFSSM_STATUS_OK
    y2n = y2.cpu().numpy()[0]
    assert (y2n == y2n).all()
    worst = {}
    for l in range(NL):
        for i, b in enumerate(rows):
            idx = torch.tensor([l * B + b, (l + 1) * B + b if l + 1 < NL else l * B + b], device="cuda")
            tap = {k: v[idx].cpu().numpy() for k, v in taps.t.items()}
            rec = {k: v[0] for k, v in tap.items()}
            PY.assert_codes_exact(rec["in_u"], rec["in_q"], rec["in_s"][0], f"B={B} l{l} b{b} in")
            PY.assert_codes_exact(rec["out_u"], rec["out_q"], rec["out_s"][0], f"B={B} l{l} b{b} out")
            PY.assert_products_exact(layers[l].in_proj, rec["in_q"], rec["in_acc"], rec["in_t"], dense[l]["in"])
            PY.assert_products_exact(layers[l].out_proj, rec["out_q"], rec["out_acc"], rec["out_t"], dense[l]["out"])
            if l == 0:
                assert (rec["h_in"] == y1.cpu().numpy()[0][b]).all()
            force = dict(in_q=rec["in_q"], in_s=rec["in_s"][0], out_q=rec["out_q"], out_s=rec["out_s"][0])
            h, cs, ss, _ = O.layer_decode(rec["h_in"], layers[l], before[l][0][i], before[l][1][i], force=force,
                                          dense=dense[l])
            errs = dict(conv=PY.err(conv[l][b].cpu().numpy(), cs), ssm=PY.err(ssm[l][b].cpu().numpy(), ss))
            errs["out"] = PY.err(tap["h_in"][1], h) if l + 1 < NL else \
                PY.err(y2n[b], O.rmsnorm(h, np.ones(BIG.d_model), BIG.eps))
            for k, v in errs.items():
                assert v < PY.TOL_LAYER, (B, l, b, errs)
                worst[k] = max(worst.get(k, 0.0), v)
    say(f"batch {B}: worst per-layer errors over rows {rows}: {worst}")
    del taps, conv, ssm, sts, ws
    torch.cuda.empty_cache()
