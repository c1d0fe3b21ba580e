"""The largest sizes the C ABI accepts, each against the oracle on sampled rows: layer decode at
batch 4096, the LM head at batch 4096 (tiny vocabulary), the 17-level projection at batch 256,
the state codec at batch 4096, and the layer prefill at batch 64 (ragged 300-token sequences)."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say, run_layer, forced_chain

pytestmark = pytest.mark.gpu
TINY = gen.DIMS["tiny"]


def test_layer_decode_batch_4096_sampled_rows():
    B, T = 4096, 2
    lw = gen.layer_weights(TINY, 0, seed=31)
    conv0, ssm0 = gen.initial_states(TINY, B, 0, 31, std=0.1)
    xs = gen.token_inputs(TINY, (T, B), 31, tag=1)
    say(f"case: tiny layer decode, batch {B} (the largest), {T} steps")
    outs, tps, final, _ = run_layer(TINY, lw, xs, conv0, ssm0)
    dense = O.dense_signs(lw)
    for b in (0, 1, 2047, 4000, 4095):
        worst, ec, es = forced_chain(lw, xs, conv0, ssm0, outs, tps, final, b=b, dense=dense)
        say(f"row {b}: forced max err {worst:.2e} conv {ec:.2e} ssm {es:.2e}")


def test_lm_head_batch_4096_sampled_rows():
    L, Dv = _lib()
    emb_np = gen.embedding(TINY, vocab=300, seed=32)
    emb = Dv.DeviceEmbedding(emb_np)
    B = 4096
    ys = O.rmsnorm(gen.token_inputs(TINY, (B,), 32, tag=2), np.ones(TINY.d_model), TINY.eps).astype(np.float32)
    y = torch.from_numpy(ys).cuda()
    logits = torch.empty((B, emb_np.vocab), device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    say(f"case: LM head, vocab 300, batch {B} (the largest)")
    Dv.lm_head(TINY, emb, y, logits, nxt)
    torch.cuda.synchronize()
    lg, nx = logits.cpu().numpy(), nxt.cpu().numpy()
    for b in (0, 7, 2048, 4095):
        lo, _, _, _ = O.lm_head(ys[b], emb_np.codes, emb_np.row_scale)
        assert PY.err(lg[b], lo) < PY.TOL_LAYER, b
        assert nx[b] == O.argmax_first(lg[b]), b


def test_dfw_project_batch_256():
    L, Dv = _lib()
    P = gen.dfw_proj(96, 256, 8, seed=33)
    B = 256
    xs = np.random.default_rng(33).standard_normal((B, 256)).astype(np.float32)
    dp = Dv.DeviceDfwProj(P)
    x = torch.from_numpy(xs).cuda()
    y = torch.empty((B, 96), device="cuda")
    acc = torch.empty((B, 96), dtype=torch.int32, device="cuda")
    say(f"case: 17-level projection 96 x 256, batch {B} (the largest)")
    Dv.dfw_project(dp, x, y, taps=dict(acc=acc))
    torch.cuda.synchronize()
    yn, an = y.cpu().numpy(), acc.cpu().numpy()
    k = O.dfw_unpack_planes(P.planes, 256)
    for b in (0, 3, 128, 255):
        q, s = O.quantize_token(xs[b])
        yo, ao, _ = O.project_dfw(q, s, P, k=k)
        assert (an[b].astype(np.int64) == ao).all(), b
        assert PY.err(yn[b], yo) < PY.TOL_LAYER, b


def test_state_codec_batch_4096_sampled_rows():
    L, Dv = _lib()
    B = 4096
    _, S = gen.initial_states(TINY, B, 0, 34, std=0.1)
    ssm = torch.from_numpy(S).cuda()
    say(f"case: state codec, tiny state at batch {B} (the largest): {S.size // 16} rows of 16")
    fields, stats = Dv.state_encode(TINY, ssm, B)
    back = torch.empty_like(ssm)
    Dv.state_decode(TINY, fields, stats, B, back)
    torch.cuda.synchronize()
    f = fields.cpu().numpy().view(np.uint32)
    st = stats.cpu().numpy()
    bk = back.cpu().numpy().reshape(-1, 16)
    flat = S.reshape(-1, 16)
    K2 = O.codec_field_side(16) ** 2
    for r in (0, 63, 64, flat.shape[0] // 2, flat.shape[0] - 1):
        bits, mu, sigma = O.state_codec_encode_row(flat[r])
        got = ((f[r][:, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(-1)[:K2]
        assert (got == bits).all() and st[r, 0] == mu and st[r, 1] == sigma, r
        ref = O.state_codec_decode_row(bits, mu, sigma, 16)
        assert np.abs(bk[r] - ref).max() <= 1e-6 * (abs(float(mu)) + 6 * float(sigma)), r


def test_layer_prefill_batch_64_ragged_sampled_sequences():
    from test_gpu_prefill import run_prefill, check_sequence
    lw = gen.layer_weights(TINY, 0, seed=35)
    B, T = 64, 300
    xs = gen.token_inputs(TINY, (B, T), 35, tag=3)
    conv0, ssm0 = gen.initial_states(TINY, B, 0, 35, std=0.1)
    say(f"case: tiny layer prefill, batch {B} (the largest), {T} tokens, chunk 64")
    out, tps, final = run_prefill(TINY, lw, xs, conv0, ssm0, 64)
    for b in (0, 31, 63):
        errs = check_sequence(lw, xs[b], conv0[b], ssm0[b], out[b], {k: v[b] for k, v in tps.items()},
                              (final[0][b], final[1][b]), what=f"batch-64 prefill row {b}")
        say(f"row {b}: {errs}")
