"""GPU parity of the tied int8 embedding and LM head (dfssm_embed, dfssm_lm_head) against the
oracle: the head's codes and integer row sums exact, logits within 1e-3 (element-wise bound), the
greedy token a maximum of the oracle's logits (the smallest index among exact ties); embedding rows
equal to the fp32 rounding of the oracle's exact products."""
import numpy as np
import pytest
import torch

from synth import gen
from oracle import dfssm_oracle as O
import dfssm_parity as PY
from test_gpu_decode import _lib, say

pytestmark = pytest.mark.gpu


def _run_head(dims, emb_np, ys, with_logits=True):
    L, Dv = _lib()
    emb = Dv.DeviceEmbedding(emb_np)
    B, V = ys.shape[0], emb_np.vocab
    y = torch.from_numpy(ys).cuda()
    logits = torch.empty((B, V), device="cuda") if with_logits else None
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    taps = dict(q=torch.empty((B, dims.d_model), dtype=torch.int8, device="cuda"),
                s=torch.empty(B, device="cuda"), acc=torch.empty((B, V), dtype=torch.int32, device="cuda"))
    Dv.lm_head(dims, emb, y, logits, nxt, taps=taps)
    torch.cuda.synchronize()
    return (None if logits is None else logits.cpu().numpy(), nxt.cpu().numpy(),
            {k: v.cpu().numpy() for k, v in taps.items()})


def _check(emb_np, ys, logits, nxt, taps, what):
    for b in range(ys.shape[0]):
        lo, acc, q, s = O.lm_head(ys[b], emb_np.codes, emb_np.row_scale)
        assert (taps["q"][b] == q).all() and np.float32(taps["s"][b]) == s, f"{what} row {b}: codes"
        bad = np.flatnonzero(taps["acc"][b].astype(np.int64) != acc)
        assert bad.size == 0, f"{what} row {b}: {bad.size} integer row sums differ, e.g. {bad[:5]}"
        if logits is not None:
            e = PY.err(logits[b], lo)
            assert e < PY.TOL_LAYER, (what, b, e)
            # the GPU's token is the first maximum of its own logits
            assert nxt[b] == O.argmax_first(logits[b]), (what, b)
        # and a maximum of the oracle's logits up to their rounding
        top = lo.max()
        assert lo[nxt[b]] >= top - 1e-6 * abs(top), (what, b, nxt[b], O.argmax_first(lo))


@pytest.mark.parametrize("B", [1, 3, 8, 11])
def test_lm_head_tiny_vocab_ragged(B):
    dims = gen.DIMS["tiny"]
    emb_np = gen.embedding(dims, vocab=1000, seed=3)
    ys = O.rmsnorm(gen.token_inputs(dims, (B,), 3, tag=20), np.ones(dims.d_model), dims.eps).astype(np.float32)
    say(f"case: LM head, vocab 1000, d_model 256, batch {B}")
    logits, nxt, taps = _run_head(dims, emb_np, ys)
    _check(emb_np, ys, logits, nxt, taps, f"tiny B={B}")


def test_lm_head_planted_maximum_and_ties():
    dims = gen.DIMS["tiny"]
    emb_np = gen.embedding(dims, vocab=777, seed=4)
    ys = O.rmsnorm(gen.token_inputs(dims, (2,), 4, tag=21), np.ones(dims.d_model), dims.eps).astype(np.float32)
    q, _ = O.quantize_token(ys[0])
    row = np.where(q >= 0, 127, -127).astype(np.int8)
    for v in (5, 600, 776):                       # three equal rows: the first must win
        emb_np.codes[v] = row
        emb_np.row_scale[v] = 2e-3
    say("case: LM head with a planted maximum in three rows")
    logits, nxt, taps = _run_head(dims, emb_np, ys)
    assert nxt[0] == 5
    _check(emb_np, ys, logits, nxt, taps, "planted")


@pytest.mark.parametrize("B", [1, 4])
def test_lm_head_1p3b_full_vocab(B):
    dims = gen.DIMS["1p3b"]
    emb_np = gen.embedding(dims, seed=0)
    ys = O.rmsnorm(gen.token_inputs(dims, (B,), 0, tag=22), np.ones(dims.d_model), dims.eps).astype(np.float32)
    say(f"case: LM head, vocab {emb_np.vocab}, d_model 2048, batch {B}")
    logits, nxt, taps = _run_head(dims, emb_np, ys)
    _check(emb_np, ys, logits, nxt, taps, f"1p3b B={B}")
    # greedy tokens without the logits output are the same
    _, nxt2, _ = _run_head(dims, emb_np, ys, with_logits=False)
    assert (nxt2 == nxt).all()


def test_embed_rows_exact():
    L, Dv = _lib()
    for dims, V in ((gen.DIMS["tiny"], 1000), (gen.DIMS["1p3b"], gen.VOCAB_1P3B)):
        emb_np = gen.embedding(dims, vocab=V, seed=5)
        toks = gen.token_ids(37, V, seed=5)
        toks[:3] = [0, V - 1, toks[5]]
        emb = Dv.DeviceEmbedding(emb_np)
        t = torch.from_numpy(toks).cuda()
        x = torch.empty((toks.size, dims.d_model), device="cuda")
        say(f"case: embedding gather, vocab {V}, {toks.size} tokens")
        Dv.embed(emb, t, x)
        torch.cuda.synchronize()
        ref = O.embed(toks, emb_np.codes, emb_np.row_scale).astype(np.float32)   # the fp32 rounding of exact products
        assert (x.cpu().numpy() == ref).all()
