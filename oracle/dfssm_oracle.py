"""CPU oracle of the DF-SSM inference hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module. The product path (the HIP library and its Python binding) never
does, and shares no code, constant or helper with it.

It is plain NumPy: floating point in fp64, integers exact, except where the method turns a float
into an integer (the per-token int8 quantizer), which is evaluated in fp32 so that the oracle and
the kernels take that decision in the same precision.

Source: the page "Density Field State Space Models: 1-Bit Distillation, Efficient Inference, and
Knowledge Organization in Mamba-2" (arXiv 2606.10932), cited below as [DF-SSM], plus the Mamba-2
/ SSD paper it builds on (Dao & Gu 2024, cited in [DF-SSM] §2), cited as [SSD].

What each function follows and what pins it (the pins live in tests/test_oracle_pins.py):

  unpack_signs      [DF-SSM] §4.1 (1-bit packed scaffold), §4.2 (64 weights per 8 bytes)
                    pinned by: pure-Python bit extraction; Table 1 byte count; complement -> -acc
  quantize_token    reading R4 (the paper gives no activation quantizer; int8 is implied by the
                    INT8 matmul of §4.1).  pinned by: amax -> +-127, constructed ties round to
                    even, zero vector, odd symmetry, Python's round() on tiny vectors
  project           [DF-SSM] §3.2 Eq. (3) with int8 factors (§3.3).  pinned by: brute force with
                    Python ints/Fractions; parity and bound of the scaffold sum
  conv_step         depthwise causal conv of Mamba-2 ([DF-SSM] §4.1 "stateful shift register").
                    pinned by: numpy.convolve over a sequence; impulse response = taps
  ssm_step          [DF-SSM] App. B Table 12 (h = A h + (x dt) (x) B) and [SSD].
                    pinned by: B = 0 -> y = D x and zero state; dt -> 0 leaves the state;
                    one step from zero has a closed form; A -> -inf is memoryless
  gated_rmsnorm     [DF-SSM] App. B Table 12, norm(y * silu(z)).  pinned by: constant gate
                    drops out (order check); scale invariance
  layer_decode      composition of the above in Mamba-2 order.  pinned by: z == 0 -> identity,
                    batch independence, code-forcing consistency
  ssd_chunked       [SSD] chunked scan.  pinned by: equals the sequential recurrence for several
                    chunk sizes and the SSD quadratic (masked-attention) form
  layer_prefill     defined as sequential decode steps (quantization is per token).
                    pinned by: prefill(L1) then decode(L2) == decode(L1 + L2)
  layer_tokens      the same steps run stage by stage over the sequence (batched projections).
                    pinned by: equals layer_decode_steps (codes, integer sums and floats)
  table1_bytes      [DF-SSM] §3.3 Table 1.  pinned by the table's printed sizes
  state_codec_*     [DF-SSM] §3.4 (density field state: mean +- 3 sigma normalisation, first-order
                    sigma-delta with an 8-bit accumulator, threshold 0.5, popcount readout) and App. D
                    (K = 23 for d_state 128, K^2 ~ 4 d_state), reading R19.  pinned by: constant rows
                    read back exactly; the sigma-delta density within one cell of each value; the
                    accumulator bounds; the field sizes App. D prints
  ssd_chunked       with codec=True: the carried state passes through the codec at every chunk
                    boundary (DF-SSD, §3.4 / App. D).  pinned by: codec off equals the plain scan
  layer_tokens      with codec_chunk: the same DF-SSD inside the layer.  pinned by: its SSM part equals
                    ssd_chunked(codec=True) on the layer's own x, dt, B, C; one chunk covering the
                    sequence equals the plain layer
  embed             [DF-SSM] §3.3 (int8 embedding, per-row scale), Table 1 (103 MB, tied).
                    pinned by: Table 1's embedding size; rows by explicit indexing
  lm_head           the tied head over the same int8 rows (Table 1 "Embedding + LM head (tied)")
                    with the per-token quantizer (R18).  pinned by: brute force with Python ints;
                    the dequantised dense product; planted maxima for the argmax
  dfw_quantize      [DF-SSM] §3.1 Eq. (1) (17 levels, K_w = 16), R20.  pinned by: the level set
                    Eq. (3) prints; end points, zero and clamping; ties to even; idempotence,
                    monotonicity and the half-step error bound
  dfw_unpack_planes the 5-bit level index in five 1-bit planes (R20).  pinned by: pure-Python
                    bit extraction
  project_dfw       Eq. (3) with the 17-level scaffold (R20).  pinned by: brute force with
                    Fractions; with only the end levels it equals the 1-bit project()

Readings where the page is silent (also listed in the design doc):
  R1 scaffold values are +-1 times a per-output-row fp16 scale (the page's 1-bit storage; 1 bit
     cannot hold the 17-level grid of Eq. (1), so no zero weights exist);
  R2 bit layout: rows along the input dimension, LSB-first in each byte, bit 1 -> +1;
  R4 activation quantizer: per token, symmetric, a = max|u|, inv = fl32(127/a),
     q = clamp(rint_half_even(fl32(u*inv)), -127, 127), s = fl32(a/127); a == 0 -> q = 0, s = 0;
  R5 the low-rank path consumes the same int8 codes as the scaffold: t = L_dn q (int32), then
     y += up_scale * L_up (dn_scale * s * t);  alpha of Eq. (3) is 1 (folded into the scales);
  R11 in_proj rows are [z | x | B | C | dt | padding], the Mamba-2 order;
  R12 pre-norm residual block h + Mixer(RMSNorm(h)), eps 1e-5 for every norm;
  R14 discretisation dA = exp(dt*A), dB x = dt * x * B (App. B Table 12), no ZOH factor;
  R15 dt = softplus(dt_raw + dt_bias);  A = -exp(A_log);
  R17 conv applies to x, B and C; SiLU after the conv on all three; the conv state keeps the last
      d_conv-1 pre-activation inputs, oldest first;
  R18 the tied LM head reads the stack's normalised output y through the same per-token int8
      quantizer as the projections: logits[v] = s * row_scale[v] * sum_k codes[v,k] q[k] (an
      integer contraction like the scaffold's); the argmax takes the smallest index among equal
      maxima;
  R19 the density field of §3.4 covers one state row (the d_state values of one (head, channel)):
      K = round(sqrt(4 d_state)) (23 for 128, App. D), value i owns cells floor(i K^2/N) up to
      floor((i+1) K^2/N) of the K x K field in raster order; mu and sigma are the row's mean and
      population standard deviation (fp32, summed in element order); x = clamp((s - (mu - 3 sigma))
      / (6 sigma), 0, 1) is taken to 8 bits, t = rint(255 x); the first-order sigma-delta runs over
      the cells in raster order with an int8 error e: v = e + t, bit = (v >= 128), e = v - 255 bit;
      the readout is mu - 3 sigma + 6 sigma * popcount(value's cells) / cells. A row with sigma = 0
      reads back as mu.
  R20 the 17-level scaffold (the pre-binarisation grid of §3.1 Eq. (1), K_w = 16) is stored as the
      level index k = round(clamp((w + 1)/2, 0, 1) * 16) in [0, 16] (round half to even, as
      torch.round), weight value (k - 8)/8 = 2k/16 - 1 times the row's fp16 scale (as in R1); the
      5-bit index sits in five bit planes, plane b holding bit b of k in the 1-bit layout of R2;
      the scaffold sum acc = sum_k (k - 8) q_k is an exact integer and y = s*sc*acc/8 + the
      low-rank term of R5.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------- packing
def unpack_signs(packed: np.ndarray, n_in: int) -> np.ndarray:
    """[n_out][n_in/8] uint8 -> int8 +-1 [n_out][n_in]; bit k%8 of byte k/8, 1 -> +1 (R2)."""
    bits = np.unpackbits(np.ascontiguousarray(packed, dtype=np.uint8), axis=1, bitorder="little")
    return bits[:, :n_in].astype(np.int8) * 2 - 1


# ----------------------------------------------------------------------------- quantizer
def quantize_token(u) -> tuple:
    """Per-token symmetric int8 quantizer (R4), decided in fp32.

    Returns (q int8 [K], s float32). Input is taken as fp32 values.
    """
    u = np.asarray(u, dtype=F32)
    a = F32(np.max(np.abs(u))) if u.size else F32(0)
    if a == F32(0):
        return np.zeros(u.shape, np.int8), F32(0)
    inv = F32(127) / a                      # IEEE fp32 division
    v = (u * inv).astype(F32)               # IEEE fp32 product
    q = np.clip(np.rint(v), -127, 127).astype(np.int8)   # rint: round half to even
    s = F32(a / F32(127))
    return q, s


# ----------------------------------------------------------------------------- elementwise
def silu(v):
    v = np.asarray(v, F64)
    return v / (1.0 + np.exp(-v))


def softplus(v):
    v = np.asarray(v, F64)
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def rmsnorm(h, w, eps: float):
    """h * (mean(h^2) + eps)^-1/2 * w over the last axis, fp64."""
    h = np.asarray(h, F64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * np.asarray(w, F64)


def gated_rmsnorm(y, z, w, eps: float):
    """norm(y * silu(z)) * w  ([DF-SSM] App. B Table 12: gate first, then normalise)."""
    g = np.asarray(y, F64) * silu(z)
    return rmsnorm(g, w, eps), g


# ----------------------------------------------------------------------------- projection
def project(q: np.ndarray, s, P, dense_sign: Optional[np.ndarray] = None) -> tuple:
    """One DF-SSM projection of one token ([DF-SSM] §3.2 Eq. (3), §3.3; R1, R5).

    q int8 [n_in], s fp32 -> (y fp64 [n_out], acc int64 [n_out], t int64 [rank]) with
      acc[n] = sum_k sgn[n,k] q[k]                      (exact integer)
      t[j]   = sum_k L_dn[j,k] q[k]                     (exact integer)
      y[n]   = s*sc[n]*acc[n] + us[n] * sum_j L_up[n,j] * ds[j] * s * t[j]
    """
    sgn = unpack_signs(P.sign, P.n_in) if dense_sign is None else dense_sign
    qf = np.asarray(q, F64)
    # every partial sum is an integer below 2^53, so fp64 products and sums are exact
    acc = sgn.astype(F64) @ qf
    t = np.asarray(P.lora_dn, F64) @ qf
    s64 = F64(F32(s))
    sc = np.asarray(P.row_scale, np.float16).astype(F64)
    v = np.asarray(P.dn_scale, F64) * s64 * t
    y = s64 * sc * acc + np.asarray(P.up_scale, F64) * (np.asarray(P.lora_up, F64) @ v)
    return y, acc.astype(np.int64), t.astype(np.int64)


def project_tokens(q: np.ndarray, s, P, dense_sign: Optional[np.ndarray] = None) -> tuple:
    """project() for many tokens at once: q int8 [M][n_in], s [M] -> (y [M][n_out], acc, t).
    The same definition evaluated with one matrix product per factor (every token is independent)."""
    sgn = unpack_signs(P.sign, P.n_in) if dense_sign is None else dense_sign
    qf = np.asarray(q, F64)
    acc = qf @ sgn.astype(F64).T
    t = qf @ np.asarray(P.lora_dn, F64).T
    s64 = np.asarray(s, np.float32).astype(F64)[:, None]
    sc = np.asarray(P.row_scale, np.float16).astype(F64)[None, :]
    v = np.asarray(P.dn_scale, F64)[None, :] * s64 * t
    y = s64 * sc * acc + np.asarray(P.up_scale, F64)[None, :] * (v @ np.asarray(P.lora_up, F64).T)
    return y, acc.astype(np.int64), t.astype(np.int64)


# ----------------------------------------------------------------------------- conv + ssm
def conv_step(conv_state, xbc, w, b):
    """Depthwise causal conv, one step (R17).

    conv_state [C][W-1] (oldest first, pre-activation), xbc [C] -> (silu(v) [C], new state)
    with v[c] = b[c] + sum_k w[c,k] * win[c,k],  win = [state | xbc].
    """
    win = np.concatenate([np.asarray(conv_state, F64), np.asarray(xbc, F64)[:, None]], axis=1)
    v = np.asarray(b, F64) + np.sum(np.asarray(w, F64) * win, axis=1)
    return silu(v), win[:, 1:]


def ssm_step(S, x, Bm, Cm, dt, A, D, ngroups: int):
    """Selective-state update and readout for one token (App. B Table 12; [SSD]; R14).

    S [H][P][N], x [H*P], Bm/Cm [G][N], dt [H] (already softplus'd), A [H] (negative), D [H]
      S <- exp(dt*A) S + (dt x) (x) B ;  y = S . C + D x
    """
    S = np.asarray(S, F64)
    H, P, N = S.shape
    grp = (np.arange(H) * ngroups) // H
    Bh = np.asarray(Bm, F64)[grp]                       # [H][N]
    Ch = np.asarray(Cm, F64)[grp]
    xh = np.asarray(x, F64).reshape(H, P)
    dt = np.asarray(dt, F64)
    dA = np.exp(dt * np.asarray(A, F64))
    S_new = dA[:, None, None] * S + (dt[:, None] * xh)[:, :, None] * Bh[:, None, :]
    y = np.sum(S_new * Ch[:, None, :], axis=2) + np.asarray(D, F64)[:, None] * xh
    return y.reshape(H * P), S_new


# ----------------------------------------------------------------------------- layer
@dataclass
class Taps:
    """Intermediate values of one token through one layer (the tap contract of the C ABI)."""
    in_u: np.ndarray
    in_q: np.ndarray
    in_s: np.float32
    in_acc: np.ndarray
    in_t: np.ndarray
    out_u: np.ndarray
    out_q: np.ndarray
    out_s: np.float32
    out_acc: np.ndarray
    out_t: np.ndarray


def layer_decode(h, W, conv_state, ssm_state, force: Optional[dict] = None,
                 dense: Optional[dict] = None):
    """One decode step of one DF-SSM Mamba-2 layer for ONE token (batch rows are independent).

    h fp [d_model]; W: weights (synth.LayerWeights layout); conv_state [C][W-1]; ssm_state
    [H][P][N]. Returns (h_out fp64 [d_model], conv_state', ssm_state', Taps).

    ``force`` may hold 'in_q','in_s','out_q','out_s': codes decided elsewhere (from the GPU's
    own fp32 u) that replace this function's quantizer output, so that the float arithmetic
    downstream of a code decision can be compared without code-flip noise. The caller must
    check separately that those codes equal quantize_token(the other side's u).
    """
    dm = W.dims
    E, H, P, N, G = dm.d_inner, dm.nheads, dm.headdim, dm.d_state, dm.ngroups
    Cd = dm.conv_dim
    # pre-norm and quantizer (R12, R4)
    u = rmsnorm(h, W.norm_w, dm.eps).astype(F32)
    q, s = quantize_token(u)
    if force is not None and "in_q" in force:
        q, s = np.asarray(force["in_q"], np.int8), F32(force["in_s"])
    Y, acc, t = project(q, s, W.in_proj, None if dense is None else dense.get("in"))
    # split [z | x B C | dt | pad] (R11)
    z = Y[:E]
    xbc = Y[E:E + Cd]
    dt_raw = Y[E + Cd:E + Cd + H]
    xbc_act, conv_new = conv_step(conv_state, xbc, W.conv_w, W.conv_b)
    x = xbc_act[:E]
    Bm = xbc_act[E:E + G * N].reshape(G, N)
    Cm = xbc_act[E + G * N:E + 2 * G * N].reshape(G, N)
    dt = softplus(dt_raw + np.asarray(W.dt_bias, F64))
    A = -np.exp(np.asarray(W.A_log, F64))
    y, ssm_new = ssm_step(ssm_state, x, Bm, Cm, dt, A, W.D, G)
    u2_64, _ = gated_rmsnorm(y, z, W.gnorm_w, dm.eps)
    u2 = u2_64.astype(F32)
    q2, s2 = quantize_token(u2)
    if force is not None and "out_q" in force:
        q2, s2 = np.asarray(force["out_q"], np.int8), F32(force["out_s"])
    o, acc2, t2 = project(q2, s2, W.out_proj, None if dense is None else dense.get("out"))
    h_out = np.asarray(h, F64) + o
    return h_out, conv_new, ssm_new, Taps(u, q, s, acc, t, u2, q2, s2, acc2, t2)


def dense_signs(W) -> dict:
    """Unpacked +-1 scaffolds of one layer, to avoid re-unpacking across many steps."""
    return {"in": unpack_signs(W.in_proj.sign, W.in_proj.n_in),
            "out": unpack_signs(W.out_proj.sign, W.out_proj.n_in)}


def layer_decode_steps(xs, W, conv_state, ssm_state):
    """xs [T][d_model] fed one token per step from the given state (single layer, no feedback).

    Returns (outs [T][d_model] fp64, conv_state, ssm_state, taps list)."""
    dense = dense_signs(W)
    cs, ss = np.asarray(conv_state, F64), np.asarray(ssm_state, F64)
    outs, taps = [], []
    for x in xs:
        o, cs, ss, tp = layer_decode(x, W, cs, ss, dense=dense)
        outs.append(o)
        taps.append(tp)
    return np.stack(outs), cs, ss, taps


def layer_prefill(xs, W, conv_state, ssm_state):
    """Prefill of L tokens, DEFINED as L sequential decode steps from the given state.

    Quantization is per token, so this is the method's exact semantics; the chunked scan a
    prefill kernel uses is an evaluation order of the same result (see ssd_chunked)."""
    return layer_decode_steps(xs, W, conv_state, ssm_state)


def layer_tokens(xs, W, conv_state, ssm_state, force: Optional[dict] = None, dense: Optional[dict] = None,
                 codec_chunk: Optional[int] = None):
    """layer_decode_steps evaluated stage by stage over a sequence xs [T][d_model].

    Stage k of token t needs only stage k-1 of tokens <= t, so running each stage over all T
    tokens before the next (projections as one matrix product, conv and recurrence as loops over
    t) gives the sequential-decode result. ``force`` may hold per-token arrays 'in_q' [T][D],
    'in_s' [T], 'out_q' [T][E], 'out_s' [T] (see layer_decode).
    With ``codec_chunk`` = Q (DF-SSD, [DF-SSM] §3.4 / App. D), the SSM state entering every chunk
    of Q tokens after the first passes through the density field codec, as in
    ssd_chunked(codec=True); ``force['state_in']`` [n_chunks][H][P][N] may then replace the coded
    state entering chunk c >= 1 (code forcing of the codec's decisions). The taps then also hold
    'state_pre' and 'state_in' [n_chunks][H][P][N] (chunk 0: the initial state) and the SSM
    inputs 'x' [T][E], 'dt' [T][H], 'B', 'C' [T][G][N].
    Returns (outs [T][d_model], conv_state, ssm_state, taps dict of arrays [T][...])."""
    dm = W.dims
    E, H, N, G = dm.d_inner, dm.nheads, dm.d_state, dm.ngroups
    Cd = dm.conv_dim
    xs = np.asarray(xs, F64)
    T = xs.shape[0]
    dense = dense_signs(W) if dense is None else dense
    u = rmsnorm(xs, W.norm_w, dm.eps).astype(F32)
    q = np.empty((T, dm.d_model), np.int8)
    s = np.empty(T, F32)
    for t in range(T):
        q[t], s[t] = quantize_token(u[t])
    if force is not None and "in_q" in force:
        q, s = np.asarray(force["in_q"], np.int8), np.asarray(force["in_s"], F32)
    Y, acc, tt = project_tokens(q, s, W.in_proj, dense["in"])
    z = Y[:, :E]
    dt = softplus(Y[:, E + Cd:E + Cd + H] + np.asarray(W.dt_bias, F64))
    A = -np.exp(np.asarray(W.A_log, F64))
    cs, ss = np.asarray(conv_state, F64), np.asarray(ssm_state, F64)
    y = np.empty((T, E))
    pre, ent, xs_in, Bs, Cs = [], [], np.empty((T, E)), np.empty((T, G, N)), np.empty((T, G, N))
    for t in range(T):
        if codec_chunk is not None and t % codec_chunk == 0:
            c = t // codec_chunk
            pre.append(ss.copy())
            if c > 0:
                if force is not None and "state_in" in force:
                    ss = np.asarray(force["state_in"][c], F64)
                else:
                    ss = state_codec_roundtrip(ss.astype(F32))
            ent.append(ss.copy())
        xbc_act, cs = conv_step(cs, Y[t, E:E + Cd], W.conv_w, W.conv_b)
        Bm = xbc_act[E:E + G * N].reshape(G, N)
        Cm = xbc_act[E + G * N:E + 2 * G * N].reshape(G, N)
        xs_in[t], Bs[t], Cs[t] = xbc_act[:E], Bm, Cm
        y[t], ss = ssm_step(ss, xbc_act[:E], Bm, Cm, dt[t], A, W.D, G)
    u2 = gated_rmsnorm(y, z, W.gnorm_w, dm.eps)[0].astype(F32)
    q2 = np.empty((T, E), np.int8)
    s2 = np.empty(T, F32)
    for t in range(T):
        q2[t], s2[t] = quantize_token(u2[t])
    if force is not None and "out_q" in force:
        q2, s2 = np.asarray(force["out_q"], np.int8), np.asarray(force["out_s"], F32)
    o, acc2, t2 = project_tokens(q2, s2, W.out_proj, dense["out"])
    taps = dict(in_u=u, in_q=q, in_s=s, in_acc=acc, in_t=tt, out_u=u2, out_q=q2, out_s=s2, out_acc=acc2, out_t=t2)
    if codec_chunk is not None:
        taps.update(state_pre=np.stack(pre), state_in=np.stack(ent), x=xs_in, dt=dt, B=Bs, C=Cs)
    return xs + o, cs, ss, taps


def stack_decode(x0, layers, conv_states, ssm_states, n_steps: int, final_w, eps: float,
                 keep_dense: bool = True, on_step=None):
    """Autoregressive-style decode through a stack of layers for one sequence.

    x(0) = x0; for each step t: h = x(t); h = layer_l(h) for l = 0..L-1; y[t] = RMSNorm(h)*final_w;
    x(t+1) = y[t]. Returns (y [n_steps][d_model] fp64, conv_states, ssm_states)."""
    cs = [np.asarray(c, F64) for c in conv_states]
    ss = [np.asarray(s, F64) for s in ssm_states]
    dense = [dense_signs(W) for W in layers] if keep_dense else [None] * len(layers)
    x = np.asarray(x0, F64)
    ys = []
    for t in range(n_steps):
        h = x
        for l, W in enumerate(layers):
            h, cs[l], ss[l], _ = layer_decode(h, W, cs[l], ss[l], dense=dense[l])
        y = rmsnorm(h, final_w, eps)
        ys.append(y)
        x = y
        if on_step is not None:
            on_step(t)
    return np.stack(ys), cs, ss


# ----------------------------------------------------------------------------- SSD chunked scan
def ssm_scan_sequential(xs, dts, A, Bs, Cs, D, S0, ngroups: int):
    """Token-by-token recurrence (ssm_step applied T times). xs [T][H][P], dts [T][H],
    Bs/Cs [T][G][N], S0 [H][P][N] -> (y [T][H][P], S_T)."""
    S = np.asarray(S0, F64)
    T, H, P = np.shape(xs)
    ys = np.empty((T, H, P))
    for t in range(T):
        y, S = ssm_step(S, np.asarray(xs[t]).reshape(-1), Bs[t], Cs[t], dts[t], A, D, ngroups)
        ys[t] = y.reshape(H, P)
    return ys, S


def ssd_chunked(xs, dts, A, Bs, Cs, D, S0, ngroups: int, chunk: int, codec: bool = False):
    """Chunked evaluation of the same recurrence ([SSD] state-space-duality block form).

    Within a chunk, with Lam_t = sum_{tau <= t in chunk} dt_tau A (per head):
      y_t = sum_{s<=t} exp(Lam_t - Lam_s) (C_t . B_s) dt_s x_s          (intra-chunk)
          + exp(Lam_t) C_t . S_prev                                      (carried state)
          + D x_t
      S_end = exp(Lam_end) S_prev + sum_s exp(Lam_end - Lam_s) dt_s x_s (x) B_s
    Exponentials are always of differences of Lam (never ratios of exponentials).
    With codec, the state carried into every chunk after the first passes through the density
    field codec first (DF-SSD: the codec at chunk boundaries, [DF-SSM] §3.4, App. D)."""
    xs = np.asarray(xs, F64)
    dts = np.asarray(dts, F64)
    A = np.asarray(A, F64)
    T, H, P = xs.shape
    grp = (np.arange(H) * ngroups) // H
    Bh = np.asarray(Bs, F64)[:, grp, :]                  # [T][H][N]
    Ch = np.asarray(Cs, F64)[:, grp, :]
    S = np.asarray(S0, F64).copy()
    ys = np.empty((T, H, P))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        if codec and c0 > 0:
            S = state_codec_roundtrip(S.astype(F32))
        a = dts[c0:c1] * A[None, :]                      # [Q][H]
        lam = np.cumsum(a, axis=0)                       # inclusive
        Q = c1 - c0
        tri = np.tril(np.ones((Q, Q), bool))
        for h in range(H):
            CB = Ch[c0:c1, h, :] @ Bh[c0:c1, h, :].T     # [Q][Q]  (t, s)
            dec = np.where(tri, np.exp(np.where(tri, lam[:, h][:, None] - lam[:, h][None, :], 0.0)), 0.0)
            M = CB * dec * dts[c0:c1, h][None, :]
            y_diag = M @ xs[c0:c1, h, :]                  # [Q][P]
            y_off = np.exp(lam[:, h])[:, None] * (Ch[c0:c1, h, :] @ S[h].T)
            ys[c0:c1, h, :] = y_diag + y_off + np.asarray(D, F64)[h] * xs[c0:c1, h, :]
            w = np.exp(lam[-1, h] - lam[:, h]) * dts[c0:c1, h]     # [Q]
            S_loc = (xs[c0:c1, h, :] * w[:, None]).T @ Bh[c0:c1, h, :]   # [P][N]
            S[h] = np.exp(lam[-1, h]) * S[h] + S_loc
    return ys, S


def ssd_quadratic(xs, dts, A, Bs, Cs, D, ngroups: int):
    """The SSD masked-attention form from a zero state: y = (L o C B^T) (dt x) + D x with
    L[t,s] = exp(sum_{s<tau<=t} dt_tau A) for s <= t. O(T^2); for short sequences."""
    xs = np.asarray(xs, F64)
    dts = np.asarray(dts, F64)
    T, H, P = xs.shape
    grp = (np.arange(H) * ngroups) // H
    ys = np.empty((T, H, P))
    for h in range(H):
        Bh = np.asarray(Bs, F64)[:, grp[h], :]
        Ch = np.asarray(Cs, F64)[:, grp[h], :]
        Lmat = np.zeros((T, T))
        for t in range(T):
            for s in range(t + 1):
                Lmat[t, s] = np.exp(np.sum(dts[s + 1:t + 1, h]) * A[h])
        M = Lmat * (Ch @ Bh.T) * dts[:, h][None, :]
        ys[:, h, :] = M @ xs[:, h, :] + D[h] * xs[:, h, :]
    return ys


# ----------------------------------------------------------------------------- byte model
def table1_bytes(d_model: int, d_inner: int, n_in_proj: int, n_layers: int, rank: int,
                 vocab: Optional[int] = None) -> dict:
    """Storage of the model parts [DF-SSM] §3.3 Table 1 counts: 1 bit per scaffold weight,
    1 byte per int8 low-rank weight, 1 byte per int8 embedding weight."""
    scaffold_bits = n_layers * (n_in_proj * d_model + d_model * d_inner)
    lora = n_layers * (rank * d_model + n_in_proj * rank + rank * d_inner + d_model * rank)
    out = {"scaffold": scaffold_bits // 8, "lora": lora}
    if vocab is not None:
        out["embedding"] = vocab * d_model
    return out


# ----------------------------------------------------------------------------- embedding + LM head
def embed(tokens, codes, row_scale):
    """[DF-SSM] §3.3: the int8 embedding with a per-row scale. tokens [B] -> x [B][d_model] fp64,
    x[b] = row_scale[tokens[b]] * codes[tokens[b]]."""
    tok = np.asarray(tokens, np.int64)
    return np.asarray(row_scale, F64)[tok][:, None] * np.asarray(codes, F64)[tok]


def lm_head(y, codes, row_scale, chunk_rows: int = 4096):
    """The tied head over the embedding rows (Table 1) for one token y [d_model] (R18).

    Returns (logits fp64 [vocab], acc int64 [vocab], q int8 [d_model], s fp32):
      (q, s) = quantize_token(y);  acc[v] = sum_k codes[v,k] q[k] (exact);  logits = s*row_scale*acc.
    The rows are taken in blocks only to bound memory; every block product is exact in fp64."""
    q, s = quantize_token(y)
    qf = np.asarray(q, F64)
    V = codes.shape[0]
    acc = np.empty(V, np.int64)
    for r0 in range(0, V, chunk_rows):
        acc[r0:r0 + chunk_rows] = (np.asarray(codes[r0:r0 + chunk_rows], F64) @ qf).astype(np.int64)
    logits = F64(s) * np.asarray(row_scale, F64) * acc.astype(F64)
    return logits, acc, q, s


def argmax_first(v) -> int:
    """Index of the largest value, the smallest such index when several are equal (R18)."""
    v = np.asarray(v)
    return int(np.flatnonzero(v == v.max())[0])


# ----------------------------------------------------------------------------- density field state codec
def codec_field_side(d_state: int) -> int:
    """K of the K x K field: K^2 ~ 4 d_state ([DF-SSM] App. D), K = round(sqrt(4 d_state))."""
    return int(round((4 * d_state) ** 0.5))


def codec_cells(d_state: int) -> np.ndarray:
    """cells[i] .. cells[i+1]: the cells of value i in raster order (R19)."""
    K2 = codec_field_side(d_state) ** 2
    return np.array([(i * K2) // d_state for i in range(d_state + 1)], np.int64)


def state_codec_stats(row) -> tuple:
    """(mu, sigma) of one state row in fp32, summed in element order (R19)."""
    r = np.asarray(row, F32)
    acc = F32(0)
    for v in r:
        acc = F32(acc + v)
    mu = F32(acc / F32(r.size))
    acc2 = F32(0)
    for v in r:
        d = F32(v - mu)
        acc2 = F32(acc2 + F32(d * d))
    sigma = F32(np.sqrt(F32(acc2 / F32(r.size))))
    return mu, sigma


def state_codec_encode_row(row, mu=None, sigma=None) -> tuple:
    """Density field of one state row ([DF-SSM] §3.4 steps 1-3, R19): returns (bits uint8 [K*K], mu,
    sigma). mu/sigma may be given (e.g. decided elsewhere in the same fp32 arithmetic)."""
    r = np.asarray(row, F32)
    N = r.size
    if mu is None:
        mu, sigma = state_codec_stats(r)
    mu, sigma = F32(mu), F32(sigma)
    cells = codec_cells(N)
    bits = np.zeros(cells[-1], np.uint8)
    if sigma == F32(0):
        return bits, mu, sigma
    lo = F32(mu - F32(F32(3) * sigma))
    span = F32(F32(6) * sigma)
    x = np.clip(((r - lo).astype(F32) / span).astype(F32), F32(0), F32(1))   # step 1: mu +- 3 sigma -> [0, 1]
    t = np.rint((x * F32(255)).astype(F32)).astype(np.int64)                   # 8-bit target per value
    e = 0                                                                       # 8-bit error accumulator
    for i in range(N):
        for c in range(cells[i], cells[i + 1]):                                # step 2: first-order sigma-delta
            v = e + int(t[i])
            b = 1 if v >= 128 else 0                                            # step 3: threshold at 0.5
            e = v - 255 * b
            bits[c] = b
    return bits, mu, sigma


def state_codec_decode_row(bits, mu, sigma, d_state: int) -> np.ndarray:
    """Readout ([DF-SSM] §3.4 step 4): popcount density of each value's cells, back through the
    normalisation. Returns fp64 [d_state]."""
    cells = codec_cells(d_state)
    mu, sigma = F64(F32(mu)), F64(F32(sigma))
    if sigma == 0:
        return np.full(d_state, mu)
    dens = np.array([np.sum(bits[cells[i]:cells[i + 1]]) / (cells[i + 1] - cells[i]) for i in range(d_state)])
    return (mu - 3 * sigma) + 6 * sigma * dens


def state_codec_roundtrip(S) -> np.ndarray:
    """Encode then decode every row of a state [..., d_state] (fp64 out)."""
    S = np.asarray(S, F32)
    flat = S.reshape(-1, S.shape[-1])
    out = np.empty(flat.shape)
    for k in range(flat.shape[0]):
        bits, mu, sigma = state_codec_encode_row(flat[k])
        out[k] = state_codec_decode_row(bits, mu, sigma, flat.shape[1])
    return out.reshape(S.shape)


# ----------------------------------------------------------------------------- 17-level DFW scaffold
DFW_KW = 16                 # Eq. (1): K_w = 16 -> 17 levels
DFW_PLANES = 5              # bits of the level index 0..16


def dfw_quantize(w, K_w: int = DFW_KW) -> tuple:
    """[DF-SSM] §3.1 Eq. (1): w_q = round(clamp((w + 1)/2, 0, 1) K_w) / K_w * 2 - 1 (R20).
    Returns (w_q fp64, level index k int64 in [0, K_w]); round is half to even, in fp64."""
    w = np.asarray(w, F64)
    k = np.rint(np.clip((w + 1.0) / 2.0, 0.0, 1.0) * K_w)
    return k / K_w * 2.0 - 1.0, k.astype(np.int64)


def dfw_unpack_planes(planes: np.ndarray, n_in: int) -> np.ndarray:
    """[5][n_out][n_in/8] uint8 bit planes -> level index k int64 [n_out][n_in] (R20, layout R2)."""
    planes = np.asarray(planes, np.uint8)
    k = np.zeros((planes.shape[1], n_in), np.int64)
    for b in range(planes.shape[0]):
        bits = np.unpackbits(planes[b], axis=1, bitorder="little")[:, :n_in].astype(np.int64)
        k += bits << b
    return k


def project_dfw(q: np.ndarray, s, P, k: Optional[np.ndarray] = None) -> tuple:
    """One projection of one token with the 17-level scaffold ([DF-SSM] §3.2 Eq. (3), R20, R5).

    q int8 [n_in], s fp32; P has planes [5][n_out][n_in/8], row_scale, lora_dn, dn_scale, lora_up,
    up_scale. Returns (y fp64 [n_out], acc int64 [n_out], t int64 [rank]):
      acc[n] = sum_k (k[n,i] - 8) q[i]      (exact integer; weight value (k - 8)/8)
      t[j]   = sum_i L_dn[j,i] q[i]
      y[n]   = s*sc[n]*acc[n]/8 + us[n] * sum_j L_up[n,j] * ds[j] * s * t[j]
    """
    lev = dfw_unpack_planes(P.planes, P.n_in) if k is None else np.asarray(k, np.int64)
    qf = np.asarray(q, F64)
    acc = (lev - 8).astype(F64) @ qf          # integers below 2^53: exact
    t = np.asarray(P.lora_dn, F64) @ qf
    s64 = F64(F32(s))
    sc = np.asarray(P.row_scale, np.float16).astype(F64)
    v = np.asarray(P.dn_scale, F64) * s64 * t
    y = s64 * sc * acc / 8.0 + np.asarray(P.up_scale, F64) * (np.asarray(P.lora_up, F64) @ v)
    return y, acc.astype(np.int64), t.astype(np.int64)
