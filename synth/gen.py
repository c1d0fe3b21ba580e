"""Seeded generators for DF-SSM layer weights, decode/prefill inputs and initial states.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed, layer, tensor_id]))``
so that a given (seed, layer, tensor) is the same array whichever workload asks for it: layer 0
of the 48-layer stack is exactly the single-layer workload's layer.

Value distributions (the synthetic stand-in for the trained DF-SSM model of arXiv 2606.10932,
whose weights are not available):

* scaffold signs: uniform random bytes, i.e. i.i.d. Bernoulli(0.5) bits, one bit per weight
  (the paper's Table 1 counts exactly one bit per scaffold weight);
* per-output-row scaffold scale: U[0.01, 0.05] rounded to IEEE fp16;
* int8 low-rank factors: integers uniform in [-127, 127]; their scales 1e-3 (a per-tensor value
  broadcast to the per-channel vectors of the paper's §3.3), or U[0.5e-3, 1.5e-3] per channel
  when ``per_channel_lora`` is set;
* A_log ~ U[0, ln 16] (so A = -exp(A_log) lies in [-16, -1]); D ~ N(0, 1);
* dt_bias is chosen so that softplus(dt_bias) is log-uniform in [1e-3, 1e-1];
* depthwise conv taps and bias ~ U[-0.5, 0.5];
* norm weights 1, or U[0.5, 1.5] when ``random_norms`` is set;
* token inputs ~ N(0, 1) fp32 (optionally rounded to bf16); initial states zero or N(0, std);
* int8 embedding (tied LM head): 50,280 rows (Table 1's 103 MB at d_model 2048), codes uniform in
  [-127, 127], per-row scales U[2e-4, 1e-3]; token ids uniform.

No function here computes any part of the layer: no norm, quantizer, projection, convolution,
gate or recurrence.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Dims:
    """Mamba-2 layer shape. ``n_in_proj`` may exceed the natural width (padding rows)."""
    d_model: int
    d_inner: int
    d_state: int
    headdim: int
    ngroups: int
    d_conv: int
    n_in_proj: int
    rank_in: int
    rank_out: int
    eps: float = 1e-5

    @property
    def nheads(self) -> int:
        return self.d_inner // self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.d_state

    @property
    def n_in_natural(self) -> int:
        """Rows the layer consumes: z | x | B | C | dt."""
        return 2 * self.d_inner + 2 * self.ngroups * self.d_state + self.nheads


# The two layer shapes the workloads use.
DIMS = {
    # tiny layer: d_model 256, expand 2, d_state 16, 8 heads of 64; in_proj written 256->1072
    # (1064 natural rows + 8 seeded padding rows), rank 8
    "tiny": Dims(d_model=256, d_inner=512, d_state=16, headdim=64, ngroups=1, d_conv=4,
                 n_in_proj=1072, rank_in=8, rank_out=8),
    # Mamba-2 1.3B layer: d_model 2048, d_inner 4096, d_state 128, 64 heads of 64, rank 32
    "1p3b": Dims(d_model=2048, d_inner=4096, d_state=128, headdim=64, ngroups=1, d_conv=4,
                 n_in_proj=8512, rank_in=32, rank_out=32),
}

# The workloads the tests and the benchmark run (each is a shape + step count + batch).
WORKLOADS = {
    "tiny_layer_decode16": dict(dims="tiny", n_layers=1, batch=1, steps=16),
    "layer1p3b_decode256": dict(dims="1p3b", n_layers=1, batch=1, steps=256),
    "stack48_1p3b_b1_decode512": dict(dims="1p3b", n_layers=48, batch=1, steps=512),
    "stack48_1p3b_prefill2048": dict(dims="1p3b", n_layers=48, batch=1, seqlen=2048,
                                     chunk=256, decode_steps=16, bf16_inputs=True),
    "stack48_1p3b_b64_decode128": dict(dims="1p3b", n_layers=48, batch=64, steps=128,
                                       state_std=0.1),
}

# tensor ids inside one layer's seed stream
_T = dict(in_sign=0, in_scale=1, in_dn=2, in_dn_scale=3, in_up=4, in_up_scale=5,
          out_sign=10, out_scale=11, out_dn=12, out_dn_scale=13, out_up=14, out_up_scale=15,
          conv_w=20, conv_b=21, dt0=22, A_log=23, D=24, norm_w=25, gnorm_w=26)
_INPUT_LAYER_KEY = 100000   # seed-stream "layer" slot used for token inputs
_STATE_TENSOR_BASE = 50     # tensor ids 50/51 hold conv/ssm initial states


def _rng(seed: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, tensor]))


@dataclass
class ProjWeights:
    """One DF-SSM projection: 1-bit scaffold + fp16 row scale + int8 low-rank factors.

    sign      uint8  [n_out][n_in/8]  bit (k % 8) of byte k/8 is weight k of the row; 1 -> +1, 0 -> -1
    row_scale fp16   [n_out]
    lora_dn   int8   [rank][n_in]     (the paper's W_B, rank x d_in)
    dn_scale  fp32   [rank]
    lora_up   int8   [n_out][rank]    (the paper's W_A, d_out x rank)
    up_scale  fp32   [n_out]
    """
    sign: np.ndarray
    row_scale: np.ndarray
    lora_dn: np.ndarray
    dn_scale: np.ndarray
    lora_up: np.ndarray
    up_scale: np.ndarray

    @property
    def n_out(self) -> int:
        return self.sign.shape[0]

    @property
    def n_in(self) -> int:
        return self.sign.shape[1] * 8

    @property
    def rank(self) -> int:
        return self.lora_dn.shape[0]


@dataclass
class LayerWeights:
    dims: Dims
    in_proj: ProjWeights
    out_proj: ProjWeights
    conv_w: np.ndarray      # fp32 [conv_dim][d_conv]; column d_conv-1 multiplies the newest input
    conv_b: np.ndarray      # fp32 [conv_dim]
    dt_bias: np.ndarray     # fp32 [nheads]
    A_log: np.ndarray       # fp32 [nheads]
    D: np.ndarray           # fp32 [nheads]
    norm_w: np.ndarray      # fp32 [d_model]  pre-norm weight
    gnorm_w: np.ndarray     # fp32 [d_inner]  gated-norm weight
    extra: dict = field(default_factory=dict)


def _proj(rng_for, prefix: str, n_out: int, n_in: int, rank: int, per_channel: bool) -> ProjWeights:
    sign = rng_for(prefix + "_sign").integers(0, 256, size=(n_out, n_in // 8), dtype=np.uint8)
    row_scale = rng_for(prefix + "_scale").uniform(0.01, 0.05, size=n_out).astype(np.float16)
    lora_dn = rng_for(prefix + "_dn").integers(-127, 128, size=(rank, n_in)).astype(np.int8)
    lora_up = rng_for(prefix + "_up").integers(-127, 128, size=(n_out, rank)).astype(np.int8)
    if per_channel:
        dn_scale = rng_for(prefix + "_dn_scale").uniform(0.5e-3, 1.5e-3, size=rank).astype(np.float32)
        up_scale = rng_for(prefix + "_up_scale").uniform(0.5e-3, 1.5e-3, size=n_out).astype(np.float32)
    else:
        dn_scale = np.full(rank, 1e-3, dtype=np.float32)
        up_scale = np.full(n_out, 1e-3, dtype=np.float32)
    return ProjWeights(sign, row_scale, lora_dn, dn_scale, lora_up, up_scale)


def layer_weights(dims: Dims, layer: int = 0, seed: int = 0, *, random_norms: bool = False,
                  per_channel_lora: bool = False) -> LayerWeights:
    """Seeded weights of one layer. Same (seed, layer) -> same bytes."""
    if dims.d_model % 8 or dims.d_inner % 8:
        raise ValueError("d_model and d_inner must be multiples of 8 (bit packing)")

    def rng_for(name: str) -> np.random.Generator:
        return _rng(seed, layer, _T[name])

    H, E, D_ = dims.nheads, dims.d_inner, dims.d_model
    in_proj = _proj(rng_for, "in", dims.n_in_proj, D_, dims.rank_in, per_channel_lora)
    out_proj = _proj(rng_for, "out", D_, E, dims.rank_out, per_channel_lora)
    conv_w = rng_for("conv_w").uniform(-0.5, 0.5, size=(dims.conv_dim, dims.d_conv)).astype(np.float32)
    conv_b = rng_for("conv_b").uniform(-0.5, 0.5, size=dims.conv_dim).astype(np.float32)
    dt0 = np.exp(rng_for("dt0").uniform(math.log(1e-3), math.log(1e-1), size=H))
    # inverse of softplus, so that softplus(dt_bias) == dt0 (distribution of the bias only)
    dt_bias = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    A_log = rng_for("A_log").uniform(0.0, math.log(16.0), size=H).astype(np.float32)
    Dp = rng_for("D").standard_normal(H).astype(np.float32)
    if random_norms:
        norm_w = rng_for("norm_w").uniform(0.5, 1.5, size=D_).astype(np.float32)
        gnorm_w = rng_for("gnorm_w").uniform(0.5, 1.5, size=E).astype(np.float32)
    else:
        norm_w = np.ones(D_, np.float32)
        gnorm_w = np.ones(E, np.float32)
    return LayerWeights(dims, in_proj, out_proj, conv_w, conv_b, dt_bias, A_log, Dp, norm_w, gnorm_w)


def stack_weights(dims: Dims, n_layers: int, seed: int = 0, **kw) -> list:
    return [layer_weights(dims, l, seed, **kw) for l in range(n_layers)]


# tensor ids of the embedding (a "layer" slot of its own)
_EMBED_LAYER_KEY = 200000
VOCAB_1P3B = 50280   # rows of the int8 embedding: 50,280 x 2,048 B = 103 MB (Table 1)


@dataclass
class Embedding:
    """int8 embedding with a per-row fp32 scale, tied to the LM head.

    codes     int8 [vocab][d_model]
    row_scale fp32 [vocab]    (weight[v][k] = codes[v][k] * row_scale[v])
    """
    codes: np.ndarray
    row_scale: np.ndarray

    @property
    def vocab(self) -> int:
        return self.codes.shape[0]


def embedding(dims: Dims, vocab: int = VOCAB_1P3B, seed: int = 0) -> Embedding:
    """Seeded int8 embedding: codes uniform in [-127, 127], per-row scales U[2e-4, 1e-3]."""
    codes = _rng(seed, _EMBED_LAYER_KEY, 0).integers(-127, 128, size=(vocab, dims.d_model)).astype(np.int8)
    scale = _rng(seed, _EMBED_LAYER_KEY, 1).uniform(2e-4, 1e-3, size=vocab).astype(np.float32)
    return Embedding(codes, scale)


def token_ids(batch: int, vocab: int, seed: int = 0, tag: int = 0) -> np.ndarray:
    """Uniform token ids in [0, vocab), int32 [batch]."""
    return _rng(seed, _INPUT_LAYER_KEY, 1000 + tag).integers(0, vocab, size=batch).astype(np.int32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even) and return them as fp32.

    Used to make bf16-valued token inputs; the kernel receives the raw 16-bit patterns.
    NaN/Inf are not produced by the generators and are not handled specially.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def token_inputs(dims: Dims, shape: tuple, seed: int = 0, tag: int = 0, *, bf16: bool = False) -> np.ndarray:
    """N(0,1) fp32 token vectors of shape ``shape + (d_model,)``."""
    x = _rng(seed, _INPUT_LAYER_KEY, tag).standard_normal(tuple(shape) + (dims.d_model,)).astype(np.float32)
    return bf16_round(x) if bf16 else x


def initial_states(dims: Dims, batch: int, layer: int = 0, seed: int = 0, std: float = 0.0):
    """(conv_state [B][conv_dim][d_conv-1], ssm_state [B][H][P][N]) fp32; zeros when std == 0."""
    cshape = (batch, dims.conv_dim, dims.d_conv - 1)
    sshape = (batch, dims.nheads, dims.headdim, dims.d_state)
    if std == 0.0:
        return np.zeros(cshape, np.float32), np.zeros(sshape, np.float32)
    conv = (_rng(seed, layer, _STATE_TENSOR_BASE).standard_normal(cshape) * std).astype(np.float32)
    ssm = (_rng(seed, layer, _STATE_TENSOR_BASE + 1).standard_normal(sshape) * std).astype(np.float32)
    return conv, ssm


@dataclass
class DfwProjWeights:
    """A projection with the 17-level scaffold: 5-bit level index in five bit planes.

    planes    uint8 [5][n_out][n_in/8]  plane b holds bit b of the level index (0..16), each in the
                                        1-bit layout (bit k % 8 of byte k/8)
    row_scale, lora_dn, dn_scale, lora_up, up_scale as in ProjWeights
    """
    planes: np.ndarray
    row_scale: np.ndarray
    lora_dn: np.ndarray
    dn_scale: np.ndarray
    lora_up: np.ndarray
    up_scale: np.ndarray

    @property
    def n_out(self) -> int:
        return self.planes.shape[1]

    @property
    def n_in(self) -> int:
        return self.planes.shape[2] * 8

    @property
    def rank(self) -> int:
        return self.lora_dn.shape[0]


_DFW_LAYER_KEY = 300000


def pack_level_planes(levels: np.ndarray) -> np.ndarray:
    """Level indices int [n_out][n_in] in [0, 16] -> uint8 [5][n_out][n_in/8] bit planes."""
    lv = np.asarray(levels, np.int64)
    return np.stack([np.packbits(((lv >> b) & 1).astype(np.uint8), axis=1, bitorder="little")
                     for b in range(5)])


def dfw_levels(n_out: int, n_in: int, seed: int = 0, tag: int = 0) -> np.ndarray:
    """Seeded level indices, int64 [n_out][n_in]: Binomial(16, 1/2) (the middle levels most) mixed
    with 1/8 uniform over 0..16, so that every one of the 17 levels, the end levels included,
    occurs in any block of a few hundred weights."""
    rng = _rng(seed, _DFW_LAYER_KEY, tag)
    lv = rng.binomial(16, 0.5, size=(n_out, n_in))
    uni = rng.integers(0, 17, size=(n_out, n_in))
    return np.where(rng.random((n_out, n_in)) < 0.125, uni, lv).astype(np.int64)


def dfw_proj(n_out: int, n_in: int, rank: int, seed: int = 0, levels: Optional[np.ndarray] = None) -> DfwProjWeights:
    """Seeded 17-level projection (row scales, LoRA factors and scales drawn as for ProjWeights)."""
    if levels is None:
        levels = dfw_levels(n_out, n_in, seed)
    base = _proj(lambda name: _rng(seed, _DFW_LAYER_KEY + 1, _T.get(name, 0) + 1000),
                 "in", n_out, n_in, rank, per_channel=True)
    return DfwProjWeights(pack_level_planes(levels), base.row_scale, base.lora_dn, base.dn_scale,
                          base.lora_up, base.up_scale)
