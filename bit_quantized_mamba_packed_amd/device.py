"""Torch-side marshalling for libdfssm: device copies of weights/states, tap buffers and thin
wrappers that pass raw device pointers and the current HIP stream to the C ABI.

PyTorch only allocates device memory and provides the stream; all arithmetic of the method
runs in the HIP kernels behind the C ABI.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib as L


def dims_struct(d) -> L.dfssm_dims:
    """dfssm_dims from any object with the Mamba-2 shape attributes (d_model, d_inner, ...)."""
    return L.dfssm_dims(d.d_model, d.d_inner, d.d_state, d.headdim, d.ngroups, d.d_conv,
                        d.n_in_proj, d.rank_in, d.rank_out, float(d.eps))


def _dev(a, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


class DeviceProj:
    def __init__(self, p, device):
        self.sign = _dev(p.sign, device)
        self.row_scale = _dev(np.asarray(p.row_scale, np.float16).view(np.uint16), device)
        self.lora_dn = _dev(p.lora_dn, device)
        self.dn_scale = _dev(np.asarray(p.dn_scale, np.float32), device)
        self.lora_up = _dev(p.lora_up, device)
        self.up_scale = _dev(np.asarray(p.up_scale, np.float32), device)

    def struct(self) -> L.dfssm_proj:
        return L.dfssm_proj(self.sign.data_ptr(), self.row_scale.data_ptr(), self.lora_dn.data_ptr(),
                            self.dn_scale.data_ptr(), self.lora_up.data_ptr(), self.up_scale.data_ptr())


class DeviceLayer:
    """Device-resident weights of one layer (keeps the tensors alive) and their C struct."""

    def __init__(self, lw, device="cuda"):
        self.in_proj = DeviceProj(lw.in_proj, device)
        self.out_proj = DeviceProj(lw.out_proj, device)
        f = lambda a: _dev(np.asarray(a, np.float32), device)
        self.conv_w, self.conv_b = f(lw.conv_w), f(lw.conv_b)
        self.dt_bias, self.A_log, self.D = f(lw.dt_bias), f(lw.A_log), f(lw.D)
        self.norm_w, self.gnorm_w = f(lw.norm_w), f(lw.gnorm_w)
        self.struct = L.dfssm_layer_weights(
            self.in_proj.struct(), self.out_proj.struct(), self.conv_w.data_ptr(), self.conv_b.data_ptr(),
            self.dt_bias.data_ptr(), self.A_log.data_ptr(), self.D.data_ptr(), self.norm_w.data_ptr(),
            self.gnorm_w.data_ptr())


class DeviceState:
    def __init__(self, conv: np.ndarray, ssm: np.ndarray, device="cuda"):
        self.conv = _dev(np.asarray(conv, np.float32), device)
        self.ssm = _dev(np.asarray(ssm, np.float32), device)
        self.struct = L.dfssm_layer_state(self.conv.data_ptr(), self.ssm.data_ptr())

    def load(self, conv: np.ndarray, ssm: np.ndarray) -> None:
        self.conv.copy_(torch.from_numpy(np.asarray(conv, np.float32)))
        self.ssm.copy_(torch.from_numpy(np.asarray(ssm, np.float32)))

    @classmethod
    def from_tensors(cls, conv: torch.Tensor, ssm: torch.Tensor, d, batch: int) -> "DeviceState":
        """A state over existing contiguous fp32 device tensors (e.g. views of one allocation that
        holds a whole stack's states, so that they can be reset with one fill). The tensors must hold
        exactly batch x conv_dim x (d_conv - 1) and batch x nheads x headdim x d_state values."""
        for name, t, n in (("conv", conv, batch * d.conv_dim * (d.d_conv - 1)),
                           ("ssm", ssm, batch * d.nheads * d.headdim * d.d_state)):
            if not t.is_cuda:
                raise ValueError(f"DeviceState.from_tensors: {name} is not a device tensor")
            if not t.is_contiguous() or t.dtype != torch.float32:
                raise ValueError(f"DeviceState.from_tensors: {name} must be contiguous fp32")
            if t.numel() != n:
                raise ValueError(f"DeviceState.from_tensors: {name} holds {t.numel()} values, expected {n}")
        st = cls.__new__(cls)
        st.conv, st.ssm = conv, ssm
        st.struct = L.dfssm_layer_state(conv.data_ptr(), ssm.data_ptr())
        return st


class Taps:
    """Tap buffers for `records` token records (layout [record][...] as include/dfssm.h states)."""

    FIELDS = ("h_in", "in_u", "in_q", "in_s", "in_acc", "in_t", "out_u", "out_q", "out_s", "out_acc", "out_t")

    def __init__(self, d, records: int, device="cuda", fields=None):
        sizes = dict(h_in=(d.d_model, torch.float32), in_u=(d.d_model, torch.float32),
                     in_q=(d.d_model, torch.int8), in_s=(1, torch.float32),
                     in_acc=(d.n_in_proj, torch.int32), in_t=(d.rank_in, torch.int32),
                     out_u=(d.d_inner, torch.float32), out_q=(d.d_inner, torch.int8), out_s=(1, torch.float32),
                     out_acc=(d.d_model, torch.int32), out_t=(d.rank_out, torch.int32))
        fields = self.FIELDS if fields is None else fields
        self.t = {}
        for k in fields:
            n, dt = sizes[k]
            # poison so that unwritten records are visible
            self.t[k] = torch.full((records, n), -7, dtype=dt, device=device) if dt != torch.float32 else \
                torch.full((records, n), float("nan"), dtype=dt, device=device)
        self.struct = L.dfssm_taps(*[(self.t[k].data_ptr() if k in self.t else None) for k in self.FIELDS])

    def numpy(self) -> dict:
        return {k: v.cpu().numpy() for k, v in self.t.items()}


def stream_handle():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace(d, op: int, batch: int, seqlen: int = 0, n_layers: int = 0, device="cuda") -> torch.Tensor:
    n = L.dfssm_workspace_bytes(dims_struct(d), op, batch, seqlen, n_layers)
    if n == 0:
        raise L.DfssmError("dfssm_workspace_bytes: unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def layer_decode(d, layer: DeviceLayer, state: DeviceState, x_in: torch.Tensor, x_out: torch.Tensor,
                 ws: torch.Tensor, taps: Taps = None) -> None:
    batch = x_in.shape[0]
    _need("x_in", x_in, torch.float32, batch * d.d_model)
    _need("x_out", x_out, torch.float32, batch * d.d_model)
    st = L.dfssm_layer_decode(dims_struct(d), layer.struct, state.struct, x_in.data_ptr(), x_out.data_ptr(),
                              batch, ws.data_ptr(), ws.numel(), None if taps is None else taps.struct,
                              stream_handle())
    L.check(st, "dfssm_layer_decode")


def _arrays(layers: list, states: list):
    n = len(layers)
    return (L.dfssm_layer_weights * n)(*[l.struct for l in layers]), (L.dfssm_layer_state * n)(*[s.struct for s in states])


def stack_decode(d, layers: list, states: list, final_w: torch.Tensor, x0: torch.Tensor, y: torch.Tensor,
                 n_steps: int, ws: torch.Tensor, taps: Taps = None, path: int = L.DFSSM_PATH_AUTO,
                 launch: int = L.DFSSM_LAUNCH_COOPERATIVE) -> None:
    """dfssm_stack_decode_ex; the call's status word stays in ws (stack_status reads it)."""
    batch = x0.shape[0]
    _need("x0", x0, torch.float32, batch * d.d_model)
    _need("y", y, torch.float32, n_steps * batch * d.d_model)
    _need("final_w", final_w, torch.float32, d.d_model)
    arr_w, arr_s = _arrays(layers, states)
    opts = L.dfssm_stack_opts(path, launch)
    st = L.dfssm_stack_decode_ex(dims_struct(d), arr_w, arr_s, len(layers), final_w.data_ptr(), x0.data_ptr(),
                                 y.data_ptr(), x0.shape[0], n_steps, ws.data_ptr(), ws.numel(),
                                 None if taps is None else taps.struct, opts, stream_handle())
    L.check(st, "dfssm_stack_decode_ex")


def stack_status(ws: torch.Tensor) -> int:
    """The status word a stack decode left in its workspace (synchronises with the device)."""
    o = L.DFSSM_STACK_STATUS_OFFSET
    return int(ws[o:o + 4].view(torch.int32).item())


def stack_prefill(d, layers: list, states: list, final_w: torch.Tensor, x_in: torch.Tensor, y: torch.Tensor,
                  chunk: int, ws: torch.Tensor, taps: Taps = None, state_codec: bool = False) -> None:
    """x_in [batch][seqlen][d_model] fp32 or bf16 -> y = RMSNorm(stack(x_in)) * final_w, fp32.
    state_codec: DF-SSD in every layer (dfssm_stack_prefill_ex)."""
    arr_w, arr_s = _arrays(layers, states)
    batch, seqlen = x_in.shape[0], x_in.shape[1]
    dtype = L.DFSSM_BF16 if x_in.dtype == torch.bfloat16 else L.DFSSM_F32
    _need("x_in", x_in, torch.bfloat16 if dtype == L.DFSSM_BF16 else torch.float32, batch * seqlen * d.d_model)
    _need("y", y, torch.float32, batch * seqlen * d.d_model)
    _need("final_w", final_w, torch.float32, d.d_model)
    opts = L.dfssm_prefill_opts(1 if state_codec else 0, 0, None, None)
    st = L.dfssm_stack_prefill_ex(dims_struct(d), arr_w, arr_s, len(layers), final_w.data_ptr(), x_in.data_ptr(),
                                  dtype, y.data_ptr(), batch, seqlen, chunk, ws.data_ptr(), ws.numel(),
                                  None if taps is None else taps.struct, opts, stream_handle())
    L.check(st, "dfssm_stack_prefill_ex")


def layer_prefill(d, layer: DeviceLayer, state: DeviceState, x_in: torch.Tensor, x_out: torch.Tensor, chunk: int,
                  ws: torch.Tensor, taps: Taps = None, state_codec: bool = False, chunk_state_pre: torch.Tensor = None,
                  chunk_state_in: torch.Tensor = None) -> None:
    """x_in [batch][seqlen][d_model] fp32 or bf16 (torch.bfloat16 is passed as its bit patterns).
    state_codec: DF-SSD (dfssm_layer_prefill_ex), with optional taps of the chunk-entering states."""
    batch, seqlen = x_in.shape[0], x_in.shape[1]
    dtype = L.DFSSM_BF16 if x_in.dtype == torch.bfloat16 else L.DFSSM_F32
    _need("x_in", x_in, torch.bfloat16 if dtype == L.DFSSM_BF16 else torch.float32, batch * seqlen * d.d_model)
    _need("x_out", x_out, torch.float32, batch * seqlen * d.d_model)
    opts = None
    nch = (seqlen + chunk - 1) // chunk if chunk > 0 else 0
    for name, t in (("chunk_state_pre", chunk_state_pre), ("chunk_state_in", chunk_state_in)):
        if t is not None:
            _need(name, t, torch.float32, nch * batch * d.nheads * d.headdim * d.d_state)
    if state_codec:
        opts = L.dfssm_prefill_opts(1, 0, None if chunk_state_pre is None else chunk_state_pre.data_ptr(),
                                    None if chunk_state_in is None else chunk_state_in.data_ptr())
    st = L.dfssm_layer_prefill_ex(dims_struct(d), layer.struct, state.struct, x_in.data_ptr(), dtype, x_out.data_ptr(),
                                  batch, seqlen, chunk, ws.data_ptr(), ws.numel(),
                                  None if taps is None else taps.struct, opts, stream_handle())
    L.check(st, "dfssm_layer_prefill_ex")


class DeviceEmbedding:
    """Device copy of the tied int8 embedding (keeps the tensors alive) and its C struct."""

    def __init__(self, emb, device="cuda"):
        self.codes = _dev(emb.codes, device)
        self.row_scale = _dev(np.asarray(emb.row_scale, np.float32), device)
        self.vocab, self.d_model = emb.codes.shape
        self.struct = L.dfssm_embedding(self.codes.data_ptr(), self.row_scale.data_ptr(), self.vocab, self.d_model)


def _need(name: str, t: torch.Tensor, dtype, numel: int) -> None:
    """A device tensor the library will read or write: on the GPU, contiguous, of the given dtype
    (or element size) and with at least `numel` elements; ValueError otherwise, before any launch."""
    if t is None:
        raise ValueError(f"{name}: missing")
    if not t.is_cuda:
        raise ValueError(f"{name}: not a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if isinstance(dtype, int):
        if t.element_size() != dtype:
            raise ValueError(f"{name}: expected {dtype}-byte elements, got {t.dtype}")
    elif t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: holds {t.numel()} elements, needs {numel}")


def embed(emb: DeviceEmbedding, tokens: torch.Tensor, x: torch.Tensor) -> None:
    """x [batch][d_model] fp32 = the embedding rows of tokens (int32 device tensor)."""
    _need("tokens", tokens, torch.int32, 1)
    _need("x", x, torch.float32, tokens.numel() * emb.d_model)
    L.check(L.dfssm_embed(emb.struct, tokens.data_ptr(), tokens.numel(), x.data_ptr(), stream_handle()), "dfssm_embed")


def lm_head(d, emb: DeviceEmbedding, y: torch.Tensor, logits: torch.Tensor = None, next_tokens: torch.Tensor = None,
            ws: torch.Tensor = None, taps: dict = None) -> torch.Tensor:
    """Logits and/or greedy next tokens of y [batch][d_model]; returns the workspace it used."""
    batch = y.shape[0]
    _need("y", y, torch.float32, batch * emb.d_model)
    if logits is not None:
        _need("logits", logits, torch.float32, batch * emb.vocab)
    if next_tokens is not None:
        _need("next_tokens", next_tokens, torch.int32, batch)
    if ws is None:
        ws = workspace(d, L.DFSSM_OP_LM_HEAD, batch)
    t = None
    if taps is not None:
        t = L.dfssm_head_taps(*[taps[k].data_ptr() if k in taps else None for k in ("q", "s", "acc")])
    st = L.dfssm_lm_head(emb.struct, y.data_ptr(), batch, None if logits is None else logits.data_ptr(),
                         None if next_tokens is None else next_tokens.data_ptr(), ws.data_ptr(), ws.numel(), t,
                         stream_handle())
    L.check(st, "dfssm_lm_head")
    return ws


def state_encode(d, ssm: torch.Tensor, batch: int):
    """Density field codec of an SSM state [batch][H][P][N] -> (fields uint32 [rows][W], stats [rows][2])."""
    rows = batch * d.nheads * d.headdim
    W = L.dfssm_state_field_words(d.d_state)
    _need("ssm", ssm, torch.float32, rows * d.d_state)
    fields = torch.empty((rows, W), dtype=torch.int32, device=ssm.device)
    stats = torch.empty((rows, 2), dtype=torch.float32, device=ssm.device)
    L.check(L.dfssm_state_encode(dims_struct(d), ssm.data_ptr(), batch, fields.data_ptr(), stats.data_ptr(),
                                 stream_handle()), "dfssm_state_encode")
    return fields, stats


def state_decode(d, fields: torch.Tensor, stats: torch.Tensor, batch: int, ssm: torch.Tensor) -> None:
    """SSM state [batch][H][P][N] read back from fields [rows][W] and stats [rows][2]."""
    rows = batch * d.nheads * d.headdim
    _need("fields", fields, 4, rows * L.dfssm_state_field_words(d.d_state))
    _need("stats", stats, torch.float32, rows * 2)
    _need("ssm", ssm, torch.float32, rows * d.d_state)
    L.check(L.dfssm_state_decode(dims_struct(d), fields.data_ptr(), stats.data_ptr(), batch, ssm.data_ptr(),
                                 stream_handle()), "dfssm_state_decode")


class DeviceDfwProj:
    """A 17-level projection's tensors on the device (planes [5][n_out][n_in/8] uint8, ...)."""

    def __init__(self, w, device="cuda"):
        self.n_out, self.n_in, self.rank = int(w.n_out), int(w.n_in), int(w.rank)
        self.planes = _dev(np.ascontiguousarray(w.planes, np.uint8), device)
        self.row_scale = _dev(np.asarray(w.row_scale, np.float16).view(np.uint16), device)
        self.lora_dn = _dev(np.ascontiguousarray(w.lora_dn, np.int8), device)
        self.dn_scale = _dev(np.ascontiguousarray(w.dn_scale, np.float32), device)
        self.lora_up = _dev(np.ascontiguousarray(w.lora_up, np.int8), device)
        self.up_scale = _dev(np.ascontiguousarray(w.up_scale, np.float32), device)
        self.struct = L.dfssm_dfw_proj(self.planes.data_ptr(), self.row_scale.data_ptr(), self.lora_dn.data_ptr(),
                                       self.dn_scale.data_ptr(), self.lora_up.data_ptr(), self.up_scale.data_ptr())


def dfw_project(p: DeviceDfwProj, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor = None, taps: dict = None) -> None:
    """y [batch][n_out] = the 17-level projection of x [batch][n_in] (both fp32 on the device)."""
    batch = int(x.shape[0])
    _need("x", x, torch.float32, batch * p.n_in)
    _need("y", y, torch.float32, batch * p.n_out)
    if taps:
        for k, dt, n in (("q", torch.int8, batch * p.n_in), ("s", torch.float32, batch),
                         ("acc", torch.int32, batch * p.n_out), ("t", torch.int32, batch * p.rank)):
            if taps.get(k) is not None:
                _need(f"taps[{k}]", taps[k], dt, n)
    need = L.dfssm_dfw_workspace_bytes(p.n_in, p.rank, batch)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    t = None
    if taps:
        t = L.dfssm_dfw_taps(*[taps[k].data_ptr() if taps.get(k) is not None else None for k in ("q", "s", "acc", "t")])
    L.check(L.dfssm_dfw_project(p.struct, p.n_out, p.n_in, p.rank, x.data_ptr(), y.data_ptr(), batch,
                                ws.data_ptr(), ws.numel(), t, stream_handle()), "dfssm_dfw_project")
