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
    def from_tensors(cls, conv: torch.Tensor, ssm: torch.Tensor) -> "DeviceState":
        """A state over existing contiguous fp32 device tensors (e.g. views of one allocation that
        holds a whole stack's states, so that they can be reset with one fill)."""
        if not (conv.is_contiguous() and ssm.is_contiguous()) or conv.dtype != torch.float32 or ssm.dtype != torch.float32:
            raise ValueError("DeviceState.from_tensors: contiguous fp32 tensors required")
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
    st = L.dfssm_layer_decode(dims_struct(d), layer.struct, state.struct, x_in.data_ptr(), x_out.data_ptr(),
                              batch, ws.data_ptr(), ws.numel(), None if taps is None else taps.struct,
                              stream_handle())
    L.check(st, "dfssm_layer_decode")


def stack_decode(d, layers: list, states: list, final_w: torch.Tensor, x0: torch.Tensor, y: torch.Tensor,
                 n_steps: int, ws: torch.Tensor, taps: Taps = None) -> None:
    n = len(layers)
    arr_w = (L.dfssm_layer_weights * n)(*[l.struct for l in layers])
    arr_s = (L.dfssm_layer_state * n)(*[s.struct for s in states])
    st = L.dfssm_stack_decode(dims_struct(d), arr_w, arr_s, n, final_w.data_ptr(), x0.data_ptr(), y.data_ptr(),
                              x0.shape[0], n_steps, ws.data_ptr(), ws.numel(),
                              None if taps is None else taps.struct, stream_handle())
    L.check(st, "dfssm_stack_decode")


def layer_prefill(d, layer: DeviceLayer, state: DeviceState, x_in: torch.Tensor, x_out: torch.Tensor, chunk: int,
                  ws: torch.Tensor, taps: Taps = None) -> None:
    """x_in [batch][seqlen][d_model] fp32 or bf16 (torch.bfloat16 is passed as its bit patterns)."""
    batch, seqlen = x_in.shape[0], x_in.shape[1]
    dtype = L.DFSSM_BF16 if x_in.dtype == torch.bfloat16 else L.DFSSM_F32
    st = L.dfssm_layer_prefill(dims_struct(d), layer.struct, state.struct, x_in.data_ptr(), dtype, x_out.data_ptr(),
                               batch, seqlen, chunk, ws.data_ptr(), ws.numel(),
                               None if taps is None else taps.struct, stream_handle())
    L.check(st, "dfssm_layer_prefill")
