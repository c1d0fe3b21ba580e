"""CPU-only checks of the C ABI: the header compiles as C99, the built library exports every
symbol the header declares, the ctypes structs match the C layout, and argument validation
rejects bad calls before anything touches a device."""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

from bit_quantized_mamba_packed_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfssm.h")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dfssm_[a-z_]+)\s*\(", txt)))


def test_header_is_c99():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write('#include "dfssm.h"\nint main(void){return 0;}\n')
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                            f"-I{os.path.dirname(HEADER)}", src], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    lib = L.load()
    decl = _declared_functions()
    assert set(decl) == set(L.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    for name in decl:
        assert re.search(rf"\bT {name}\b", out), name


def test_struct_layout_matches_c():
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "dfssm.h"
int main(void){
 printf("%zu %zu %zu %zu %zu\n", sizeof(dfssm_dims), sizeof(dfssm_proj), sizeof(dfssm_layer_weights),
        sizeof(dfssm_layer_state), sizeof(dfssm_taps));
 printf("%zu %zu %zu %zu\n", offsetof(dfssm_dims, norm_eps), offsetof(dfssm_layer_weights, conv_w),
        offsetof(dfssm_layer_weights, gnorm_w), offsetof(dfssm_taps, out_t));
 return 0;}
'''
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", f"-I{os.path.dirname(HEADER)}", src, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = [int(v) for v in lines[0].split()]
    offs = [int(v) for v in lines[1].split()]
    assert sizes == [C.sizeof(L.dfssm_dims), C.sizeof(L.dfssm_proj), C.sizeof(L.dfssm_layer_weights),
                     C.sizeof(L.dfssm_layer_state), C.sizeof(L.dfssm_taps)]
    assert offs == [L.dfssm_dims.norm_eps.offset, L.dfssm_layer_weights.conv_w.offset,
                    L.dfssm_layer_weights.gnorm_w.offset, L.dfssm_taps.out_t.offset]


def _dims(**kw):
    d = dict(d_model=256, d_inner=512, d_state=16, headdim=64, ngroups=1, d_conv=4, n_in_proj=1072,
             rank_in=8, rank_out=8, norm_eps=1e-5)
    d.update(kw)
    return L.dfssm_dims(**d)


FAKE = 0x7f0000001000   # aligned, never dereferenced: every call below fails validation first


def _fake_weights():
    p = L.dfssm_proj(*([FAKE] * 6))
    return L.dfssm_layer_weights(p, p, *([FAKE] * 7))


def test_workspace_bytes_and_shape_validation():
    assert L.dfssm_workspace_bytes(_dims(), L.DFSSM_OP_LAYER_DECODE, 1) > 0
    assert L.dfssm_workspace_bytes(_dims(), L.DFSSM_OP_STACK_DECODE, 1, 0, 48) > \
        L.dfssm_workspace_bytes(_dims(), L.DFSSM_OP_LAYER_DECODE, 1)
    for bad in (dict(d_model=200), dict(headdim=32), dict(d_state=24), dict(d_conv=3), dict(n_in_proj=1000),
                dict(rank_in=65), dict(ngroups=3), dict(norm_eps=0.0), dict(d_model=0)):
        assert L.dfssm_workspace_bytes(_dims(**bad), L.DFSSM_OP_LAYER_DECODE, 1) == 0, bad
    assert L.dfssm_workspace_bytes(_dims(), L.DFSSM_OP_LAYER_DECODE, 0) == 0
    assert L.dfssm_workspace_bytes(_dims(), 99, 1) == 0


def test_layer_decode_rejects_bad_arguments_without_touching_a_device():
    d = _dims()
    w = _fake_weights()
    st = L.dfssm_layer_state(FAKE, FAKE)
    need = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_DECODE, 2)
    ok = dict(x_in=FAKE, x_out=FAKE, batch=2, ws=FAKE, ws_bytes=need)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.dfssm_layer_decode(d, w, st, a["x_in"], a["x_out"], a["batch"], a["ws"], a["ws_bytes"])

    assert call(x_in=None) == L.DFSSM_EINVAL
    assert call(x_out=FAKE + 4) == L.DFSSM_EINVAL          # misaligned
    assert call(batch=0) == L.DFSSM_EINVAL
    assert call(batch=5000) == L.DFSSM_EUNSUPPORTED
    assert call(ws=None) == L.DFSSM_EINVAL
    assert call(ws_bytes=need - 1) == L.DFSSM_EWORKSPACE
    assert L.dfssm_layer_decode(_dims(d_conv=2), w, st, FAKE, FAKE, 1, FAKE, need) == L.DFSSM_EUNSUPPORTED
    w_bad = _fake_weights()
    w_bad.in_proj.lora_up = None
    assert L.dfssm_layer_decode(d, w_bad, st, FAKE, FAKE, 1, FAKE, need) == L.DFSSM_EINVAL
    st_bad = L.dfssm_layer_state(FAKE, None)
    assert L.dfssm_layer_decode(d, w, st_bad, FAKE, FAKE, 1, FAKE, need) == L.DFSSM_EINVAL
    taps = L.dfssm_taps()
    taps.in_q = FAKE + 1
    assert L.dfssm_layer_decode(d, w, st, FAKE, FAKE, 1, FAKE, need, taps) == L.DFSSM_EINVAL


def test_stack_decode_rejects_bad_arguments():
    d = _dims()
    n = 3
    ws_need = L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_DECODE, 1, 0, n)
    arr_w = (L.dfssm_layer_weights * n)(*[_fake_weights() for _ in range(n)])
    arr_s = (L.dfssm_layer_state * n)(*[L.dfssm_layer_state(FAKE, FAKE) for _ in range(n)])
    f = L.dfssm_stack_decode
    assert f(d, arr_w, arr_s, 0, FAKE, FAKE, FAKE, 1, 4, FAKE, ws_need) == L.DFSSM_EINVAL
    assert f(d, arr_w, arr_s, n, FAKE, FAKE, FAKE, 1, 0, FAKE, ws_need) == L.DFSSM_EINVAL
    assert f(d, arr_w, arr_s, n, FAKE, FAKE, FAKE, 1, 4, FAKE, ws_need - 1) == L.DFSSM_EWORKSPACE
    arr_s[2].ssm = None
    assert f(d, arr_w, arr_s, n, FAKE, FAKE, FAKE, 1, 4, FAKE, ws_need) == L.DFSSM_EINVAL


def test_strerror():
    for s in (L.DFSSM_OK, L.DFSSM_EINVAL, L.DFSSM_EUNSUPPORTED, L.DFSSM_EWORKSPACE, L.DFSSM_EHIP):
        assert len(L.dfssm_strerror(s)) > 3
    assert L.dfssm_strerror(12345) == "unknown status"


def test_prefill_workspace_and_rejects_bad_arguments():
    d = _dims()
    ws1 = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 1, 300)
    assert ws1 > 0
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 2, 300) > ws1
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 1, 0) == 0
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 1, 65537) == 0
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 65, 16) == 0
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 32, 65536) == 0     # > 2^20 tokens
    assert L.dfssm_workspace_bytes(_dims(rank_in=4), L.DFSSM_OP_LAYER_PREFILL, 1, 16) == 0
    w = _fake_weights()
    st = L.dfssm_layer_state(FAKE, FAKE)
    X2 = FAKE + 0x100000
    ok = dict(x_in=FAKE, dt=L.DFSSM_F32, x_out=X2, batch=1, seqlen=300, chunk=64, ws=FAKE, ws_bytes=ws1)

    def call(dims=d, **kw):
        a = dict(ok)
        a.update(kw)
        return L.dfssm_layer_prefill(dims, w, st, a["x_in"], a["dt"], a["x_out"], a["batch"], a["seqlen"],
                                     a["chunk"], a["ws"], a["ws_bytes"])

    assert call(x_in=None) == L.DFSSM_EINVAL
    assert call(x_out=FAKE) == L.DFSSM_EINVAL                 # aliases x_in
    assert call(dt=7) == L.DFSSM_EINVAL
    assert call(seqlen=0) == L.DFSSM_EINVAL
    assert call(chunk=48) == L.DFSSM_EUNSUPPORTED
    assert call(chunk=512) == L.DFSSM_EUNSUPPORTED
    assert call(batch=65) == L.DFSSM_EUNSUPPORTED
    assert call(seqlen=65537) == L.DFSSM_EUNSUPPORTED
    assert call(dims=_dims(rank_out=12)) == L.DFSSM_EUNSUPPORTED
    assert call(ws_bytes=4096) == L.DFSSM_EWORKSPACE       # below what any chunk length needs
    assert call(ws=FAKE + 8) == L.DFSSM_EINVAL


def test_batched_decode_workspace_covers_the_mfma_path():
    d = _dims()
    w4 = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_DECODE, 4)
    w5 = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_DECODE, 5)
    # beyond 4 tokens the projections run as GEMMs over per-token codes held in the workspace
    assert w5 > w4 * 5 // 4 + 5 * d.d_model
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_DECODE, 64, 0, 48) > 0


def test_stack_decode_ex_rejects_bad_options():
    d = _dims()
    n = 2
    ws_need = L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_DECODE, 1, 0, n)
    arr_w = (L.dfssm_layer_weights * n)(*[_fake_weights() for _ in range(n)])
    arr_s = (L.dfssm_layer_state * n)(*[L.dfssm_layer_state(FAKE, FAKE) for _ in range(n)])

    def call(**kw):
        return L.dfssm_stack_decode_ex(d, arr_w, arr_s, n, FAKE, FAKE, FAKE, 1, 4, FAKE, ws_need,
                                       None, L.dfssm_stack_opts(**kw))

    assert call(path=7) == L.DFSSM_EINVAL
    assert call(path=-1) == L.DFSSM_EINVAL
    assert call(launch=2) == L.DFSSM_EINVAL
    assert call(launch=-1) == L.DFSSM_EINVAL
    # batch 5 has no persistent kernel: asking for one is unsupported, not silently rerouted
    ws5 = L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_DECODE, 5, 0, n)
    st = L.dfssm_stack_decode_ex(d, arr_w, arr_s, n, FAKE, FAKE, FAKE, 5, 4, FAKE, ws5, None,
                                 L.dfssm_stack_opts(path=L.DFSSM_PATH_FLOW))
    assert st == L.DFSSM_EUNSUPPORTED


def test_stack_prefill_workspace_and_rejects_bad_arguments():
    d = _dims()
    n = 3
    one = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 2, 100)
    need = L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_PREFILL, 2, 100, n)
    # one layer's prefill workspace plus one residual buffer of batch x seqlen x d_model floats
    assert need >= one + 2 * 100 * d.d_model * 4
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_PREFILL, 2, 100, 0) == 0
    assert L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_PREFILL, 65, 100, n) == 0
    arr_w = (L.dfssm_layer_weights * n)(*[_fake_weights() for _ in range(n)])
    arr_s = (L.dfssm_layer_state * n)(*[L.dfssm_layer_state(FAKE, FAKE) for _ in range(n)])
    Y = FAKE + 0x100000
    ok = dict(nl=n, x=FAKE, dt=L.DFSSM_F32, y=Y, batch=2, seqlen=100, chunk=64, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.dfssm_stack_prefill(d, arr_w, arr_s, a["nl"], FAKE, a["x"], a["dt"], a["y"], a["batch"],
                                     a["seqlen"], a["chunk"], a["ws"], a["wsb"])

    assert call(nl=0) == L.DFSSM_EINVAL
    assert call(y=FAKE) == L.DFSSM_EINVAL            # aliases x_in
    assert call(dt=3) == L.DFSSM_EINVAL
    assert call(chunk=100) == L.DFSSM_EUNSUPPORTED
    assert call(batch=65) == L.DFSSM_EUNSUPPORTED
    assert call(wsb=2 * 100 * d.d_model * 4) == L.DFSSM_EWORKSPACE     # the residual buffer alone
    arr_s[1].conv = None
    assert call() == L.DFSSM_EINVAL


def test_stack_workspace_covers_status_word_and_every_layer_step():
    """A stack decode's workspace holds its status word (256 bytes) ahead of what one layer step of
    the same batch needs, for the packed-sign GEMV batches and the MFMA GEMM batches alike."""
    for d in (_dims(), _dims(d_model=2048, d_inner=4096, d_state=128, n_in_proj=8512, rank_in=32, rank_out=32)):
        for B in (1, 2, 4, 5, 8, 64, 65, 512):
            layer = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_DECODE, B)
            stack = L.dfssm_workspace_bytes(d, L.DFSSM_OP_STACK_DECODE, B, 0, 3)
            assert stack >= layer + 256 + 2 * B * d.d_model * 4, (B, layer, stack)


def test_state_codec_field_size_and_rejects_bad_arguments():
    # K = round(sqrt(4 d_state)): 8, 11, 16, 23, 32 -> ceil(K^2 / 32) words
    assert [L.dfssm_state_field_words(n) for n in (16, 32, 64, 128, 256)] == [2, 4, 8, 17, 32]
    assert L.dfssm_state_field_words(100) == 0
    d = _dims()
    for fn in (lambda **k: L.dfssm_state_encode(k.get("dims", d), k.get("a", FAKE), k.get("batch", 1),
                                                k.get("b", FAKE), k.get("c", FAKE)),
               lambda **k: L.dfssm_state_decode(k.get("dims", d), k.get("b", FAKE), k.get("c", FAKE),
                                                k.get("batch", 1), k.get("a", FAKE))):
        assert fn(a=None) == L.DFSSM_EINVAL
        assert fn(b=FAKE + 4) == L.DFSSM_EINVAL
        assert fn(c=None) == L.DFSSM_EINVAL
        assert fn(batch=0) == L.DFSSM_EINVAL
        assert fn(batch=4097) == L.DFSSM_EUNSUPPORTED
        assert fn(dims=_dims(d_state=100)) == L.DFSSM_EUNSUPPORTED


def test_dfw_project_workspace_and_rejects_bad_arguments():
    assert L.dfssm_dfw_workspace_bytes(2048, 32, 4) > 0
    assert L.dfssm_dfw_workspace_bytes(100, 32, 4) == 0
    assert L.dfssm_dfw_workspace_bytes(2048, 65, 4) == 0
    assert L.dfssm_dfw_workspace_bytes(2048, 32, 257) == 0
    w = L.dfssm_dfw_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = L.dfssm_dfw_workspace_bytes(2048, 32, 2)

    def call(**kw):
        a = dict(w=w, n_out=512, n_in=2048, rank=32, x=FAKE, y=FAKE, batch=2, ws=FAKE, ws_bytes=need, taps=None)
        a.update(kw)
        return L.dfssm_dfw_project(a["w"], a["n_out"], a["n_in"], a["rank"], a["x"], a["y"], a["batch"],
                                   a["ws"], a["ws_bytes"], a["taps"])

    assert call(x=None) == L.DFSSM_EINVAL
    assert call(y=FAKE + 8) == L.DFSSM_EINVAL
    assert call(w=L.dfssm_dfw_proj(None, FAKE, FAKE, FAKE, FAKE, FAKE)) == L.DFSSM_EINVAL
    assert call(batch=0) == L.DFSSM_EINVAL
    assert call(n_in=2000) == L.DFSSM_EUNSUPPORTED
    assert call(n_in=16384) == L.DFSSM_EUNSUPPORTED
    assert call(rank=65) == L.DFSSM_EUNSUPPORTED
    assert call(batch=257) == L.DFSSM_EUNSUPPORTED
    assert call(ws_bytes=need - 1) == L.DFSSM_EWORKSPACE
    assert call(taps=L.dfssm_dfw_taps(FAKE + 1, None, None, None)) == L.DFSSM_EINVAL


def test_dfw_workspace_holds_every_region():
    # codes [B][K] i8 + their eight bit planes (K bytes per token) + s + sum(q) + t [B][rank] i32,
    # each region rounded to 256 bytes
    r = lambda v: (v + 255) // 256 * 256
    for K, rank, B in ((256, 8, 3), (2048, 32, 4), (8192, 64, 256), (384, 5, 5)):
        assert L.dfssm_dfw_workspace_bytes(K, rank, B) == r(B * K) + r(B * K) + r(4 * B) + r(4 * B) + r(4 * B * rank)


def test_layer_prefill_ex_rejects_bad_options():
    d = _dims()
    w = _fake_weights()
    st = L.dfssm_layer_state(FAKE, FAKE)
    need = L.dfssm_workspace_bytes(d, L.DFSSM_OP_LAYER_PREFILL, 1, 64)

    def call(opts):
        return L.dfssm_layer_prefill_ex(d, w, st, FAKE, L.DFSSM_F32, FAKE + 4096, 1, 64, 16, FAKE, need, None, opts)

    assert call(L.dfssm_prefill_opts(2, 0, None, None)) == L.DFSSM_EINVAL
    assert call(L.dfssm_prefill_opts(1, 1, None, None)) == L.DFSSM_EINVAL
    assert call(L.dfssm_prefill_opts(1, 0, FAKE + 4, None)) == L.DFSSM_EINVAL
    assert call(L.dfssm_prefill_opts(0, 0, FAKE, None)) == L.DFSSM_EINVAL      # taps without the codec


def test_device_wrappers_reject_host_and_short_tensors():
    import torch
    from bit_quantized_mamba_packed_amd import device as Dv
    with pytest.raises(ValueError, match="not a device tensor"):
        Dv._need("x", torch.zeros(4), torch.float32, 4)
    with pytest.raises(ValueError):
        Dv._need("x", None, torch.float32, 4)
