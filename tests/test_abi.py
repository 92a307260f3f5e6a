"""The C-ABI library loads, exports every symbol include/moe_nvfp4.h declares, and
turns bad arguments into the documented error codes on the host (CPU only: no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a4_expert_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_four_steps():
    names = declared_functions()
    for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_quantize_act",
              "moe_workspace_bytes", "moe_strerror", "moe_abi_version"):
        assert f in names, f


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), "missing export " + f


def test_abi_version_and_strerror():
    assert moe.lib.moe_abi_version() == 4
    for code in (0, -1, -2, -3, -4):
        assert moe.strerror(code) and moe.strerror(code) != "unknown error"
    assert moe.strerror(-99) == "unknown error"


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def fake_bank():
    return moe.Bank(FAKE, FAKE, FAKE)


def layer(H=2048, I=512, E=512, k=10, shared=1, **kw):
    d = moe.LayerDesc(H, I, E, k, shared, FAKE, fake_bank(), fake_bank(), fake_bank(), fake_bank(), 1.0, 1.0)
    for a, v in kw.items():
        setattr(d, a, v)
    return d


def route(L, T=4, x=FAKE, idx=FAKE, w=FAKE, ws=FAKE, wsb=1 << 30):
    return moe.lib.moe_route(ctypes.byref(L) if L is not None else None, x, T, None, idx, w, ws, wsb, None)


@pytest.mark.parametrize("H,I,E,k", [(2000, 512, 512, 10), (2048, 500, 512, 10), (2048, 512, 0, 1),
                                     (2048, 512, 2048, 10), (2048, 512, 8, 9), (2048, 512, 512, 0),
                                     (2048, 512, 512, 33), (32768, 512, 512, 10), (2048, 8192, 512, 10)])
def test_bad_shapes(H, I, E, k):
    L = layer(H, I, E, k)
    assert route(L) == moe.MOE_ESHAPE
    assert moe.lib.moe_workspace_bytes(ctypes.byref(L), 16) == 0


def test_null_and_misaligned_pointers():
    assert route(None) == moe.MOE_EINVAL
    assert route(layer(), x=None) == moe.MOE_EINVAL
    assert route(layer(), idx=FAKE + 4) == moe.MOE_EINVAL
    assert route(layer(router_w=None)) == moe.MOE_EINVAL
    L = layer()
    L.w13.codes = FAKE + 8
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL


def test_non_power_of_two_activation_scale():
    L = layer(a_gscale_in=3.0)
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL
    assert moe.lib.moe_quantize_act(FAKE, 0, 4, 64, 0.75, FAKE, FAKE, None) == moe.MOE_EINVAL


def test_shared_output_required_when_shared():
    L = layer()
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL


def test_negative_T_and_zero_T():
    L = layer()
    assert route(L, T=-1) == moe.MOE_ESHAPE
    assert route(L, T=0, x=None, idx=None, w=None, ws=None) == moe.MOE_OK
    assert moe.lib.moe_permute(ctypes.byref(L), None, 0, FAKE, None, None, None, 0, None) == moe.MOE_OK
    assert moe.lib.moe_expert_ffn(ctypes.byref(L), None, 0, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert moe.lib.moe_combine(ctypes.byref(L), 0, None, None, None, None, None, None, None) == moe.MOE_OK
    assert moe.lib.moe_quantize_act(None, 0, 0, 64, 1.0, None, None, None) == moe.MOE_OK


def test_router_mode_gate_and_act_bits_validated():
    """Router precision modes, the shared-expert gate vector, the cached router pieces
    and the activation width are checked on the host."""
    for mode in (-1, 3):
        assert route(layer(router_mode=mode)) == moe.MOE_ESHAPE
    for bits in (1, 5, 16):
        assert route(layer(act_bits=bits)) == moe.MOE_ESHAPE
    # the reduced-precision routers run on the matrix cores: E a multiple of 128
    for mode in (moe.MOE_ROUTER_SPLIT3_F32, moe.MOE_ROUTER_BF16):
        assert route(layer(E=96, router_mode=mode), wsb=0) == moe.MOE_ESHAPE
        assert route(layer(router_mode=mode), wsb=0) == moe.MOE_EWORKSPACE
    assert route(layer(E=96), wsb=0) == moe.MOE_EWORKSPACE  # the exact router takes any E
    assert route(layer(router_pieces=FAKE + 8)) == moe.MOE_EINVAL
    bad_gate = layer(shared_gate_w=FAKE + 4)
    rc = moe.lib.moe_expert_ffn(ctypes.byref(bad_gate), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL
    # a gate adds T floats of workspace, only with a shared expert
    base = moe.lib.moe_workspace_bytes(ctypes.byref(layer()), 4096)
    assert moe.lib.moe_workspace_bytes(ctypes.byref(layer(shared_gate_w=FAKE)), 4096) > base
    assert moe.lib.moe_workspace_bytes(ctypes.byref(layer(shared=0, shared_gate_w=FAKE)), 4096) == \
        moe.lib.moe_workspace_bytes(ctypes.byref(layer(shared=0)), 4096)
    assert moe.lib.moe_pack_router(FAKE, 0, 2048, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_pack_router(FAKE, 512, 2048, None, None) == moe.MOE_EINVAL


def test_pre_norm_validated():
    """pre_norm (moe_layer_forward only) takes 0 or 1 and an eps in [0, 1]; it adds the
    normed input's T * H BF16 to the workspace, checked before anything runs."""
    def fwd(L, wsb=1 << 30):
        return moe.lib.moe_layer_forward(ctypes.byref(L), FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, None, FAKE, wsb, None)
    assert fwd(layer(pre_norm=2, pre_norm_eps=1e-6)) == moe.MOE_EINVAL
    assert fwd(layer(pre_norm=-1)) == moe.MOE_EINVAL
    for eps in (-1e-6, 1.5, float("nan")):
        assert fwd(layer(pre_norm=1, pre_norm_eps=eps)) == moe.MOE_EINVAL
    assert fwd(layer(pre_norm=1, pre_norm_eps=1e-6), wsb=4 * 2048 * 2 - 1) == moe.MOE_EWORKSPACE
    base = moe.lib.moe_workspace_bytes(ctypes.byref(layer()), 300)
    normed = moe.lib.moe_workspace_bytes(ctypes.byref(layer(pre_norm=1, pre_norm_eps=1e-6)), 300)
    assert normed - base >= 300 * 2048 * 2


def test_w4a8_validation_and_workspace():
    """act_bits 8 (the W4A8 variant) is accepted; its code buffers take one byte per
    element, so its workspace is larger; moe_quantize_act8 validates like its A4 twin."""
    a4 = moe.lib.moe_workspace_bytes(ctypes.byref(layer()), 300)
    a8 = moe.lib.moe_workspace_bytes(ctypes.byref(layer(act_bits=8)), 300)
    assert a8 > a4
    assert moe.lib.moe_quantize_act8(FAKE, 0, 4, 20, 1.0, FAKE, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_quantize_act8(FAKE, 2, 4, 32, 1.0, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_quantize_act8(FAKE, 0, 4, 32, 0.3, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_quantize_act8(None, 0, 0, 32, 1.0, None, None, None) == moe.MOE_OK


def test_token_bound():
    """T * H * 2 and T * (k + 1) must stay below 2^31 (32-bit row offsets of the
    router's and the matrix-core kernels' buffer resources, int32 pair ids): the
    first count past the bound is refused by every layer entry point, the last
    one below it is not refused for its shape."""
    L = layer()  # H 2048, k 10: the bound is 2^31 / 4096 = 524,288 tokens
    big = (1 << 31) // (2 * L.H)
    assert big == 524288
    assert moe.lib.moe_workspace_bytes(ctypes.byref(L), big) == 0
    assert moe.lib.moe_workspace_bytes(ctypes.byref(L), big - 1) > 0
    assert route(L, T=big) == moe.MOE_ESHAPE
    assert route(L, T=big - 1, wsb=0) == moe.MOE_EWORKSPACE
    assert moe.lib.moe_permute(ctypes.byref(L), FAKE, big, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, big, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                  None) == moe.MOE_ESHAPE
    assert moe.lib.moe_combine(ctypes.byref(L), big, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_combine_f32(ctypes.byref(L), big, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_layer_forward(ctypes.byref(L), FAKE, big, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None, FAKE, 1 << 40, None) == moe.MOE_ESHAPE
    # the smallest hidden size: 2^31 / 64 tokens
    Ls = layer(H=32, I=32, E=64, k=32)
    assert route(Ls, T=(1 << 31) // 64) == moe.MOE_ESHAPE
    assert route(Ls, T=(1 << 31) // 64 - 1, wsb=0) == moe.MOE_EWORKSPACE


def test_noalloc_refuses_beyond_its_array():
    """The allocation-free layer call checks its size before touching the GPU: a
    token count whose workspace exceeds the library's 64 MiB array is refused."""
    L = layer()
    lim = moe.lib.moe_noalloc_scratch_bytes()
    assert lim == 64 << 20
    T = 1
    while moe.lib.moe_workspace_bytes(ctypes.byref(L), T) <= lim:
        T += 256
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert moe.lib.moe_layer_forward_noalloc(ctypes.byref(L), FAKE, T, None, *args) == moe.MOE_EWORKSPACE
    assert moe.lib.moe_layer_forward_noalloc(ctypes.byref(L), FAKE, -1, None, *args) == moe.MOE_ESHAPE
    assert moe.lib.moe_layer_forward_noalloc(None, FAKE, 4, None, *args) == moe.MOE_EINVAL


def test_workspace_too_small():
    L = layer()
    need = moe.lib.moe_workspace_bytes(ctypes.byref(L), 4)
    assert need > 0
    assert route(L, wsb=0) == moe.MOE_EWORKSPACE
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1024, None)
    assert rc == moe.MOE_EWORKSPACE
    rc = moe.lib.moe_layer_forward(ctypes.byref(L), FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None, FAKE, 1024, None)
    assert rc == moe.MOE_EWORKSPACE
    rc = moe.lib.moe_permute(ctypes.byref(L), FAKE, 100000, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert rc == moe.MOE_EWORKSPACE


def test_kmajor_copies_validated():
    L = layer()
    L.w13k = moe.Bank(FAKE + 8, FAKE, None)  # misaligned codes
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL
    L = layer()
    L.w2k = moe.Bank(FAKE, None, None)  # codes without scales
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL
    L = layer(I=544)  # I not a whole number of 64-element steps
    L.w2k = moe.Bank(FAKE, FAKE, None)
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe.MOE_ESHAPE
    pack = moe.lib.moe_pack_kmajor
    assert pack(FAKE, FAKE, 1, 64, 96, FAKE, FAKE, None) == moe.MOE_ESHAPE
    assert pack(FAKE, FAKE, 0, 64, 128, FAKE, FAKE, None) == moe.MOE_ESHAPE
    assert pack(FAKE, FAKE, 1, 64, 128, FAKE + 4, FAKE, None) == moe.MOE_EINVAL
    assert pack(FAKE, FAKE + 2, 1, 64, 128, FAKE, FAKE, None) == moe.MOE_EINVAL


def test_workspace_monotone_in_T():
    L = layer()
    sizes = [moe.lib.moe_workspace_bytes(ctypes.byref(L), T) for T in (1, 4, 4096, 15360)]
    assert sizes == sorted(sizes) and all(s % 256 == 0 for s in sizes)


def test_bad_dtype_and_cols():
    assert moe.lib.moe_quantize_act(FAKE, 7, 4, 64, 1.0, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_quantize_act(FAKE, 0, 4, 60, 1.0, FAKE, FAKE, None) == moe.MOE_ESHAPE


def test_null_event_entry_is_rejected():
    L = layer()
    arr = (ctypes.c_void_p * (2 * moe.FFN_KERNELS))(*([FAKE] * (2 * moe.FFN_KERNELS - 1) + [None]))
    dbg = moe.Debug(None, None, None, None, None, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
    rc = moe.lib.moe_expert_ffn(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, ctypes.byref(dbg), FAKE, 1 << 30,
                                None)
    assert rc == moe.MOE_EINVAL
    rc = moe.lib.moe_layer_forward(ctypes.byref(L), FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   ctypes.byref(dbg), FAKE, 1 << 30, None)
    assert rc == moe.MOE_EINVAL


def test_rms_norm_validation():
    assert moe.lib.moe_rms_norm(FAKE, -1, 2048, 1e-6, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_rms_norm(FAKE, 4, 0, 1e-6, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_rms_norm(FAKE, 4, 2048, -1.0, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_rms_norm(FAKE, 4, 2048, float("nan"), FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_rms_norm(None, 4, 2048, 1e-6, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_rms_norm(None, 0, 2048, 1e-6, None, None) == moe.MOE_OK


def test_krange_validation():
    L = layer()
    args = lambda kb0, kb1: (ctypes.byref(L), FAKE, 64, FAKE, FAKE, kb0, kb1, FAKE, FAKE, FAKE, 1 << 30, None)
    for kb0, kb1 in ((0, 33), (-2, 16), (16, 16), (3, 16), (0, 15), (20, 10)):
        assert moe.lib.moe_expert_ffn_krange(*args(kb0, kb1)) == moe.MOE_ESHAPE, (kb0, kb1)
    assert moe.lib.moe_combine_f32(ctypes.byref(L), -1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_ESHAPE
    assert moe.lib.moe_combine_f32(ctypes.byref(L), 4, FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL


def test_package_refuses_to_load_without_the_library(tmp_path):
    """No CPU fallback: a copy of the binding next to no built library raises
    ImportError on import (checked in a fresh interpreter)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "nvfp4_w4a4_expert_router_amd", "__init__.py")
    pkg = tmp_path / "nvfp4_w4a4_expert_router_amd"
    pkg.mkdir()
    shutil.copy(src, pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import nvfp4_w4a4_expert_router_amd\nexcept ImportError as e:\n    print('refused:', e)\n"
            "else:\n    print('loaded')\n") % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert "refused:" in r.stdout and "not built" in r.stdout, r.stdout + r.stderr


def test_noalloc_token_bound():
    """The allocation-free entry point's stated bound: its 64 MiB array holds the
    workspace of 3,391 tokens at the decode shape, and 3,392 tokens are refused with
    MOE_EWORKSPACE before anything touches the GPU."""
    L = layer()
    cap = moe.lib.moe_noalloc_scratch_bytes()
    assert cap == 64 << 20
    assert moe.lib.moe_workspace_bytes(ctypes.byref(L), 3391) <= cap < moe.lib.moe_workspace_bytes(ctypes.byref(L), 3392)
    rc = moe.lib.moe_layer_forward_noalloc(ctypes.byref(L), FAKE, 3392, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, None, None)
    assert rc == moe.MOE_EWORKSPACE
