"""Host-only checks of the C ABI: the library loads, exports every symbol the header declares,
and rejects bad arguments with the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest
import torch

import bit_expert_ffn_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")

OK, INVALID, SHAPE, WS = 0, -1, -2, -3
A = 0x10000  # a 16-byte aligned fake device address: never dereferenced, every case fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    declared = _declared()
    assert set(declared) == set(moe.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    assert moe.abi_version() == 5
    for code in (OK, INVALID, SHAPE, WS, -4, -5, -6, -7, 7):
        assert isinstance(moe.status_string(code), str) and moe.status_string(code)


@pytest.mark.parametrize("T,H,I,E,k,ok", [
    (1, 7168, 2048, 256, 8, True), (4, 256, 128, 8, 2, True), (16384, 7168, 2048, 256, 8, True),
    # x and h are read through 32-bit element offsets: T*H and T*k*I below 2^32
    (65536, 65536, 128, 8, 2, False), (65535, 65536, 128, 8, 2, True),
    (262144, 256, 2048, 256, 8, False), (262143, 256, 2048, 256, 8, True),
    (0, 256, 128, 8, 2, False), (4, 250, 128, 8, 2, False), (4, 256, 100, 8, 2, False),
    (4, 256, 128, 300, 2, False), (4, 256, 128, 8, 9, False), (4, 256, 128, 8, 0, False),
])
def test_workspace_size(T, H, I, E, k, ok):
    n = moe.workspace_size(T, H, I, E, k)
    assert (n > 0) == ok
    if ok:
        assert n % 256 == 0
        # the FFN needs at least x and h in f16
        assert n >= T * H * 2 + T * k * I * 2


def _route(**over):
    a = dict(x=A, wr=A, bias=None, T=4, H=256, E=8, k=2, logits=None, ids=A, w=A, ws=A,
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    return moe.lib().moe_route(a["x"], a["wr"], a["bias"], a["T"], a["H"], a["E"], a["k"],
                               a["logits"], a["ids"], a["w"], a["ws"], a["ws_bytes"], a["stream"])


def test_route_rejects_bad_arguments():
    assert _route(x=None) == INVALID
    assert _route(ids=None) == INVALID
    assert _route(x=A + 2) == INVALID
    assert _route(bias=A + 4) == INVALID
    assert _route(T=0) == INVALID
    assert _route(k=9) == INVALID
    assert _route(k=0) == INVALID
    assert _route(E=300, k=2) == SHAPE
    assert _route(H=200) == SHAPE
    assert _route(ws_bytes=16) == WS


def _group(**over):
    a = dict(ids=A, T=4, k=2, E=8, ws=A, ws_bytes=1 << 30)
    a.update(over)
    return moe.lib().moe_group(a["ids"], a["T"], a["k"], a["E"], A, A, A, A, A, A, a["ws"],
                               a["ws_bytes"], None)


def test_group_rejects_bad_arguments():
    assert _group(ids=None) == INVALID
    assert _group(ids=A + 8) == INVALID
    assert _group(T=0) == INVALID
    assert _group(E=257, k=2) == SHAPE
    assert _group(k=9) == INVALID
    # the three-pass grouping needs workspace
    assert _group(T=4096, k=8, E=256, ws_bytes=0) == WS
    assert _group(T=4096, k=8, E=256, ws=None) == INVALID


def _experts(**over):
    f = dict(gate_q=A, up_q=A, down_q=A, gate_s=A, up_s=A, down_s=A, tensor_scale=A, E=8, H=256, I=128)
    f.update(over)
    return moe._Experts(**f)


def _ffn(w=None, **over):
    a = dict(x=A, T=4, k=2, y=A, yd=0, ws=A, ws_bytes=1 << 30)
    a.update(over)
    s = w if w is not None else _experts()
    return moe.lib().moe_expert_ffn_nvfp4(a["x"], ctypes.byref(s), A, A, A, A, A, a["T"], a["k"],
                                          a["y"], a["yd"], a["ws"], a["ws_bytes"], None)


def test_ffn_rejects_bad_arguments():
    assert _ffn(x=None) == INVALID
    assert _ffn(yd=2) == INVALID
    assert _ffn(y=A + 1) == INVALID
    assert _ffn(_experts(down_s=None)) == INVALID
    assert _ffn(_experts(gate_q=A + 4)) == INVALID
    assert _ffn(_experts(H=200)) == SHAPE
    assert _ffn(_experts(I=96)) == SHAPE
    assert _ffn(_experts(E=512)) == SHAPE
    assert _ffn(k=9) == INVALID
    assert _ffn(T=0) == INVALID
    assert _ffn(ws_bytes=1024) == WS
    assert moe.lib().moe_expert_ffn_nvfp4(A, None, A, A, A, A, A, 4, 2, A, 0, A, 1 << 30, None) == INVALID


def test_combine_rejects_bad_arguments():
    c = moe.lib().moe_combine
    assert c(None, 0, A, A, 4, 2, 256, A, None) == INVALID
    assert c(A, 3, A, A, 4, 2, 256, A, None) == INVALID
    assert c(A, 0, A, A + 4, 4, 2, 256, A, None) == INVALID
    assert c(A, 0, A, A, 0, 2, 256, A, None) == INVALID
    assert c(A, 0, A, A, 4, 2, 200, A, None) == SHAPE


def _cn(flags=0, eps=1e-6, resid=A, gain=A, out=A, xn=A, y=A, yd=1, H=256, T=4, k=2):
    return moe.lib().moe_combine_norm(y, yd, A, A, T, k, H, flags, eps, resid, 1.0, 1.0, gain,
                                      out, xn, None)


def test_combine_norm_rejects_bad_arguments():
    assert _cn(flags=4) == INVALID
    assert _cn(flags=1, eps=-1.0) == INVALID
    assert _cn(flags=1, eps=float("inf")) == INVALID
    assert _cn(flags=1, eps=float("nan")) == INVALID
    assert _cn(flags=3, resid=None) == INVALID
    assert _cn(flags=2, gain=None) == INVALID
    assert _cn(flags=2, xn=None) == INVALID
    assert _cn(flags=2, xn=A + 8) == INVALID
    assert _cn(flags=2, resid=A + 4) == INVALID
    assert _cn(out=A + 4) == INVALID
    assert _cn(y=None) == INVALID
    assert _cn(yd=2) == INVALID
    assert _cn(T=0) == INVALID
    assert _cn(H=200) == SHAPE
    assert _cn(H=65536 + 128) == SHAPE


def test_python_binding_validates_before_calling():
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.route(x, torch.zeros(256, 8), None, 2, torch.zeros(4, 2, dtype=torch.int32),
                  torch.zeros(4, 2), torch.zeros(16, dtype=torch.uint8))


def test_pack_rejects_bad_arguments():
    p = moe.lib().moe_nvfp4_pack
    B = A + (1 << 40)  # a second, non-overlapping fake region
    C, D = A + (2 << 40), A + (3 << 40)
    assert p(None, A, 2, 16, 128, B, C, None) == INVALID
    assert p(A, B, 2, 16, 128, C + 4, D, None) == INVALID
    assert p(A, B, 0, 16, 128, C, D, None) == INVALID
    assert p(A, B, 2, 24, 128, C, D, None) == SHAPE
    assert p(A, B, 2, 16, 96, C, D, None) == SHAPE
    assert p(A, B, 2, 16, 128, A, D, None) == INVALID  # in place


def test_nvfp4_to_mxfp8_rejects_bad_arguments():
    f = moe.lib().moe_nvfp4_to_mxfp8
    B, C, D, F = A + (1 << 40), A + (2 << 40), A + (3 << 40), A + (4 << 40)
    assert f(None, B, C, 0, 2, 32, 256, D, F, None) == INVALID
    assert f(A, B, None, 0, 2, 32, 256, D, F, None) == INVALID
    assert f(A, B, C, 3, 2, 32, 256, D, F, None) == INVALID  # matrix
    assert f(A, B, C, -1, 2, 32, 256, D, F, None) == INVALID
    assert f(A, B, C, 0, 0, 32, 256, D, F, None) == INVALID
    assert f(A, B, C, 0, 2, 32, 256, D + 8, F, None) == INVALID  # alignment
    assert f(A, B, C, 0, 2, 16, 256, D, F, None) == SHAPE  # N % 32
    assert f(A, B, C, 0, 2, 32, 128, D, F, None) == SHAPE  # K % 256
    assert f(A, B, C, 0, 300, 32, 256, D, F, None) == SHAPE
    assert f(A, B, C, 0, 2, 32, 256, A, F, None) == INVALID  # output over the input codes
    assert f(A, B, C, 0, 2, 32, 256, D, B, None) == INVALID  # output over the input scales
    assert f(A, B, C, 0, 2, 32, 256, D, D + 256, None) == INVALID  # outputs overlap


def _mx8(**over):
    a = dict(x=A, ex=moe._Mx8Experts(A, A, A, A, A, A, 8, 256, 256), T=4, k=2, y=A, ws=A,
             ws_bytes=1 << 30)
    a.update(over)
    return moe.lib().moe_expert_ffn_mx8(a["x"], ctypes.byref(a["ex"]), A, A, A, A, A, a["T"],
                                        a["k"], a["y"], a["ws"], a["ws_bytes"], None)


def test_expert_ffn_mx8_rejects_bad_arguments():
    assert _mx8(x=None) == INVALID
    assert _mx8(y=A + 2) == INVALID
    assert _mx8(ex=moe._Mx8Experts(A, None, A, A, A, A, 8, 256, 256)) == INVALID
    assert _mx8(T=0) == INVALID
    assert _mx8(k=9) == INVALID
    assert _mx8(ex=moe._Mx8Experts(A, A, A, A, A, A, 8, 384, 256)) == SHAPE  # H % 256
    assert _mx8(ex=moe._Mx8Experts(A, A, A, A, A, A, 8, 256, 128)) == SHAPE  # I % 256
    assert _mx8(ws_bytes=1024) == WS


def _layer(**over):
    ex = moe._Experts(A, A, A, A, A, A, A, 8, 256, 128)
    a = dict(x=A, wr=A, bias=None, ex=ex, T=1, k=2, logits=None, out=A, y=A, ydt=0, ws=A,
             ws_bytes=1 << 30, topk=A)
    a.update(over)
    return moe.lib().moe_layer_nvfp4(a["x"], a["wr"], a["bias"], ctypes.byref(a["ex"]), a["T"],
                                     a["k"], a["logits"], a["topk"], A, A, A, A, A, A, A, a["y"],
                                     a["ydt"], a["out"], a["ws"], a["ws_bytes"], None)


def test_layer_rejects_bad_arguments():
    assert _layer(x=None) == INVALID
    assert _layer(out=None) == INVALID
    assert _layer(y=None) == INVALID
    assert _layer(topk=A + 4) == INVALID
    assert _layer(ydt=5) == INVALID
    assert _layer(k=9) == INVALID
    assert _layer(ex=moe._Experts(A, A, A, A, A, A, None, 8, 256, 128)) == INVALID
    assert _layer(ex=moe._Experts(A, A, A, A, A, A, A, 8, 250, 128)) == SHAPE
    assert _layer(ws_bytes=1024) == WS


def test_ffn_and_layer_reject_offsets_beyond_32_bits():
    # T*k*I = 2^32: the down GEMM's h offsets would wrap
    big = _experts(E=256, H=256, I=2048)
    assert _ffn(big, T=262144, k=8) == SHAPE
    assert _layer(ex=moe._Experts(A, A, A, A, A, A, A, 256, 256, 2048), T=262144, k=8) == SHAPE
    ex = moe._Mx8Experts(A, A, A, A, A, A, 256, 256, 2048)
    assert _mx8(ex=ex, T=262144, k=8) == SHAPE


def test_layer_check_rejects_bad_arguments():
    c = moe.lib().moe_layer_check
    assert c(None, 1 << 20, None) == INVALID
    assert c(A + 4, 1 << 20, None) == INVALID
    assert c(A, 1024, None) == WS


def test_workspace_leaves_room_for_the_sync_words():
    # the single-launch layer's counters and flags occupy the first 64 KiB; every region follows
    for T in (1, 2, 64):
        assert moe.workspace_size(T, 7168, 2048, 256, 8) >= 65536 + T * 7168 * 2


def test_layer_noalloc_refuses_shapes_beyond_its_scratch():
    # refused on the host, before the library looks up its scratch array on the device
    ex = moe._Experts(A, A, A, A, A, A, A, 256, 7168, 2048)
    assert moe.workspace_size(4096, 7168, 2048, 256, 8) > 16 << 20
    st = moe.lib().moe_layer_nvfp4_noalloc(A, A, None, ctypes.byref(ex), 4096, 8, None, A, A, A,
                                           A, A, A, A, A, A, 1, A, None)
    assert st == -7
