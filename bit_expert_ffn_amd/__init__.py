"""Python binding of libmoe_nvfp4.so: one NVFP4 sparse-MoE FFN layer on MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.  torch is
used for device memory and streams.  The functions mirror the C ABI in include/moe_nvfp4.h
(same names without the `moe_` prefix); they check dtype, device, shape and contiguity, raise
ValueError on bad arguments and RuntimeError with the library's status text on a failing call.
There is no fallback: if the library is missing, loading it raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_nvfp4.so")

MOE_F32 = 0
MOE_F16 = 1
MOE_COMBINE_EXPERT_NORM = 1
MOE_COMBINE_RESIDUAL_NORM = 2
_lib = None


class _Experts(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32)]


class _Mx8Experts(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32)]


def lib():
    """The loaded library (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_nvfp4.so not found at %s: build it first "
                               "(python -m bit_expert_ffn_amd.build)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_abi_version.restype = i32
        L.moe_abi_version.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_workspace_size.restype = sz
        L.moe_workspace_size.argtypes = [i32] * 5
        L.moe_route.restype = i32
        L.moe_route.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_group.restype = i32
        L.moe_group.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn_nvfp4.restype = i32
        L.moe_expert_ffn_nvfp4.argtypes = [vp, ctypes.POINTER(_Experts), vp, vp, vp, vp, vp,
                                           i32, i32, vp, i32, vp, sz, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp]
        L.moe_combine_norm.restype = i32
        L.moe_combine_norm.argtypes = [vp, i32, vp, vp, i32, i32, i32, ctypes.c_uint32,
                                       ctypes.c_float, vp, ctypes.c_float, ctypes.c_float, vp,
                                       vp, vp, vp]
        L.moe_nvfp4_pack.restype = i32
        L.moe_nvfp4_pack.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.moe_layer_nvfp4.restype = i32
        L.moe_layer_nvfp4.argtypes = [vp, vp, vp, ctypes.POINTER(_Experts), i32, i32, vp, vp,
                                      vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_nvfp4_to_mxfp8.restype = i32
        L.moe_nvfp4_to_mxfp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_layer_nvfp4_noalloc.restype = i32
        L.moe_layer_nvfp4_noalloc.argtypes = [vp, vp, vp, ctypes.POINTER(_Experts), i32, i32,
                                              vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                              vp]
        L.moe_layer_check.restype = i32
        L.moe_layer_check.argtypes = [vp, sz, vp]
        L.moe_expert_ffn_mx8.restype = i32
        L.moe_expert_ffn_mx8.argtypes = [vp, ctypes.POINTER(_Mx8Experts), vp, vp, vp, vp, vp,
                                         i32, i32, vp, vp, sz, vp]
        _lib = L
    return _lib


EXPORTED = ("moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_route",
            "moe_group", "moe_expert_ffn_nvfp4", "moe_combine", "moe_combine_norm",
            "moe_nvfp4_pack", "moe_layer_nvfp4", "moe_layer_nvfp4_noalloc", "moe_layer_check",
            "moe_nvfp4_to_mxfp8", "moe_expert_ffn_mx8")


def abi_version():
    return lib().moe_abi_version()


def status_string(code):
    return lib().moe_status_string(int(code)).decode()


def workspace_size(T, H, I, E, k):
    """Bytes of scratch workspace one layer call of these sizes needs."""
    return int(lib().moe_workspace_size(T, H, I, E, k))


def _check(code, what):
    if code != 0:
        raise RuntimeError("%s failed: %d (%s)" % (what, code, status_string(code)))


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def route(x, w_router, bias, k, topk_id, topk_w, ws, logits=None, stream=None):
    """moe_route: x [T][H] bf16, w_router [H][E] fp32, bias [E] fp32 or None ->
    topk_id [T][k] int32, topk_w [T][k] fp32 (and logits [T][E] fp32 if given)."""
    T, H = x.shape
    E = w_router.shape[1]
    args = (_dev(x, "x", torch.bfloat16), _dev(w_router, "w_router", torch.float32, (H, E)),
            None if bias is None else _dev(bias, "bias", torch.float32, (E,)), T, H, E, k,
            None if logits is None else _dev(logits, "logits", torch.float32, (T, E)),
            _dev(topk_id, "topk_id", torch.int32, (T, k)),
            _dev(topk_w, "topk_w", torch.float32, (T, k)), _dev(ws, "ws", torch.uint8),
            ws.numel(), _stream(stream, x.device))
    _check(lib().moe_route(*args), "moe_route")


def group(topk_id, E, count, offset, sorted_slot, slot_row, active, n_active, ws, stream=None):
    """moe_group: stable grouping of the T*k slots by expert (outputs are int32 tensors)."""
    T, k = topk_id.shape
    n = T * k
    args = (_dev(topk_id, "topk_id", torch.int32), T, k, E,
            _dev(count, "count", torch.int32, (E,)), _dev(offset, "offset", torch.int32, (E + 1,)),
            _dev(sorted_slot, "sorted_slot", torch.int32, (n,)),
            _dev(slot_row, "slot_row", torch.int32, (n,)),
            _dev(active, "active", torch.int32, (E,)),
            _dev(n_active, "n_active", torch.int32, (1,)), _dev(ws, "ws", torch.uint8),
            ws.numel(), _stream(stream, topk_id.device))
    _check(lib().moe_group(*args), "moe_group")


def nvfp4_pack(q, s, q_out=None, s_out=None, stream=None):
    """moe_nvfp4_pack: row-major codes q [E][N][K/2] and scales s [E][N][K/16] (uint8, on the
    GPU) -> tile-major tensors of the same shapes (new tensors unless given)."""
    E, N, k2 = q.shape
    K = k2 * 2
    if q_out is None:
        q_out = torch.empty_like(q)
    if s_out is None:
        s_out = torch.empty_like(s)
    args = (_dev(q, "q", torch.uint8, (E, N, K // 2)), _dev(s, "s", torch.uint8, (E, N, K // 16)),
            E, N, K, _dev(q_out, "q_out", torch.uint8, (E, N, K // 2)),
            _dev(s_out, "s_out", torch.uint8, (E, N, K // 16)), _stream(stream, q.device))
    _check(lib().moe_nvfp4_pack(*args), "moe_nvfp4_pack")
    return q_out, s_out


def pack_experts(experts, stream=None):
    """Tile-major copy of a dict of row-major NVFP4 expert tensors (see experts_struct)."""
    out = {"ts": experts["ts"]}
    for m in ("gate", "up", "down"):
        out[m + "_q"], out[m + "_s"] = nvfp4_pack(experts[m + "_q"], experts[m + "_s"],
                                                  stream=stream)
    return out


def experts_struct(experts):
    """ctypes struct for a dict of tile-major NVFP4 expert tensors (gate_q, up_q, down_q,
    gate_s, up_s, down_s: uint8 with the row-major shapes [E][N][K/2] / [E][N][K/16];
    ts: [E][3] float32)."""
    E, I, h2 = experts["gate_q"].shape
    H = h2 * 2
    shapes = dict(gate_q=(E, I, H // 2), up_q=(E, I, H // 2), down_q=(E, H, I // 2),
                  gate_s=(E, I, H // 16), up_s=(E, I, H // 16), down_s=(E, H, I // 16))
    ptr = {n: _dev(experts[n], n, torch.uint8, s) for n, s in shapes.items()}
    ts = _dev(experts["ts"], "ts", torch.float32, (E, 3))
    return _Experts(ptr["gate_q"], ptr["up_q"], ptr["down_q"], ptr["gate_s"], ptr["up_s"],
                    ptr["down_s"], ts, E, H, I)


def expert_ffn_nvfp4(x, experts, count, offset, sorted_slot, active, n_active, k, y, ws,
                     stream=None):
    """moe_expert_ffn_nvfp4: y [T*k][H] (float32 or float16) in grouped row order."""
    T, H = x.shape
    s = experts_struct(experts)
    if s.H != H:
        raise ValueError("x hidden size %d does not match experts %d" % (H, s.H))
    if y.dtype == torch.float32:
        yd = MOE_F32
    elif y.dtype == torch.float16:
        yd = MOE_F16
    else:
        raise ValueError("y must be float32 or float16")
    E = s.E
    args = (_dev(x, "x", torch.bfloat16), ctypes.byref(s), _dev(count, "count", torch.int32, (E,)),
            _dev(offset, "offset", torch.int32, (E + 1,)),
            _dev(sorted_slot, "sorted_slot", torch.int32, (T * k,)),
            _dev(active, "active", torch.int32, (E,)),
            _dev(n_active, "n_active", torch.int32, (1,)), T, k,
            _dev(y, "y", y.dtype, (T * k, H)), yd, _dev(ws, "ws", torch.uint8), ws.numel(),
            _stream(stream, x.device))
    _check(lib().moe_expert_ffn_nvfp4(*args), "moe_expert_ffn_nvfp4")


_MATRIX = {"gate": 0, "up": 1, "down": 2}


def nvfp4_to_mxfp8(q, s, ts, matrix, q8=None, s8=None, stream=None):
    """moe_nvfp4_to_mxfp8: row-major NVFP4 codes q [E][N][K/2] and scales s [E][N][K/16]
    (uint8), tensor scales ts [E][3] float32 and matrix "gate", "up" or "down" -> MXFP8 codes
    q8 [E][N][K] and scales s8 [E][N][K/32] (uint8, new tensors unless given) in the tile
    layout the fp8 FFN reads (the tensor shapes give sizes only)."""
    E, N, k2 = q.shape
    K = k2 * 2
    if matrix not in _MATRIX:
        raise ValueError("matrix must be gate, up or down")
    if q8 is None:
        q8 = torch.empty((E, N, K), dtype=torch.uint8, device=q.device)
    if s8 is None:
        s8 = torch.empty((E, N, K // 32), dtype=torch.uint8, device=q.device)
    args = (_dev(q, "q", torch.uint8, (E, N, K // 2)), _dev(s, "s", torch.uint8, (E, N, K // 16)),
            _dev(ts, "ts", torch.float32, (E, 3)), _MATRIX[matrix], E, N, K,
            _dev(q8, "q8", torch.uint8, (E, N, K)), _dev(s8, "s8", torch.uint8, (E, N, K // 32)),
            _stream(stream, q.device))
    _check(lib().moe_nvfp4_to_mxfp8(*args), "moe_nvfp4_to_mxfp8")
    return q8, s8


def mx8_experts(experts, stream=None):
    """MXFP8 copy (dict gate_q, up_q, down_q, gate_s, up_s, down_s) of a dict of ROW-MAJOR NVFP4
    expert tensors (gate_q, up_q, down_q, gate_s, up_s, down_s, ts)."""
    out = {}
    for m in ("gate", "up", "down"):
        out[m + "_q"], out[m + "_s"] = nvfp4_to_mxfp8(experts[m + "_q"], experts[m + "_s"],
                                                      experts["ts"], m, stream=stream)
    return out


def mx8_struct(mx8):
    """ctypes struct for a dict of MXFP8 expert tensors as mx8_experts returns."""
    E, I, H = mx8["gate_q"].shape
    shapes = dict(gate_q=(E, I, H), up_q=(E, I, H), down_q=(E, H, I),
                  gate_s=(E, I, H // 32), up_s=(E, I, H // 32), down_s=(E, H, I // 32))
    ptr = {n: _dev(mx8[n], n, torch.uint8, s) for n, s in shapes.items()}
    return _Mx8Experts(ptr["gate_q"], ptr["up_q"], ptr["down_q"], ptr["gate_s"], ptr["up_s"],
                       ptr["down_s"], E, H, I)


def expert_ffn_mx8(x, mx8, count, offset, sorted_slot, active, n_active, k, y, ws, stream=None):
    """moe_expert_ffn_mx8: y [T*k][H] float16 in grouped row order (fp8 compute)."""
    T, H = x.shape
    s = mx8_struct(mx8)
    if s.H != H:
        raise ValueError("x hidden size %d does not match experts %d" % (H, s.H))
    E = s.E
    args = (_dev(x, "x", torch.bfloat16), ctypes.byref(s), _dev(count, "count", torch.int32, (E,)),
            _dev(offset, "offset", torch.int32, (E + 1,)),
            _dev(sorted_slot, "sorted_slot", torch.int32, (T * k,)),
            _dev(active, "active", torch.int32, (E,)),
            _dev(n_active, "n_active", torch.int32, (1,)), T, k,
            _dev(y, "y", torch.float16, (T * k, H)), _dev(ws, "ws", torch.uint8), ws.numel(),
            _stream(stream, x.device))
    _check(lib().moe_expert_ffn_mx8(*args), "moe_expert_ffn_mx8")


def combine(y, slot_row, topk_w, out, stream=None):
    """moe_combine: out [T][H] fp32 = routing-weighted sum of each token's k expert rows."""
    T, k = topk_w.shape
    H = y.shape[1]
    yd = MOE_F16 if y.dtype == torch.float16 else MOE_F32
    args = (_dev(y, "y", y.dtype, (T * k, H)), yd, _dev(slot_row, "slot_row", torch.int32, (T * k,)),
            _dev(topk_w, "topk_w", torch.float32, (T, k)), T, k, H,
            _dev(out, "out", torch.float32, (T, H)), _stream(stream, y.device))
    _check(lib().moe_combine(*args), "moe_combine")


def combine_norm(y, slot_row, topk_w, out, expert_norm=False, resid=None, alpha=1.0, beta=1.0,
                 gain=None, x_next=None, eps=1e-6, stream=None):
    """moe_combine_norm: the weighted sum with a per-expert RMS norm of each expert row
    (expert_norm) and, when resid is given, the epilogue out = alpha * resid + beta * s * f with
    s = f's RMS factor, x_next [T][H] bf16 = gain * RMS-norm(out).  resid may be out itself."""
    T, k = topk_w.shape
    H = y.shape[1]
    yd = MOE_F16 if y.dtype == torch.float16 else MOE_F32
    flags = MOE_COMBINE_EXPERT_NORM if expert_norm else 0
    epi = (None, None, None)
    if resid is not None:
        flags |= MOE_COMBINE_RESIDUAL_NORM
        epi = (_dev(resid, "resid", torch.float32, (T, H)), _dev(gain, "gain", torch.float32, (H,)),
               _dev(x_next, "x_next", torch.bfloat16, (T, H)))
    args = (_dev(y, "y", y.dtype, (T * k, H)), yd, _dev(slot_row, "slot_row", torch.int32, (T * k,)),
            _dev(topk_w, "topk_w", torch.float32, (T, k)), T, k, H, flags, float(eps), epi[0],
            float(alpha), float(beta), epi[1], _dev(out, "out", torch.float32, (T, H)), epi[2],
            _stream(stream, y.device))
    _check(lib().moe_combine_norm(*args), "moe_combine_norm")


class LayerBuffers:
    """Device buffers for one layer call of given sizes (plain torch allocations)."""

    def __init__(self, T, H, I, E, k, device="cuda", y_dtype=torch.float32, logits=True):
        d = torch.device(device)
        i32 = dict(dtype=torch.int32, device=d)
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.logits = torch.empty((T, E), dtype=torch.float32, device=d) if logits else None
        self.topk_id = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.count = torch.empty(E, **i32)
        self.offset = torch.empty(E + 1, **i32)
        self.sorted_slot = torch.empty(T * k, **i32)
        self.slot_row = torch.empty(T * k, **i32)
        self.active = torch.empty(E, **i32)
        self.n_active = torch.empty(1, **i32)
        self.y = torch.empty((T * k, H), dtype=y_dtype, device=d)
        self.out = torch.empty((T, H), dtype=torch.float32, device=d)
        n = workspace_size(T, H, I, E, k)
        if n == 0:
            raise ValueError("unsupported layer shape T=%d H=%d I=%d E=%d k=%d" % (T, H, I, E, k))
        # zero-filled: the single-launch layer's counters and flags live in the first 64 KiB
        self.ws = torch.zeros(n, dtype=torch.uint8, device=d)


def layer(x, w_router, bias, experts, k, buf, stream=None):
    """The four calls in order; results are left in `buf` (out, topk ids/weights, grouping, y)."""
    route(x, w_router, bias, k, buf.topk_id, buf.topk_w, buf.ws, logits=buf.logits, stream=stream)
    group(buf.topk_id, w_router.shape[1], buf.count, buf.offset, buf.sorted_slot, buf.slot_row,
          buf.active, buf.n_active, buf.ws, stream=stream)
    expert_ffn_nvfp4(x, experts, buf.count, buf.offset, buf.sorted_slot, buf.active,
                     buf.n_active, k, buf.y, buf.ws, stream=stream)
    combine(buf.y, buf.slot_row, buf.topk_w, buf.out, stream=stream)
    return buf.out


def layer_nvfp4(x, w_router, bias, experts, k, buf, stream=None):
    """moe_layer_nvfp4: the whole layer in one call (one persistent kernel for one or two
    tokens).  Results are left in `buf` like layer(); buf.y is written only by the four-call
    path."""
    prepare_layer_nvfp4(x, w_router, bias, experts, k, buf, stream)()
    return buf.out


def layer_nvfp4_noalloc(x, w_router, bias, experts, k, buf, stream=None):
    """moe_layer_nvfp4_noalloc: as layer_nvfp4, with the library's own per-GPU scratch instead of
    buf.ws (which is not used).  Results are left in `buf`."""
    T, H = x.shape
    s = experts_struct(experts)
    E = s.E
    if s.H != H or w_router.shape != (H, E):
        raise ValueError("x, w_router and experts disagree on H or E")
    y = buf.y
    yd = MOE_F16 if y.dtype == torch.float16 else MOE_F32
    n = T * k
    args = (_dev(x, "x", torch.bfloat16), _dev(w_router, "w_router", torch.float32, (H, E)),
            None if bias is None else _dev(bias, "bias", torch.float32, (E,)), ctypes.byref(s),
            T, k, None if buf.logits is None else _dev(buf.logits, "logits", torch.float32, (T, E)),
            _dev(buf.topk_id, "topk_id", torch.int32, (T, k)),
            _dev(buf.topk_w, "topk_w", torch.float32, (T, k)),
            _dev(buf.count, "count", torch.int32, (E,)),
            _dev(buf.offset, "offset", torch.int32, (E + 1,)),
            _dev(buf.sorted_slot, "sorted_slot", torch.int32, (n,)),
            _dev(buf.slot_row, "slot_row", torch.int32, (n,)),
            _dev(buf.active, "active", torch.int32, (E,)),
            _dev(buf.n_active, "n_active", torch.int32, (1,)),
            _dev(y, "y", y.dtype, (n, H)), yd, _dev(buf.out, "out", torch.float32, (T, H)),
            _stream(stream, x.device))
    _check(lib().moe_layer_nvfp4_noalloc(*args), "moe_layer_nvfp4_noalloc")
    return buf.out


def layer_check(ws, stream=None):
    """moe_layer_check: waits for the stream, then raises RuntimeError if a wait inside an
    earlier single-launch layer call on this workspace gave up (that call's outputs are
    undefined; the library has cleared the workspace's sync region for the next call)."""
    _check(lib().moe_layer_check(_dev(ws, "ws", torch.uint8), ws.numel(),
                                 _stream(stream, ws.device)), "moe_layer_check")


def set_layer_spin_limit(ws, polls):
    """Sets the number of polls after which a wait of the single-launch layer gives up (word 49
    of the workspace; 0 = the library's default of about 2 s).  Ordered on the current stream."""
    ws[:256].view(torch.int32)[49] = int(polls)


def prepare_layer_nvfp4(x, w_router, bias, experts, k, buf, stream=None):
    """Checks and marshals the arguments of moe_layer_nvfp4 once and returns a callable that
    makes the call (raising on a non-zero status).  For repeated calls on the same tensors,
    e.g. a decode loop, where per-call argument checking would cost more host time than the
    layer takes on the GPU."""
    T, H = x.shape
    s = experts_struct(experts)
    E = s.E
    if s.H != H or w_router.shape != (H, E):
        raise ValueError("x, w_router and experts disagree on H or E")
    y = buf.y
    yd = MOE_F16 if y.dtype == torch.float16 else MOE_F32
    n = T * k
    args = (_dev(x, "x", torch.bfloat16), _dev(w_router, "w_router", torch.float32, (H, E)),
            None if bias is None else _dev(bias, "bias", torch.float32, (E,)), ctypes.byref(s),
            T, k, None if buf.logits is None else _dev(buf.logits, "logits", torch.float32, (T, E)),
            _dev(buf.topk_id, "topk_id", torch.int32, (T, k)),
            _dev(buf.topk_w, "topk_w", torch.float32, (T, k)),
            _dev(buf.count, "count", torch.int32, (E,)),
            _dev(buf.offset, "offset", torch.int32, (E + 1,)),
            _dev(buf.sorted_slot, "sorted_slot", torch.int32, (n,)),
            _dev(buf.slot_row, "slot_row", torch.int32, (n,)),
            _dev(buf.active, "active", torch.int32, (E,)),
            _dev(buf.n_active, "n_active", torch.int32, (1,)),
            _dev(y, "y", y.dtype, (n, H)), yd, _dev(buf.out, "out", torch.float32, (T, H)),
            _dev(buf.ws, "ws", torch.uint8), buf.ws.numel(), _stream(stream, x.device))
    fn = lib().moe_layer_nvfp4
    keep = (s,)  # the experts struct must outlive the callable

    def call():
        code = fn(*args)
        if code != 0:
            _check(code, "moe_layer_nvfp4")
        return keep

    return call
