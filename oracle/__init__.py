"""CPU oracle for the NVFP4 sparse-MoE FFN layer (ctypes wrapper around oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this module; the product package never does.  It shares no code with the HIP
library.  Parity pins: tests/test_oracle.py.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=False):
    """Compile oracle.c with gcc (IEEE double, no fast-math) into liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


class _Experts(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("ts", ctypes.c_void_p), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _lib.oracle_e2m1.restype = ctypes.c_double
        _lib.oracle_e4m3.restype = ctypes.c_double
        _lib.oracle_bf16.restype = ctypes.c_double
        _lib.oracle_bf16.argtypes = [ctypes.c_uint16]
        _lib.oracle_weight.restype = ctypes.c_double
        _lib.oracle_weight.argtypes = [ctypes.POINTER(_Experts)] + [ctypes.c_int] * 4
        _lib.oracle_threads.restype = ctypes.c_int
        _lib.oracle_mx_exp.restype = ctypes.c_int
        _lib.oracle_e4m3_code.restype = ctypes.c_int
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class Experts:
    """NVFP4 expert weights in the library's byte format, held as numpy arrays."""

    def __init__(self, gate_q, up_q, down_q, gate_s, up_s, down_s, ts):
        self.gate_q = _c(gate_q, np.uint8)
        self.up_q = _c(up_q, np.uint8)
        self.down_q = _c(down_q, np.uint8)
        self.gate_s = _c(gate_s, np.uint8)
        self.up_s = _c(up_s, np.uint8)
        self.down_s = _c(down_s, np.uint8)
        self.ts = _c(ts, np.float32)
        self.E, self.I, h2 = self.gate_q.shape
        self.H = h2 * 2
        assert self.down_q.shape == (self.E, self.H, self.I // 2)
        assert self.gate_s.shape == (self.E, self.I, self.H // 16)
        assert self.down_s.shape == (self.E, self.H, self.I // 16)
        assert self.ts.shape == (self.E, 3)

    def _struct(self):
        return _Experts(self.gate_q.ctypes.data, self.up_q.ctypes.data, self.down_q.ctypes.data,
                        self.gate_s.ctypes.data, self.up_s.ctypes.data, self.down_s.ctypes.data,
                        self.ts.ctypes.data, self.E, self.H, self.I)


def e2m1(code):
    return _load().oracle_e2m1(int(code))


def e4m3(code):
    return _load().oracle_e4m3(int(code))


def bf16(bits):
    return _load().oracle_bf16(int(bits))


def threads():
    return _load().oracle_threads()


def weight(experts, e, m, n, kk):
    s = experts._struct()
    return _load().oracle_weight(ctypes.byref(s), e, m, n, kk)


def dequant(experts, e, m):
    """Whole dequantised matrix m (0 gate, 1 up, 2 down) of expert e, float64 [N][K]."""
    N = experts.H if m == 2 else experts.I
    K = experts.I if m == 2 else experts.H
    q = (experts.gate_q, experts.up_q, experts.down_q)[m][e]
    s = (experts.gate_s, experts.up_s, experts.down_s)[m][e]
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = q & 15
    codes[:, 1::2] = q >> 4
    t2 = np.array([e2m1(c) for c in range(16)])
    t8 = np.array([e4m3(c) for c in range(256)])
    scale = np.repeat(t8[s.astype(np.int64)], 16, axis=1)
    return t2[codes] * scale * float(experts.ts[e, m])


def router(x_bits, w_router, bias=None):
    x_bits = _c(x_bits, np.uint16)
    w_router = _c(w_router, np.float32)
    T, H = x_bits.shape
    E = w_router.shape[1]
    out = np.empty((T, E), np.float32)
    b = _c(bias, np.float32) if bias is not None else None
    _load().oracle_router(_p(x_bits), _p(w_router), _p(b), T, H, E, _p(out))
    return out


def topk(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_topk(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def group(topk_id, E):
    topk_id = _c(topk_id, np.int32)
    T, k = topk_id.shape
    n = T * k
    count = np.empty(E, np.int32)
    offset = np.empty(E + 1, np.int32)
    sorted_slot = np.empty(n, np.int32)
    slot_row = np.empty(n, np.int32)
    active = np.empty(E, np.int32)
    n_active = np.empty(1, np.int32)
    _load().oracle_group(_p(topk_id), T, k, E, _p(count), _p(offset), _p(sorted_slot),
                         _p(slot_row), _p(active), _p(n_active))
    return dict(count=count, offset=offset, sorted_slot=sorted_slot, slot_row=slot_row,
                active=active, n_active=int(n_active[0]))


def expert_rows(x_bits, experts, e, tokens):
    x_bits = _c(x_bits, np.uint16)
    tok = _c(tokens, np.int32)
    y = np.empty((len(tok), experts.H), np.float64)
    s = experts._struct()
    _load().oracle_expert_rows(_p(x_bits), experts.H, ctypes.byref(s), int(e), _p(tok),
                               len(tok), _p(y))
    return y


def expert_hidden(x_bits, experts, e, tokens):
    x_bits = _c(x_bits, np.uint16)
    tok = _c(tokens, np.int32)
    h = np.empty((len(tok), experts.I), np.float64)
    s = experts._struct()
    _load().oracle_expert_hidden(_p(x_bits), experts.H, ctypes.byref(s), int(e), _p(tok),
                                 len(tok), _p(h))
    return h


def ffn(x_bits, experts, grouping, k):
    """y [T*k][H] (float64) in grouped row order, from the oracle's own grouping."""
    off = grouping["offset"]
    ss = grouping["sorted_slot"]
    y = np.empty((len(ss), experts.H), np.float64)
    for e in range(experts.E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            y[a:b] = expert_rows(x_bits, experts, e, ss[a:b] // k)
    return y


def combine(y, slot_row, topk_w, k, H):
    y = _c(y, np.float64)
    slot_row = _c(slot_row, np.int32)
    topk_w = _c(topk_w, np.float64)
    T = topk_w.shape[0]
    out = np.empty((T, H), np.float64)
    _load().oracle_combine(_p(y), _p(slot_row), _p(topk_w), T, k, H, _p(out))
    return out


def combine_norm(y, slot_row, topk_w, k, H, expert_norm=False, resid=None, alpha=1.0,
                 beta=1.0, gain=None, eps=1e-6):
    """Combine variants in fp64: per-expert RMS norm before the weighted sum (expert_norm) and,
    when resid is given, the post-norm + scaled residual + next pre-norm epilogue.  Returns a
    dict: f (the combined MoE output), out (new residual, or f without the epilogue) and, with
    the epilogue, s and r (per-token norm factors) and xn (the next layer's input, unrounded)."""
    y = _c(y, np.float64)
    slot_row = _c(slot_row, np.int32)
    topk_w = _c(topk_w, np.float64)
    T = topk_w.shape[0]
    epi = resid is not None
    f = np.empty((T, H), np.float64)
    out = np.empty((T, H), np.float64)
    res = dict(f=f, out=out)
    args = [None] * 5
    if epi:
        resid = _c(resid, np.float64)
        gain = _c(gain, np.float64)
        res.update(s=np.empty(T), r=np.empty(T), xn=np.empty((T, H)))
        args = [resid, gain, res["s"], res["r"], res["xn"]]
    _load().oracle_combine_norm(
        _p(y), _p(slot_row), _p(topk_w), T, k, H, int(expert_norm), int(epi),
        ctypes.c_double(eps), _p(args[0]), ctypes.c_double(alpha), ctypes.c_double(beta),
        _p(args[1]), _p(f), _p(args[2]), _p(out), _p(args[3]), _p(args[4]))
    return res


def layer(x_bits, w_router, bias, experts, k):
    """Whole layer on every token: dict of logits, topk ids/weights, grouping, y, out."""
    logits = router(x_bits, w_router, bias)
    ids, w = topk(logits, k)
    g = group(ids, experts.E)
    y = ffn(x_bits, experts, g, k)
    out = combine(y, g["slot_row"], w, k, experts.H)
    return dict(logits=logits, topk_id=ids, topk_w=w, group=g, y=y, out=out)


def layer_tokens(x_bits, w_router, bias, experts, k, tokens):
    """Whole layer for the listed tokens only (exact: routing and FFN are per token)."""
    x_bits = _c(x_bits, np.uint16)
    w_router = _c(w_router, np.float32)
    b = _c(bias, np.float32) if bias is not None else None
    tok = _c(tokens, np.int32)
    n = len(tok)
    E = w_router.shape[1]
    H = x_bits.shape[1]
    logits = np.empty((n, E), np.float32)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    out = np.empty((n, H), np.float64)
    s = experts._struct()
    _load().oracle_layer_tokens(_p(x_bits), _p(w_router), _p(b), ctypes.byref(s), H, E, k,
                                _p(tok), n, _p(logits), _p(ids), _p(w), _p(out))
    return dict(logits=logits, topk_id=ids, topk_w=w, out=out)


# ------------------------------------------------------------ low precision: fp8 compute (MX)
def mx_exp(amax, emax):
    return _load().oracle_mx_exp(ctypes.c_double(amax), int(emax))


def e4m3_code(v):
    return _load().oracle_e4m3_code(ctypes.c_double(v))


def mx_scale(byte):
    return 2.0 ** (int(byte) - 127)


def mx8_quant(v):
    """MXFP8 (e4m3 codes, e8m0 scale per 32 consecutive values) of a float64 array whose last
    dimension is a multiple of 32: (codes uint8, scales uint8)."""
    v = _c(v, np.float64)
    shape = v.shape
    flat = v.reshape(-1)
    codes = np.empty(flat.size, np.uint8)
    scales = np.empty(flat.size // 32, np.uint8)
    _load().oracle_mx8_quant(_p(flat), flat.size, _p(codes), _p(scales))
    return codes.reshape(shape), scales.reshape(shape[:-1] + (shape[-1] // 32,))


def mx8_dequant(codes, scales):
    t8 = np.array([e4m3(c) for c in range(256)])
    v = t8[np.asarray(codes, np.int64)]
    return v * np.repeat(2.0 ** (np.asarray(scales, np.int64) - 127), 32, axis=-1)


class Mx8Experts:
    """MXFP8 expert weights, logical row-major: *_q [E][N][K] e4m3 codes, *_s [E][N][K/32] e8m0
    scale bytes; gate/up N = I, K = H; down N = H, K = I."""

    def __init__(self, gate_q, up_q, down_q, gate_s, up_s, down_s):
        self.gate_q, self.up_q, self.down_q = (_c(a, np.uint8) for a in (gate_q, up_q, down_q))
        self.gate_s, self.up_s, self.down_s = (_c(a, np.uint8) for a in (gate_s, up_s, down_s))
        self.E, self.I, self.H = self.gate_q.shape


def nvfp4_to_mxfp8(experts):
    """Requantise every NVFP4 matrix to MXFP8 (tensor scales folded in): Mx8Experts."""
    s = experts._struct()
    out = []
    for m in range(3):
        N = experts.H if m == 2 else experts.I
        K = experts.I if m == 2 else experts.H
        q = np.empty((experts.E, N, K), np.uint8)
        sc = np.empty((experts.E, N, K // 32), np.uint8)
        _load().oracle_nvfp4_to_mxfp8(ctypes.byref(s), m, _p(q), _p(sc))
        out.append((q, sc))
    return Mx8Experts(out[0][0], out[1][0], out[2][0], out[0][1], out[1][1], out[2][1])


def mx8_weights(mx, e, m):
    """Dequantised MXFP8 matrix m of expert e, float64 [N][K]."""
    q = (mx.gate_q, mx.up_q, mx.down_q)[m][e]
    s = (mx.gate_s, mx.up_s, mx.down_s)[m][e]
    return mx8_dequant(q, s)


def expert_rows_mx(x_bits, mx, e, tokens):
    """Expert e's FFN in the fp8 (MX) variant on the listed token rows: y float64 [n][H]."""
    x_bits = _c(x_bits, np.uint16)
    tok = _c(tokens, np.int32)
    y = np.empty((len(tok), mx.H), np.float64)
    _load().oracle_expert_rows_mx(_p(x_bits), mx.H, mx.I, int(e), _p(mx.gate_q), _p(mx.gate_s),
                                  _p(mx.up_q), _p(mx.up_s), _p(mx.down_q), _p(mx.down_s),
                                  _p(tok), len(tok), _p(y))
    return y


def ffn_mx(x_bits, mx, grouping, k):
    """y [T*k][H] (float64) of the fp8 variant in grouped row order."""
    off = grouping["offset"]
    ss = grouping["sorted_slot"]
    y = np.empty((len(ss), mx.H), np.float64)
    for e in range(mx.E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            y[a:b] = expert_rows_mx(x_bits, mx, e, ss[a:b] // k)
    return y
