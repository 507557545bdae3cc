"""Bit-exact GPU decode of every NVFP4 code on every path of the layer.

The format ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", "NVFP4 experts": 4-bit
e2m1 weights with one scale per 16 values; the scale read as OCP E4M3FN) fixes each weight as
e2m1(code) * e4m3(scale) * tensor_scale.  One expert (E = 1, k = 1, H = I = 4096) is built so
that one output element equals one decoded weight exactly:

  down  x = one-hot at hidden column 0; gate and up make h one-hot at feature 5 with h = 1.0
        exactly (g = 4 * 16 = 64, silu(64) = 64 in fp32 and fp64, u = 0.5 * 2^-5 = 1/64); row n
        of the down matrix holds e2m1 code n % 16 at column 5 and e4m3 scale code n // 16 on its
        block, so y[n] = e2m1(n % 16) * e4m3(n // 16): all 16 x 256 code pairs, including the
        e4m3 subnormals 0x01..0x07 and 0x81..0x87, -0 and the NaN codes 0x7F / 0xFF;
  up    every gate row gives g = 64; row i of the up matrix holds code i % 16 with scale code
        i // 16 and the up tensor scale is 2^-6, so h[i] = the decoded up weight exactly; the
        down matrix is the identity, so y[i] = h[i];
  gate  row i of the gate matrix holds code i % 16 with scale code i // 16, u = 1, the down
        matrix is the identity, so y[i] = silu(decoded gate weight) rounded to f16: compared
        within that rounding (a wrong decode moves g by a factor, far outside it).
For up and gate the NaN scale codes are replaced by 0x00 (a NaN h would reach every output
through the zero weights); the down case covers them.

The expected values come from the oracle (whose decode tables are pinned to hand-worked tables
and torch's own fp8 decoder); for down and up they must match bit for bit.  Paths: the
single-launch layer (one and two tokens), the few-row VALU kernels (1 and 4 rows), and the
matrix-core grouped GEMM with 32-, 64- and 128-row tiles (64, 512 and 2048 rows)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

H = I = 4096
COL = 0      # the hidden column that x selects
FEAT = 5     # the intermediate feature that carries h = 1 in the down case
E2M1 = {0.5: 1, 1.0: 2, 4.0: 6}
E4M3 = {2.0 ** -5: 0x10, 1.0: 0x38, 16.0: 0x58}
NAN_SCALES = (0x7F, 0xFF)


def _set(q, s, n, kk, code, scale):
    """Row-major NVFP4 bytes of one weight: code at (n, kk) (low nibble = even kk), scale code of
    its 16-value block."""
    b = int(q[n, kk // 2])
    q[n, kk // 2] = (b & 0xF0) | code if kk % 2 == 0 else (b & 0x0F) | (code << 4)
    s[n, kk // 16] = scale


def _experts(case):
    for v, c in E2M1.items():
        assert oracle.e2m1(c) == v
    for v, c in E4M3.items():
        assert oracle.e4m3(c) == v
    gq = np.zeros((I, H // 2), np.uint8)
    gs = np.zeros((I, H // 16), np.uint8)
    uq, us = gq.copy(), gs.copy()
    dq = np.zeros((H, I // 2), np.uint8)
    ds = np.zeros((H, I // 16), np.uint8)
    ts = np.ones(3, np.float32)
    rows = np.arange(4096)
    codes, scales = rows % 16, rows // 16
    finite = np.where(np.isin(scales, NAN_SCALES), 0, scales)
    if case == "down":
        _set(gq, gs, FEAT, COL, E2M1[4.0], E4M3[16.0])
        _set(uq, us, FEAT, COL, E2M1[0.5], E4M3[2.0 ** -5])
        for n in range(H):
            _set(dq, ds, n, FEAT, int(codes[n]), int(scales[n]))
    else:
        for i in range(I):
            if case == "up":
                _set(gq, gs, i, COL, E2M1[4.0], E4M3[16.0])
                _set(uq, us, i, COL, int(codes[i]), int(finite[i]))
            else:
                _set(gq, gs, i, COL, int(codes[i]), int(finite[i]))
                _set(uq, us, i, COL, E2M1[1.0], E4M3[1.0])
        for n in range(H):  # identity down matrix
            _set(dq, ds, n, n, E2M1[1.0], E4M3[1.0])
        if case == "up":
            ts[1] = 2.0 ** -6
    return {n: torch.from_numpy(v[None].copy()) for n, v in
            dict(gate_q=gq, up_q=uq, down_q=dq, gate_s=gs, up_s=us, down_s=ds).items()} | {
                "ts": torch.from_numpy(ts[None].copy())}


_ref = {}


def _reference(case):
    """(experts on the host, the oracle's expert output for the one-hot token, float64)."""
    if case not in _ref:
        ex = _experts(case)
        xb = np.zeros((1, H), np.uint16)
        xb[0, COL] = 0x3F80  # bf16 1.0
        exn = oracle.Experts(**{n: v.numpy() for n, v in ex.items()})
        y = oracle.expert_rows(xb, exn, 0, [0])[0]
        # the oracle against the decode tables directly
        rows = np.arange(4096)
        t2 = np.array([oracle.e2m1(c) for c in range(16)])
        t8 = np.array([oracle.e4m3(c) for c in range(256)])
        sc = np.where(np.isin(rows // 16, NAN_SCALES), 0, rows // 16)
        if case == "down":
            want = t2[rows % 16] * t8[rows // 16]
            assert np.array_equal(np.isnan(y), np.isnan(want))
            assert np.array_equal(y[~np.isnan(y)], want[~np.isnan(want)])
        elif case == "up":
            assert np.array_equal(y, t2[rows % 16] * t8[sc])
        else:
            g = t2[rows % 16] * t8[sc]
            with np.errstate(over="ignore"):  # exp(2688) = inf: silu(-2688) = -0
                assert np.allclose(y, g / (1 + np.exp(-g)), rtol=1e-15, atol=0)
        _ref[case] = (ex, y)
    return _ref[case]


def _compare(case, got, y):
    """got: [rows][H] float32 on the GPU; y: the oracle's row (float64)."""
    g = got.double().cpu().numpy()
    nan = np.isnan(y)
    assert np.all(np.isnan(g[:, nan])), "NaN scale codes must decode to NaN"
    g, r = g[:, ~nan], y[~nan]
    if case == "gate":
        # h = f16(silu(g)): within half an f16 step (relative 2^-11, absolute 2^-25 for f16
        # subnormals) plus the fp32 silu's few-ulp error
        bound = np.abs(r) * (2.0 ** -11 + 1e-6) + 2.0 ** -24
        bad = np.abs(g - r) > bound
        assert not bad.any(), "feature %d: %r vs %r" % (np.argmax(bad.any(0)), g[bad][:4], r[bad.any(0)][:4])
    else:
        bad = g != r
        assert not bad.any(), "%d of %d outputs differ, first at feature %d: %r vs %r" % (
            bad.sum(), bad.size, np.argmax(bad.any(0)), g[bad][:4], r[bad.any(0)][:4])


def _x(T):
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    x[:, COL] = 1.0
    return x


PATHS = {
    "single_launch_t1": 1, "single_launch_t2": 2, "few_rows_t1": 1, "few_rows_t4": 4,
    "gemm_rows32_t64": 64, "gemm_rows64_t512": 512, "gemm_rows128_t2048": 2048,
}


@pytest.mark.parametrize("case", ["down", "up", "gate"])
@pytest.mark.parametrize("path", list(PATHS))
def test_decode_every_code_exact(path, case):
    import bit_expert_ffn_amd as moe
    T = PATHS[path]
    print("case decode", case, path, "T=%d" % T, flush=True)
    ex_host, y_ref = _reference(case)
    ex = moe.pack_experts({n: v.cuda() for n, v in ex_host.items()})
    buf = moe.LayerBuffers(T, H, I, 1, 1, device="cuda", y_dtype=torch.float32)
    x = _x(T)
    if path.startswith("single_launch"):
        wr = torch.zeros((H, 1), dtype=torch.float32, device="cuda")
        moe.layer_nvfp4(x, wr, None, ex, 1, buf)
        torch.cuda.synchronize()
        assert torch.all(buf.topk_w == 1.0)
        got = buf.out
    else:
        ids = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
        buf.topk_w.fill_(1.0)
        moe.group(ids, 1, buf.count, buf.offset, buf.sorted_slot, buf.slot_row, buf.active,
                  buf.n_active, buf.ws)
        moe.expert_ffn_nvfp4(x, ex, buf.count, buf.offset, buf.sorted_slot, buf.active,
                             buf.n_active, 1, buf.y, buf.ws)
        moe.combine(buf.y, buf.slot_row, buf.topk_w, buf.out)
        torch.cuda.synchronize()
        _compare(case, buf.y, y_ref)
        got = buf.out  # weight 1.0: out = y exactly
    _compare(case, got, y_ref)
