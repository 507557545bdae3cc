"""GPU parity of the fp8-compute variant (MXFP8 weights, x and h on gfx950's scaled matrix cores)
against the oracle's fp8 variant, and its accuracy against the exact NVFP4 layer.

Bars (the arithmetic is stated in the header of the fp8 entry points):
  - load-time requantisation NVFP4 -> MXFP8: bit-exact (both sides decode every weight exactly
    in double and apply the same quantiser);
  - x -> MXFP8: bit-exact (x is bf16, each block's scale is a power of two, the hardware
    conversion rounds to nearest even like the oracle);
  - h -> MXFP8: h comes from fp32 sums on the GPU and fp64 sums in the oracle.  With the
    products exact (x8 and the weights are checked bit-exact), an fp32 sum of H terms in any
    order is within 2 H 2^-24 sum|terms| of the exact one; propagated through silu(g) * u this
    bounds |h_gpu - h| per element.  A code may differ from the oracle's only if it lies between
    the codes of h - bound and h + bound, and a block scale only if the block's largest |h| is
    within its bound of a power of two; as a guard against systematic error, at most 1 % of the
    codes may differ at all;
  - y (f16) against the oracle's fp64 y: normwise max relative error <= 2e-2 (a moved h code
    changes one term of a row's sum by one e4m3 step) and mean error <= 2e-3 of the mean |y|
    (f16 output rounding is 2^-11 relative, fp32 accumulation ~1e-5);
  - accuracy bar of the variant itself against the exact NVFP4 layer: relative L2 error <= 0.1
    (the oracle's fp8 variant measures ~0.074 on these shapes).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import experts_np, out_errors

pytestmark = pytest.mark.gpu

# internal workspace layout of the fp8 FFN call (x8, xs, h8, hs after the 64 KiB of counters);
# used only to inspect the intermediate quantisations
SYNC = 65536


def _a256(n):
    return (n + 255) // 256 * 256


def _dev_i32(a):
    return torch.tensor(np.asarray(a, np.int32), dtype=torch.int32, device="cuda")


def mx_tiled_to_rowmajor(q8, s8, E, N, K):
    """Row-major codes [E][N][K] and scales [E][N][K/32] from the MX tile layout, by the offset
    formulas of the ABI header (numpy); also checks that the formulas cover every byte once."""
    q8 = np.asarray(q8).reshape(-1)
    s8 = np.asarray(s8).reshape(-1)
    n = np.arange(N)[:, None]
    kk = np.arange(K)[None, :]
    i, b, st, r = kk % 32, kk // 32, kk // 64, n // 32
    off = ((r * (K // 64) + st) * 64 + n % 32 + 32 * (i // 16)) * 32 + 16 * (b % 2) + i % 16
    bb = np.arange(K // 32)[None, :]
    s2 = bb // 2
    soff = ((r * (K // 256) + s2 // 4) * 64 + n % 32 + 32 * (bb % 2)) * 4 + s2 % 4
    assert np.array_equal(np.sort(off.ravel()), np.arange(N * K))
    assert np.array_equal(np.sort(soff.ravel()), np.arange(N * K // 32))
    q = np.stack([q8[e * N * K + off] for e in range(E)])
    s = np.stack([s8[e * N * K // 32 + soff] for e in range(E)])
    return q, s


def _gpu_mx8(experts_dev):
    import bit_expert_ffn_amd as moe
    mx = moe.mx8_experts(experts_dev)
    torch.cuda.synchronize()
    return mx


@pytest.mark.parametrize("E,H,I", [(2, 256, 256), (3, 512, 768), (1, 1024, 256)])
def test_nvfp4_to_mxfp8_bit_exact(E, H, I):
    print("convert", E, H, I, flush=True)
    W = synth.make_experts(E, H, I, seed=E + H)
    # extreme tensor scales: tiny (an fp32 subnormal: the shared exponent clamps at -127 and
    # codes go subnormal) and huge; one all-zero block row
    W["ts"][0, 0] = 2.0 ** -140
    W["ts"][-1, 2] = 2.0 ** 100
    W["gate_q"][0, 3, :16] = 0
    ex = experts_np(W)
    ref = oracle.nvfp4_to_mxfp8(ex)
    mx = _gpu_mx8({n: v.cuda() for n, v in W.items()})
    for m, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        q, s = mx_tiled_to_rowmajor(mx[m + "_q"].cpu().numpy(), mx[m + "_s"].cpu().numpy(),
                                    E, N, K)
        assert np.array_equal(q, getattr(ref, m + "_q")), m
        assert np.array_equal(s, getattr(ref, m + "_s")), m
    # the planted cases took their special paths
    assert ref.gate_s[0].max() == 0  # clamped exponent -127
    assert (ref.gate_q[0, 3, :32] == 0).all() and ref.gate_s[0, 3, 0] == 0


SHAPES = {
    "ragged": dict(T=37, H=512, I=256, E=16, k=4, router="normal", zipf=None),
    "multi_tile": dict(T=200, H=256, I=512, E=32, k=6, router="normal", zipf=None),
    "zipf_skew": dict(T=96, H=256, I=256, E=64, k=8, router="normal", zipf=1.1),
    "one_token": dict(T=1, H=1024, I=256, E=32, k=8, router="normal", zipf=None),
    "single_expert": dict(T=300, H=256, I=256, E=1, k=1, router="normal", zipf=None),
    "max_e": dict(T=64, H=256, I=256, E=256, k=8, router="uniform", zipf=None),
    "tall_128_row_tiles": dict(T=2100, H=256, I=256, E=8, k=2, router="normal", zipf=None),
}


def _run(sp, seed, x_override=None):
    import bit_expert_ffn_amd as moe
    L = synth.make_layer(sp, seed=seed)
    if x_override is not None:
        L["x"] = x_override
    N = synth.to_numpy(L)
    ex = experts_np(L["experts"])
    k = sp["k"]
    ids, _ = oracle.topk(oracle.router(N["x"], N["w_router"], N["bias"]), k)
    grp = oracle.group(ids, sp["E"])
    x = L["x"].cuda()
    mx = _gpu_mx8({n: v.cuda() for n, v in L["experts"].items()})
    T, H = x.shape
    ws = torch.zeros(moe.workspace_size(T, H, sp["I"], sp["E"], k), dtype=torch.uint8,
                     device="cuda")
    y = torch.full((T * k, H), float("nan"), dtype=torch.float16, device="cuda")
    moe.expert_ffn_mx8(x, mx, _dev_i32(grp["count"]), _dev_i32(grp["offset"]),
                       _dev_i32(grp["sorted_slot"]), _dev_i32(grp["active"]),
                       _dev_i32([grp["n_active"]]), k, y, ws)
    torch.cuda.synchronize()
    return dict(N=N, ex=ex, grp=grp, k=k, y=y.float().cpu().numpy(), ws=ws.cpu().numpy(), T=T,
                H=H, I=sp["I"], mx_dev=mx)


@pytest.mark.parametrize("name", list(SHAPES))
def test_ffn_mx8_parity(name):
    sp = SHAPES[name]
    print("ffn_mx8", name, sp, flush=True)
    r = _run(sp, seed=11)
    mx_ref = oracle.nvfp4_to_mxfp8(r["ex"])
    y_ref = oracle.ffn_mx(r["N"]["x"], mx_ref, r["grp"], r["k"])
    assert np.isfinite(r["y"]).all()
    mr, _ = out_errors(r["y"], y_ref)
    rel_mean = np.abs(r["y"] - y_ref).mean() / np.abs(y_ref).mean()
    assert mr <= 2e-2 and rel_mean <= 2e-3, (mr, rel_mean)

    # intermediate quantisations, read from the workspace
    T, H, I, k = r["T"], r["H"], r["I"], r["k"]
    n = T * k
    ws = r["ws"]
    o_xs = SYNC + _a256(T * H)
    o_h8 = o_xs + _a256(T * H // 32)
    o_hs = o_h8 + _a256(n * I)
    x8, xs = ws[SYNC:SYNC + T * H].reshape(T, H), ws[o_xs:o_xs + T * H // 32].reshape(T, -1)
    xf = (r["N"]["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # bf16 bits
    xq, xsc = oracle.mx8_quant(xf)
    assert np.array_equal(x8, xq) and np.array_equal(xs, xsc)

    h8 = ws[o_h8:o_h8 + n * I].reshape(n, I)
    hs = ws[o_hs:o_hs + n * I // 32].reshape(n, I // 32)
    xd = oracle.mx8_dequant(xq, xsc)
    off, ss = r["grp"]["offset"], r["grp"]["sorted_slot"]
    href = np.empty((n, I))
    dh = np.empty((n, I))  # bound on |h_gpu - h|
    gam = 2.0 * H * 2.0 ** -24  # fp32 sum of H exact products, any order: <= gam * sum |terms|
    for e in range(mx_ref.E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            xe = xd[ss[a:b] // k]
            wg, wu = oracle.mx8_weights(mx_ref, e, 0), oracle.mx8_weights(mx_ref, e, 1)
            g, u = xe @ wg.T, xe @ wu.T
            eg, eu = gam * (np.abs(xe) @ np.abs(wg).T), gam * (np.abs(xe) @ np.abs(wu).T)
            sg = g / (1.0 + np.exp(-g))
            href[a:b] = sg * u
            # |d silu / dg| <= 1.1; fp32 silu and product: a few ulp of |h|
            dh[a:b] = 1.1 * eg * (np.abs(u) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(sg * u)
    hq, hsc = oracle.mx8_quant(href)
    # a block's scale may differ only where its largest |h| is within the bound of a power of 2
    amax = np.abs(href).reshape(n, I // 32, 32).max(axis=2)
    dmax = dh.reshape(n, I // 32, 32).max(axis=2)
    p2 = 2.0 ** np.round(np.log2(np.maximum(amax, 1e-300)))
    bad_scale = (hs != hsc) & ~(np.abs(amax - p2) <= dmax)
    assert not bad_scale.any(), np.argwhere(bad_scale)[:5]
    # a code may differ only where the oracle's h is within the bound of a rounding boundary:
    # the GPU code must lie between the codes of h - dh and h + dh (under the common scale)
    same = np.repeat(hs == hsc, 32, axis=1)
    diff = (h8 != hq) & same
    assert diff.mean() <= 1e-2, diff.mean()

    def val(c):
        return np.array([oracle.e4m3(int(v)) for v in c])

    rows, cols = np.nonzero(diff)
    sc = 2.0 ** (hsc[rows, cols // 32].astype(np.float64) - 127)
    lo = np.array([oracle.e4m3_code(v) for v in (href[rows, cols] - dh[rows, cols]) / sc])
    hi = np.array([oracle.e4m3_code(v) for v in (href[rows, cols] + dh[rows, cols]) / sc])
    gv = val(h8[rows, cols])
    assert ((val(lo) <= gv) & (gv <= val(hi))).all()
    print("h codes moved by the fp32 sums: %d of %d" % (len(rows), diff.size), flush=True)


def test_ffn_mx8_zero_input_gives_zero():
    sp = SHAPES["ragged"]
    x = torch.zeros((sp["T"], sp["H"]), dtype=torch.bfloat16)
    x[3] = synth.make_x(1, sp["H"], seed=4)[0]  # one live row among zero rows
    r = _run(sp, seed=3, x_override=x)
    ss = r["grp"]["sorted_slot"]
    rows = ss // r["k"] != 3
    assert (r["y"][rows] == 0).all()
    assert np.abs(r["y"][~rows]).max() > 0


def test_ffn_mx8_deterministic():
    sp = SHAPES["multi_tile"]
    a = _run(sp, seed=8)["y"]
    b = _run(sp, seed=8)["y"]
    assert np.array_equal(a, b)


def test_ffn_mx8_accuracy_against_exact_layer():
    sp = dict(T=48, H=2048, I=512, E=16, k=4, router="normal", zipf=None)
    print("accuracy", sp, flush=True)
    r = _run(sp, seed=21)
    y_exact = oracle.ffn(r["N"]["x"], r["ex"], r["grp"], r["k"])
    rel = np.linalg.norm(r["y"] - y_exact) / np.linalg.norm(y_exact)
    print("fp8 variant rel-L2 vs exact layer %.4f" % rel, flush=True)
    assert rel <= 0.1
