"""Seeded synthetic inputs for the NVFP4 sparse-MoE FFN layer.

This module is the input recipe shared by the tests and the benchmark.  It holds none of the
layer's arithmetic: it draws activations and router weights, draws fp32 expert weights and
encodes them into the NVFP4 byte format the layer reads (the encoding happens before the layer
runs; decoding is done separately by the oracle and by the HIP kernels).

NVFP4 byte format (one expert matrix W of shape [N][K], quantised along K):
  q   [N][K/2]   two e2m1 codes per byte, low nibble = even k
  s   [N][K/16]  OCP E4M3FN scale code per 16 consecutive k of a row
  ts  float32    tensor scale of the whole matrix
Encoding (the reading taken where the pages only say "4-bit, one scale per 16 values"):
  ts = amax|W| / (6 * 448); block scale = e4m3_rne_sat((blockamax / 6) / ts);
  code = e2m1_rne_sat(w / (e4m3(s) * ts)), ties to the even code, sign kept (-0 allowed);
  a block whose scale rounds to 0 gets all-zero codes.
"""
import math

import torch

# Workload shapes.  Common to every large shape: 256 experts, 8 selected per token, NVFP4
# weights ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", Background / "The
# model" and "NVFP4 experts").  hidden 7168, expert intermediate 2048 (256 for a 1/8 tensor-
# parallel shard).  A verify step's rows are (request, draft position) pairs: 8 x 16 = 128
# (same page, section 1).  Prefill is 8 x 2048 tokens (page 1, "A 501B sparse model gets
# day-one serving support").
SPECS = {
    "tiny": dict(T=4, H=256, I=128, E=8, k=2, router="normal", zipf=None),
    "decode1": dict(T=1, H=7168, I=2048, E=256, k=8, router="normal", zipf=None),
    "decode64": dict(T=64, H=7168, I=2048, E=256, k=8, router="uniform", zipf=None),
    "verify128": dict(T=128, H=7168, I=256, E=256, k=8, router="normal", zipf=1.1),
    "prefill16k": dict(T=16384, H=7168, I=2048, E=256, k=8, router="normal", zipf=None),
}

W_STD = 0.02          # router and expert weights ~ N(0, 0.02)
E4M3_MAX = 448.0
E2M1_MAX = 6.0
# e2m1 magnitudes by code 0..7 and the rounding boundaries between neighbouring codes.
_E2M1_BOUNDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _gen(device, seed, role, sub=0):
    g = torch.Generator(device=device)
    # distinct, reproducible streams per (seed, role, sub-index)
    g.manual_seed((seed * 1000003 + role * 7919 + sub * 104729) & 0x7FFFFFFFFFFFFFFF)
    return g


def e2m1_encode(a):
    """fp32 tensor (already divided by its block scale) -> e2m1 codes (uint8, 0..15).
    Round to nearest, ties to the even code; saturate to +-6; keep the sign bit."""
    mag = a.abs()
    b = torch.tensor(_E2M1_BOUNDS, dtype=mag.dtype, device=mag.device)
    idx = torch.bucketize(mag, b, right=False)  # value on a boundary -> lower code
    # boundaries between an odd code and the next even code: ties go up to the even code
    for lo_code, bound in ((1, 0.75), (3, 1.75), (5, 3.5)):
        idx = torch.where(mag == bound, torch.full_like(idx, lo_code + 1), idx)
    idx = idx.clamp(max=7).to(torch.uint8)
    sign = torch.signbit(a).to(torch.uint8) << 3
    return idx | sign


def quantize_nvfp4(W):
    """W [N][K] float32 (K % 16 == 0) -> (q [N][K/2] u8, s [N][K/16] u8, ts float32 scalar)."""
    W = W.float()
    N, K = W.shape
    assert K % 16 == 0
    amax = W.abs().amax()
    ts = (amax / (E2M1_MAX * E4M3_MAX)).float()
    if float(ts) == 0.0:
        ts = torch.ones((), dtype=torch.float32, device=W.device)
    blocks = W.view(N, K // 16, 16)
    bscale = (blocks.abs().amax(-1) / E2M1_MAX) / ts
    s8 = bscale.clamp(max=E4M3_MAX).to(torch.float8_e4m3fn)
    sval = s8.float()
    denom = (sval * ts).unsqueeze(-1)
    safe = torch.where(denom > 0, denom, torch.ones_like(denom))
    scaled = torch.where(denom > 0, blocks / safe, torch.zeros_like(blocks))
    codes = e2m1_encode(scaled).view(N, K)
    q = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return q.contiguous(), s8.view(torch.uint8).contiguous(), ts.reshape(())


def make_experts(E, H, I, seed=0, device="cpu", experts=None):
    """NVFP4 weights for experts 0..E-1 (or only the listed ones; the others stay zero).
    Returns dict of gate_q, up_q, down_q [E][N][K/2], gate_s, up_s, down_s [E][N][K/16], ts [E][3]."""
    d = torch.device(device)
    out = dict(
        gate_q=torch.zeros((E, I, H // 2), dtype=torch.uint8, device=d),
        up_q=torch.zeros((E, I, H // 2), dtype=torch.uint8, device=d),
        down_q=torch.zeros((E, H, I // 2), dtype=torch.uint8, device=d),
        gate_s=torch.zeros((E, I, H // 16), dtype=torch.uint8, device=d),
        up_s=torch.zeros((E, I, H // 16), dtype=torch.uint8, device=d),
        down_s=torch.zeros((E, H, I // 16), dtype=torch.uint8, device=d),
        ts=torch.ones((E, 3), dtype=torch.float32, device=d),
    )
    for e in (range(E) if experts is None else experts):
        g = _gen(d, seed, 3, e)
        for m, (name, shape) in enumerate((("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))):
            W = torch.randn(shape, generator=g, device=d, dtype=torch.float32) * W_STD
            q, s, ts = quantize_nvfp4(W)
            out[name + "_q"][e].copy_(q)
            out[name + "_s"][e].copy_(s)
            out["ts"][e, m] = ts
            del W
    return out


def make_x(T, H, seed=0, device="cpu", role=0):
    """Activations: fp32 N(0,1) rounded to bf16."""
    g = _gen(torch.device(device), seed, role)
    return torch.randn((T, H), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_router(H, E, kind="normal", seed=0, device="cpu"):
    """Router weights [H][E] fp32: N(0, 0.02), or uniform with the same standard deviation."""
    g = _gen(torch.device(device), seed, 1)
    if kind == "normal":
        return torch.randn((H, E), generator=g, device=device, dtype=torch.float32) * W_STD
    if kind == "uniform":
        a = math.sqrt(3.0) * W_STD
        return (torch.rand((H, E), generator=g, device=device, dtype=torch.float32) * 2 - 1) * a
    raise ValueError(kind)


def make_zipf_bias(E, s=1.1, seed=0, device="cpu"):
    """Expert-popularity bias added to the router logits: a seeded permutation gives every
    expert a rank r in 1..E and bias = -s * ln r (the log of the unnormalised Zipf mass)."""
    g = _gen(torch.device("cpu"), seed, 2)
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-s * torch.log(rank)).to(torch.float32).to(device)


def make_combine_inputs(T, k, H, seed=0, device="cpu", y_dtype=torch.float16):
    """Inputs of the combine variants.  y [T*k][H]: N(0,1) rows, each scaled by exp(N(0,1)) so
    the expert rows differ in magnitude (as expert outputs do); slot_row: a seeded permutation
    of the T*k rows (any grouping is a permutation); topk_w [T][k]: positive, each row summing to
    one; resid [T][H]: N(0, 9); gain [H]: uniform in [0.5, 1.5]."""
    d = torch.device(device)
    g = _gen(d, seed, 20)
    y = torch.randn((T * k, H), generator=g, device=d, dtype=torch.float32)
    y *= torch.exp(torch.randn((T * k, 1), generator=g, device=d, dtype=torch.float32))
    slot_row = torch.randperm(T * k, generator=g, device=d).to(torch.int32)
    w = torch.rand((T, k), generator=g, device=d, dtype=torch.float32) + 0.05
    w /= w.sum(dim=1, keepdim=True)
    resid = torch.randn((T, H), generator=g, device=d, dtype=torch.float32) * 3.0
    gain = torch.rand((H,), generator=g, device=d, dtype=torch.float32) + 0.5
    return dict(y=y.to(y_dtype), slot_row=slot_row, topk_w=w, resid=resid, gain=gain)


def make_layer(spec, seed=0, device="cpu", T=None, experts=None):
    """All inputs of one layer call for a spec (a SPECS key or a dict with the same fields)."""
    sp = dict(SPECS[spec]) if isinstance(spec, str) else dict(spec)
    if T is not None:
        sp["T"] = T
    x = make_x(sp["T"], sp["H"], seed, device)
    wr = make_router(sp["H"], sp["E"], sp.get("router", "normal"), seed, device)
    bias = make_zipf_bias(sp["E"], sp["zipf"], seed, device) if sp.get("zipf") else None
    w = make_experts(sp["E"], sp["H"], sp["I"], seed, device, experts)
    return dict(spec=sp, x=x, w_router=wr, bias=bias, experts=w)


def to_numpy(layer):
    """Host copies in the byte formats the oracle reads (x as bf16 bit patterns)."""
    ex = {k: v.cpu().numpy() for k, v in layer["experts"].items()}
    return dict(
        x=layer["x"].cpu().view(torch.int16).numpy().view("uint16"),
        w_router=layer["w_router"].cpu().numpy(),
        bias=None if layer["bias"] is None else layer["bias"].cpu().numpy(),
        experts=ex,
    )
