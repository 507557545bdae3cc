"""GPU parity of moe_combine_norm, the combine variants: per-expert RMS norm of each expert row
before the weighted sum, and the epilogue (the MoE output's RMS factor, scaled residual, RMS
norm with a gain for the next layer's input).  Both sides read the same seeded y, so the only
differences are fp32 against fp64 arithmetic and the final bf16 rounding of x_next.

Bars, element by element: out within 2e-5 of the magnitude its terms add up to (fp32 sums of
at most 64 terms and norm factors from fp32 sums of squares: a few 1e-6 relative); x_next within
half a bf16 ulp of the oracle's value (2^-8 relative) plus that same fp32 error carried through
the last norm."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

RTOL_F32 = 2e-5
BF16_HALF_ULP = 2.0 ** -8

CASES = {
    # name: T, k, H, y dtype, alpha, beta
    "tiny_f32": (3, 2, 128, torch.float32, 1.0, 1.0),
    "ragged_k_f16": (5, 11, 384, torch.float16, 0.5, 2.0),      # two row chunks, short tail
    "hidden7168_f16": (6, 8, 7168, torch.float16, 1.0, 0.8),    # last group half past the row
    "hidden4096_f32": (4, 8, 4096, torch.float32, 1.0, -1.5),   # exactly one group per thread
    "hidden16512_f16": (2, 3, 16512, torch.float16, 0.9, 1.1),  # 8 groups, ragged
    "hidden16512_f32": (2, 5, 16512, torch.float32, 1.0, 1.0),
    "hidden65536_f16": (1, 2, 65536, torch.float16, 1.0, 1.0),  # largest hidden size
    "k1_f16": (7, 1, 256, torch.float16, 1.0, 1.0),
    "k64_f32": (2, 64, 256, torch.float32, 0.25, 3.0),
}
FLAGS = [(False, False), (True, False), (False, True), (True, True)]


def _oracle(inp, k, H, expert_norm, epilogue, alpha, beta, eps, tokens=None):
    """Oracle on all tokens, or on the listed tokens only (their rows of y, gathered on the
    device before the copy to the host)."""
    y, sr, w, resid = inp["y"], inp["slot_row"], inp["topk_w"], inp["resid"]
    if tokens is not None:
        idx = torch.as_tensor(tokens, device=y.device)
        rows = sr.view(-1, k)[idx].reshape(-1).long()
        y, w, resid = y[rows], w[idx], resid[idx]
        sr = torch.arange(rows.numel(), dtype=torch.int32)
    y = y.float().cpu().numpy()
    sr, w, resid = sr.cpu().numpy(), w.cpu().numpy(), resid.cpu().numpy()
    kw = dict(expert_norm=expert_norm, eps=eps)
    if epilogue:
        kw.update(resid=resid, alpha=alpha, beta=beta, gain=inp["gain"].cpu().numpy())
    ref = oracle.combine_norm(y, sr, w, k, H, **kw)
    # magnitude scale of every output element (for the fp32 error bars)
    yk = np.abs(y[sr].reshape(w.shape[0], k, H))
    c = np.abs(w)
    if expert_norm:
        c = c / np.sqrt(np.mean(y[sr].reshape(w.shape[0], k, H) ** 2, axis=2) + eps)
    mag_f = np.einsum("tj,tjh->th", c, yk)
    if epilogue:
        mag_o = np.abs(alpha * resid) + np.abs(beta * ref["s"])[:, None] * mag_f
        mag_x = np.abs(inp["gain"].cpu().numpy())[None, :] * ref["r"][:, None] * mag_o
        return ref, mag_o, mag_x
    return ref, mag_f, None


def _check(out, xn, ref, mag_o, mag_x, epilogue):
    out = out.cpu().numpy().astype(np.float64)
    err = np.abs(out - ref["out"])
    assert np.all(err <= RTOL_F32 * mag_o + 1e-30), "out: max err %.3e at %s" % (
        err.max(), np.unravel_index(np.argmax(err - RTOL_F32 * mag_o), err.shape))
    if epilogue:
        x = xn.float().cpu().numpy().astype(np.float64)
        e = np.abs(x - ref["xn"])
        bar = BF16_HALF_ULP * np.abs(ref["xn"]) + RTOL_F32 * mag_x + 1e-30
        assert np.all(e <= bar), "x_next: worst excess %.3e" % (e - bar).max()


def _run(inp, k, out, expert_norm, epilogue, alpha, beta, eps, xn=None, resid=None):
    import bit_expert_ffn_amd as moe
    kw = dict(expert_norm=expert_norm, eps=eps)
    if epilogue:
        kw.update(resid=inp["resid"] if resid is None else resid, alpha=alpha, beta=beta,
                  gain=inp["gain"], x_next=xn)
    moe.combine_norm(inp["y"], inp["slot_row"], inp["topk_w"], out, **kw)
    torch.cuda.synchronize()


@pytest.mark.parametrize("flags", FLAGS, ids=["plain", "expert_norm", "epilogue", "both"])
@pytest.mark.parametrize("name", list(CASES))
def test_combine_norm_parity(name, flags):
    T, k, H, ydt, alpha, beta = CASES[name]
    expert_norm, epilogue = flags
    print("case combine_norm", name, flags, flush=True)
    inp = {n: v.cuda() for n, v in synth.make_combine_inputs(T, k, H, seed=4, y_dtype=ydt).items()}
    out = torch.full((T, H), float("nan"), device="cuda")
    xn = torch.full((T, H), float("nan"), device="cuda", dtype=torch.bfloat16)
    eps = 1e-6
    _run(inp, k, out, expert_norm, epilogue, alpha, beta, eps, xn)
    ref, mag_o, mag_x = _oracle(inp, k, H, expert_norm, epilogue, alpha, beta, eps)
    _check(out, xn, ref, mag_o, mag_x, epilogue)


def test_combine_norm_flags_off_bit_identical_to_combine():
    import bit_expert_ffn_amd as moe
    T, k, H = 9, 8, 7168
    print("case combine_norm flags off vs combine", flush=True)
    for ydt in (torch.float16, torch.float32):
        inp = {n: v.cuda() for n, v in synth.make_combine_inputs(T, k, H, seed=5, y_dtype=ydt).items()}
        a = torch.empty((T, H), device="cuda")
        b = torch.empty((T, H), device="cuda")
        moe.combine(inp["y"], inp["slot_row"], inp["topk_w"], a)
        moe.combine_norm(inp["y"], inp["slot_row"], inp["topk_w"], b)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_combine_norm_in_place_residual():
    """resid and out the same tensor: same bits as writing to a separate output."""
    T, k, H = 4, 8, 7168
    print("case combine_norm in place", flush=True)
    inp = {n: v.cuda() for n, v in synth.make_combine_inputs(T, k, H, seed=6).items()}
    sep = torch.empty((T, H), device="cuda")
    xa = torch.empty((T, H), device="cuda", dtype=torch.bfloat16)
    _run(inp, k, sep, True, True, 1.0, 0.7, 1e-6, xa)
    stream = inp["resid"].clone()
    xb = torch.empty_like(xa)
    _run(inp, k, stream, True, True, 1.0, 0.7, 1e-6, xb, resid=stream)
    assert torch.equal(stream, sep) and torch.equal(xa, xb)


def test_combine_norm_zero_rows_with_eps():
    """All-zero expert rows with eps > 0: factor 1/sqrt(eps) times zero, so f = 0, the new
    residual is alpha * resid exactly (fp32 multiply) and x_next the RMS norm of it."""
    T, k, H = 3, 4, 256
    print("case combine_norm zero rows", flush=True)
    inp = {n: v.cuda() for n, v in synth.make_combine_inputs(T, k, H, seed=7).items()}
    inp["y"].zero_()
    out = torch.empty((T, H), device="cuda")
    xn = torch.empty((T, H), device="cuda", dtype=torch.bfloat16)
    _run(inp, k, out, True, True, 0.5, 2.0, 1e-6, xn)
    assert torch.equal(out, inp["resid"] * 0.5)
    ref, mag_o, mag_x = _oracle(inp, k, H, True, True, 0.5, 2.0, 1e-6)
    _check(out, xn, ref, mag_o, mag_x, True)


def test_combine_norm_prefill_size_sampled():
    """8 x 2048 tokens, hidden 7168, top-8, f16 y, both variants, in the launch configuration
    the benchmark times: sampled tokens (first, last, a spread between) against the oracle."""
    T, k, H = 16384, 8, 7168
    print("case combine_norm prefill size", flush=True)
    inp = synth.make_combine_inputs(T, k, H, seed=9, device="cuda")
    out = torch.empty((T, H), device="cuda")
    xn = torch.empty((T, H), device="cuda", dtype=torch.bfloat16)
    _run(inp, k, out, True, True, 1.0, 1.0, 1e-6, xn)
    toks = np.unique(np.concatenate([[0, 1, T - 1], np.linspace(0, T - 1, 29).astype(int)]))
    ref, mag_o, mag_x = _oracle(inp, k, H, True, True, 1.0, 1.0, 1e-6, tokens=toks)
    idx = torch.from_numpy(toks).cuda()
    _check(out[idx], xn[idx], ref, mag_o, mag_x, True)
    del inp
