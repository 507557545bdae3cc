"""Pins for the CPU oracle: each check compares it with something other than itself
(hand-worked tables, torch's own fp8/bf16 decoders, brute force, closed forms, invariants,
numpy matmul/einsum on tiny dense cases)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _bits(x_bf16):
    return x_bf16.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- decode tables
def test_e2m1_hand_table():
    rows = _read_table("e2m1_table.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got)


def test_e4m3_hand_values():
    for code, val in _read_table("e4m3_values.txt"):
        got = oracle.e4m3(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            want = float(val)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got)


def test_e4m3_all_codes_match_torch_decoder():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c


def test_bf16_decode_matches_torch():
    bits = torch.arange(0, 65536, 97, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits.numpy().view(np.uint16), ref):
        got = oracle.bf16(int(b))
        assert (math.isnan(got) and math.isnan(r)) or got == r


# ---------------------------------------------------------------- quantiser (input recipe)
def _experts_np(ex):
    return oracle.Experts(**{k: v.cpu().numpy() for k, v in ex.items()})


def _dequant_matrix(q, s, ts):
    """dequantise a single [N][K] matrix through the oracle's decoders"""
    ex = oracle.Experts(gate_q=q[None], up_q=q[None], down_q=np.zeros((1, q.shape[1] * 2, q.shape[0] // 2), np.uint8),
                        gate_s=s[None], up_s=s[None],
                        down_s=np.zeros((1, q.shape[1] * 2, q.shape[0] // 16), np.uint8),
                        ts=np.array([[ts, ts, 1.0]], np.float32))
    return oracle.dequant(ex, 0, 0)


def test_quantizer_on_grid_round_trip_exact():
    g = torch.Generator().manual_seed(5)
    N, K = 8, 64
    grid = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float32)
    codes = torch.randint(0, 8, (N, K), generator=g)
    sign = torch.randint(0, 2, (N, K), generator=g) * 2 - 1
    W = grid[codes] * sign
    W.view(N, K // 16, 16)[:, :, 0] = 6.0  # every block reaches the top code
    # per-block scales drawn from exact e4m3 values; one block at 448 so ts = 2^-10 exactly
    cb = torch.tensor([448.0, 56.0, 1.5, 0.013671875, 240.0, 3.25, 0.5, 96.0])
    c = cb[torch.randint(0, 8, (N, K // 16), generator=g)]
    c[0, 0] = 448.0
    W = (W.view(N, K // 16, 16) * c[..., None] * 2.0 ** -10).view(N, K)
    q, s, ts = synth.quantize_nvfp4(W)
    assert float(ts) == 2.0 ** -10
    D = _dequant_matrix(q.numpy(), s.numpy(), float(ts))
    assert np.array_equal(D, W.double().numpy())


def test_quantizer_idempotent():
    g = torch.Generator().manual_seed(6)
    W = torch.randn(16, 256, generator=g) * 0.02
    q, s, ts = synth.quantize_nvfp4(W)
    D = torch.from_numpy(_dequant_matrix(q.numpy(), s.numpy(), float(ts))).float()
    q2, s2, ts2 = synth.quantize_nvfp4(D)
    # same codes and block scales; the fp32 tensor scale may move by one ulp
    assert torch.equal(q2, q) and torch.equal(s2, s)
    assert abs(float(ts2) - float(ts)) <= 1.2e-7 * float(ts)


def test_quantizer_error_bound_and_saturation():
    g = torch.Generator().manual_seed(7)
    W = torch.randn(32, 512, generator=g) * 0.02
    q, s, ts = synth.quantize_nvfp4(W)
    D = _dequant_matrix(q.numpy(), s.numpy(), float(ts))
    Wd = W.double().numpy()
    sval = np.array([oracle.e4m3(int(c)) for c in range(256)])[s.numpy().astype(np.int64)]
    S = np.repeat(sval, 16, axis=1) * float(ts)
    # half the e2m1 gap at |w|/S (gap 0.5 below 2, 1 in [2,4), 2 above), plus saturation from
    # the RNE-rounded block scale (at most 6 * S * 2^-4 past the largest code)
    a = np.abs(Wd) / S
    gap = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = 0.5 * gap * S + np.maximum(a - 6.0, 0) * S + 1e-12
    assert np.all(np.abs(Wd - D) <= bound)
    assert np.all(np.abs(D) <= 6.0 * S + 1e-12)


def test_quantizer_ties_to_even_and_sign():
    a = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.1, -0.0, 0.3])
    codes = synth.e2m1_encode(a).tolist()
    vals = [oracle.e2m1(c) for c in codes]
    assert vals[:8] == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    assert codes[8] == 8 and codes[9] == 8  # negative values that round to zero keep the sign
    assert vals[10] == 0.5


def test_quantizer_zero_block():
    W = torch.zeros(2, 32)
    W[1, 16:] = 0.01
    q, s, ts = synth.quantize_nvfp4(W)
    assert int(s[0, 0]) == 0 and int(s[0, 1]) == 0 and int(s[1, 0]) == 0
    assert q[0].sum() == 0


# ---------------------------------------------------------------- router, top-k, softmax
def _tiny(seed=0, **over):
    sp = dict(synth.SPECS["tiny"])
    sp.update(over)
    L = synth.make_layer(sp, seed=seed)
    return sp, L, synth.to_numpy(L)


def test_router_matches_numpy_fp64():
    sp, L, N = _tiny()
    got = oracle.router(N["x"], N["w_router"])
    x = L["x"].double().numpy()
    ref = x @ N["w_router"].astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-7)


def test_router_one_hot_row_exact():
    H, E = 64, 8
    wr = (np.random.default_rng(3).standard_normal((H, E)) * 0.02).astype(np.float32)
    for h in (0, 17, 63):
        x = torch.zeros(1, H, dtype=torch.bfloat16)
        x[0, h] = 1.0
        got = oracle.router(_bits(x), wr)
        assert np.array_equal(got[0], wr[h])


def test_router_bias_added():
    sp, L, N = _tiny()
    b = (np.arange(sp["E"]) * 0.25).astype(np.float32)
    a = oracle.router(N["x"], N["w_router"])
    c = oracle.router(N["x"], N["w_router"], b)
    ref = (L["x"].double().numpy() @ N["w_router"].astype(np.float64)) + b
    assert np.allclose(c, ref, rtol=1e-6, atol=1e-6)
    assert not np.array_equal(a, c)


def test_topk_brute_force_sort():
    rng = np.random.default_rng(11)
    for E, k in ((8, 2), (16, 5), (256, 8)):
        logits = rng.standard_normal((20, E)).astype(np.float32)
        logits[3, :4] = logits[3, 5]  # exact ties: lower id first
        ids, w = oracle.topk(logits, k)
        for t in range(20):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == order
            l = logits[t, order].astype(np.float64)
            p = np.exp(l - l.max())
            assert np.allclose(w[t], p / p.sum(), rtol=0, atol=1e-15)
            assert abs(w[t].sum() - 1.0) < 1e-12


def test_topk_zero_logits_and_special_weights():
    for E, k in ((8, 2), (256, 8)):
        ids, w = oracle.topk(np.zeros((1, E), np.float32), k)
        assert list(ids[0]) == list(range(k))
        assert np.all(w[0] == 1.0 / k)
    ids, w = oracle.topk(np.array([[0.1, 3.0, -2.0]], np.float32), 1)
    assert ids[0, 0] == 1 and w[0, 0] == 1.0
    l = np.array([[math.log(3.0), 0.0, -5.0]], np.float32)
    ids, w = oracle.topk(l, 2)
    assert abs(w[0, 0] - 0.75) < 1e-7 and abs(w[0, 1] - 0.25) < 1e-7


def test_softmax_renormalised_equals_full_softmax_restricted():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((5, 32)).astype(np.float32)
    ids, w = oracle.topk(l, 6)
    full = np.exp(l.astype(np.float64))
    full /= full.sum(1, keepdims=True)
    for t in range(5):
        sel = full[t, ids[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-12)


# ---------------------------------------------------------------- grouping
def _brute_group(ids, E):
    T, k = ids.shape
    slots = sorted(range(T * k), key=lambda s: (int(ids.flat[s]), s))
    count = np.bincount(ids.ravel(), minlength=E)
    active = sorted([e for e in range(E) if count[e] > 0], key=lambda e: (-count[e], e))
    return slots, count, active


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (4, 2, 8), (64, 8, 256), (37, 3, 16), (5, 16, 16)])
def test_group_brute_force_and_invariants(T, k, E):
    rng = np.random.default_rng(T * 31 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    g = oracle.group(ids, E)
    slots, count, active = _brute_group(ids, E)
    assert list(g["sorted_slot"]) == slots
    assert np.array_equal(g["count"], count)
    assert g["offset"][0] == 0 and np.array_equal(np.diff(g["offset"]), count)
    assert g["offset"][-1] == T * k
    assert g["n_active"] == len(active) and list(g["active"][: len(active)]) == active
    assert np.all(g["active"][len(active):] == -1)
    assert np.array_equal(g["slot_row"][g["sorted_slot"]], np.arange(T * k))
    for e in range(E):
        seg = g["sorted_slot"][g["offset"][e]:g["offset"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids.ravel()[seg] == e)


# ---------------------------------------------------------------- expert FFN
def _silu(g):
    return g / (1.0 + np.exp(-g))


def test_ffn_single_expert_is_textbook_swiglu_mlp():
    sp, L, N = _tiny(E=1, k=1)
    ex = _experts_np(L["experts"])
    Wg, Wu, Wd = (oracle.dequant(ex, 0, m) for m in range(3))
    x = L["x"].double().numpy()
    ref = (_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    got = oracle.expert_rows(N["x"], ex, 0, np.arange(sp["T"]))
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)
    # whole layer with E = k = 1: weight 1, out = that MLP
    res = oracle.layer(N["x"], N["w_router"], None, ex, 1)
    assert np.all(res["topk_w"] == 1.0)
    assert np.allclose(res["out"], ref, rtol=1e-10, atol=1e-12)


def test_dequant_weight_matches_per_element_definition():
    sp, L, N = _tiny()
    ex = _experts_np(L["experts"])
    rng = np.random.default_rng(1)
    for _ in range(50):
        e, m = int(rng.integers(sp["E"])), int(rng.integers(3))
        Nn = sp["H"] if m == 2 else sp["I"]
        K = sp["I"] if m == 2 else sp["H"]
        n, kk = int(rng.integers(Nn)), int(rng.integers(K))
        q = (ex.gate_q, ex.up_q, ex.down_q)[m][e, n, kk // 2]
        code = (q >> 4) if kk % 2 else (q & 15)
        s = (ex.gate_s, ex.up_s, ex.down_s)[m][e, n, kk // 16]
        want = oracle.e2m1(code) * oracle.e4m3(s) * float(ex.ts[e, m])
        assert oracle.weight(ex, e, m, n, kk) == want
        assert oracle.dequant(ex, e, m)[n, kk] == want


def test_zero_input_gives_zero_output():
    sp, L, N = _tiny()
    ex = _experts_np(L["experts"])
    x0 = np.zeros_like(N["x"])
    res = oracle.layer(x0, N["w_router"], None, ex, sp["k"])
    assert np.all(res["out"] == 0.0)
    assert list(res["topk_id"][0]) == list(range(sp["k"]))


def test_doubling_down_scale_doubles_output_exactly():
    sp, L, N = _tiny()
    ex = _experts_np(L["experts"])
    res = oracle.layer(N["x"], N["w_router"], None, ex, sp["k"])
    ts2 = ex.ts.copy()
    ts2[:, 2] *= 2
    ex2 = oracle.Experts(ex.gate_q, ex.up_q, ex.down_q, ex.gate_s, ex.up_s, ex.down_s, ts2)
    res2 = oracle.layer(N["x"], N["w_router"], None, ex2, sp["k"])
    assert np.array_equal(res2["out"], 2 * res["out"])


# ---------------------------------------------------------------- whole layer
def test_dense_equivalent_all_experts_selected():
    sp, L, N = _tiny(E=8, k=8)
    ex = _experts_np(L["experts"])
    res = oracle.layer(N["x"], N["w_router"], None, ex, 8)
    x = L["x"].double().numpy()
    W = [[oracle.dequant(ex, e, m) for m in range(3)] for e in range(8)]
    Wg = np.stack([w[0] for w in W])
    Wu = np.stack([w[1] for w in W])
    Wd = np.stack([w[2] for w in W])
    g = np.einsum("th,eih->tei", x, Wg)
    u = np.einsum("th,eih->tei", x, Wu)
    y = np.einsum("tei,ehi->teh", _silu(g) * u, Wd)
    logits = (x @ N["w_router"].astype(np.float64)).astype(np.float32).astype(np.float64)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.einsum("te,teh->th", p, y)
    assert np.allclose(res["out"], ref, rtol=1e-9, atol=1e-11)


def test_permuting_expert_labels_relabels_ids_only():
    sp, L, N = _tiny()
    ex = _experts_np(L["experts"])
    res = oracle.layer(N["x"], N["w_router"], None, ex, sp["k"])
    perm = np.random.default_rng(4).permutation(sp["E"])  # new label p[e] for old e
    inv = np.argsort(perm)
    ex2 = oracle.Experts(*(a[inv] for a in (ex.gate_q, ex.up_q, ex.down_q, ex.gate_s, ex.up_s, ex.down_s, ex.ts)))
    wr2 = N["w_router"][:, inv]
    res2 = oracle.layer(N["x"], wr2, None, ex2, sp["k"])
    assert np.array_equal(res2["out"], res["out"])
    assert np.array_equal(res2["topk_id"], perm[res["topk_id"]])


def test_layer_tokens_matches_full_layer():
    sp, L, N = _tiny(T=9)
    ex = _experts_np(L["experts"])
    full = oracle.layer(N["x"], N["w_router"], None, ex, sp["k"])
    sub = oracle.layer_tokens(N["x"], N["w_router"], None, ex, sp["k"], [7, 2])
    assert np.array_equal(sub["topk_id"], full["topk_id"][[7, 2]])
    assert np.allclose(sub["out"], full["out"][[7, 2]], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- combine
def test_combine_one_hot_and_equal_rows():
    T, k, H = 3, 4, 16
    rng = np.random.default_rng(9)
    y = rng.standard_normal((T * k, H))
    slot_row = rng.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k))
    w[np.arange(T), [1, 3, 0]] = 1.0
    out = oracle.combine(y, slot_row, w, k, H)
    for t, j in enumerate([1, 3, 0]):
        assert np.array_equal(out[t], y[slot_row[t * k + j]])
    yy = np.tile(rng.standard_normal(H), (T * k, 1))
    w2 = np.full((T, k), 0.25)
    out2 = oracle.combine(yy, slot_row, w2, k, H)
    assert np.allclose(out2, yy[:T], rtol=1e-15)


def test_planted_transpose_is_caught_by_dense_pin():
    """A plausible mistake (down projection applied with the transposed index) must fail the
    textbook pin: shown on a copy of the arithmetic, on the CPU."""
    sp, L, N = _tiny(E=1, k=1, H=128, I=128)
    ex = _experts_np(L["experts"])
    Wg, Wu, Wd = (oracle.dequant(ex, 0, m) for m in range(3))
    x = L["x"].double().numpy()
    good = oracle.expert_rows(N["x"], ex, 0, np.arange(sp["T"]))
    bad = (_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd  # transposed down weights
    assert not np.allclose(good, bad, rtol=1e-3)


# ---------------------------------------------------------------- combine variants
def _golden_kv(name):
    return {r[0]: np.array([float(v) for v in r[1:]]) for r in _read_table(name)}


def test_combine_norm_hand_example():
    """Hand-worked example (tests/golden/combine_norm_example.txt): per-expert norm, plain
    weighted sum, and the post-norm + scaled residual + next pre-norm epilogue."""
    g = _golden_kv("combine_norm_example.txt")
    y = np.stack([g["y0"], g["y1"]])
    slot_row = g["slot_row"].astype(np.int32)
    w = g["topk_w"][None, :]
    plain = oracle.combine_norm(y, slot_row, w, 2, 4, eps=0.0)
    assert np.allclose(plain["out"][0], g["f_plain"], rtol=0, atol=1e-15)
    normed = oracle.combine_norm(y, slot_row, w, 2, 4, expert_norm=True, eps=0.0)
    assert np.allclose(normed["out"][0], g["f"], rtol=0, atol=1e-15)
    epi = oracle.combine_norm(y, slot_row, w, 2, 4, expert_norm=True, resid=g["resid"][None, :],
                              alpha=float(g["alpha"][0]), beta=float(g["beta"][0]),
                              gain=g["gain"], eps=0.0)
    assert np.allclose(epi["f"][0], g["f"], rtol=0, atol=1e-15)
    assert abs(epi["s"][0] - g["s"][0]) < 1e-13
    assert np.allclose(epi["out"][0], g["out"], rtol=0, atol=1e-13)
    assert abs(epi["r"][0] - g["r"][0]) < 1e-15
    assert np.allclose(epi["xn"][0], g["xn"], rtol=0, atol=1e-14)


def test_combine_norm_epsilon_closed_form():
    """One expert row of constant value c: mean square c^2, factor 1/sqrt(c^2 + eps)."""
    H = 8
    y = np.full((1, H), 2.0)
    out = oracle.combine_norm(y, np.array([0], np.int32), np.array([[0.5]]), 1, H,
                              expert_norm=True, eps=5.0)["out"]
    assert np.allclose(out, 0.5 * 2.0 / 3.0, rtol=1e-15)


def test_combine_norm_flags_off_is_weighted_sum():
    """Without the per-expert norm and the epilogue the variant is the plain routing-weighted
    sum: numpy's einsum over the gathered rows."""
    T, k, H = 5, 3, 24
    rng = np.random.default_rng(21)
    y = rng.standard_normal((T * k, H))
    slot_row = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    got = oracle.combine_norm(y, slot_row, w, k, H)["out"]
    want = np.einsum("tj,tjh->th", w, y[slot_row].reshape(T, k, H))
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


def test_combine_expert_norm_is_scale_invariant_per_expert():
    """With eps = 0 each expert's row is normalised before weighting: scaling one expert row by
    a positive factor leaves f unchanged, a negative one flips that expert's contribution.  A
    norm applied after the sum (or to the wrong rows) fails this."""
    T, k, H = 4, 3, 32
    rng = np.random.default_rng(22)
    y = rng.standard_normal((T * k, H))
    slot_row = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    base = oracle.combine_norm(y, slot_row, w, k, H, expert_norm=True, eps=0.0)["out"]
    y2 = y * rng.uniform(0.01, 100.0, (T * k, 1))
    same = oracle.combine_norm(y2, slot_row, w, k, H, expert_norm=True, eps=0.0)["out"]
    assert np.allclose(same, base, rtol=1e-12, atol=1e-13)
    t, j = 2, 1
    y3 = y.copy()
    y3[slot_row[t * k + j]] *= -7.0
    flip = oracle.combine_norm(y3, slot_row, w, k, H, expert_norm=True, eps=0.0)["out"]
    row = y[slot_row[t * k + j]]
    contrib = w[t, j] * row / np.sqrt(np.mean(row * row))
    assert np.allclose(flip[t], base[t] - 2 * contrib, rtol=1e-12, atol=1e-13)
    # k = 1, weight 1: the output row has root-mean-square exactly 1
    one = oracle.combine_norm(y[:T], np.arange(T, dtype=np.int32), np.ones((T, 1)), 1, H,
                              expert_norm=True, eps=0.0)["out"]
    assert np.allclose(np.sqrt(np.mean(one * one, axis=1)), 1.0, rtol=1e-14)


def test_combine_norm_after_sum_is_caught():
    """Planted mistake on the CPU: normalising the weighted sum instead of each expert row must
    differ from the oracle on rows of unequal scale."""
    T, k, H = 3, 4, 16
    rng = np.random.default_rng(23)
    y = rng.standard_normal((T * k, H)) * rng.uniform(0.1, 10.0, (T * k, 1))
    slot_row = np.arange(T * k, dtype=np.int32)
    w = rng.random((T, k))
    good = oracle.combine_norm(y, slot_row, w, k, H, expert_norm=True, eps=0.0)["out"]
    s = np.einsum("tj,tjh->th", w, y.reshape(T, k, H))
    bad = s / np.sqrt(np.mean(s * s, axis=1, keepdims=True))
    assert not np.allclose(good, bad, rtol=1e-3)


def test_combine_norm_epilogue_special_cases():
    """beta = 0, alpha = 1: the new residual is the old one and the next input is torch's RMS
    norm of it with the gain.  alpha = 0: the new residual is beta times the RMS-normalised MoE
    output (root-mean-square |beta|).  Scaling alpha and beta together scales the residual and
    leaves the next input unchanged (eps = 0)."""
    T, k, H = 6, 2, 40
    rng = np.random.default_rng(24)
    y = rng.standard_normal((T * k, H))
    slot_row = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    resid = rng.standard_normal((T, H)) * 3.0
    gain = rng.uniform(0.5, 1.5, H)
    eps = 1e-6
    a = oracle.combine_norm(y, slot_row, w, k, H, resid=resid, alpha=1.0, beta=0.0, gain=gain,
                            eps=eps)
    assert np.array_equal(a["out"], resid)
    want = torch.nn.functional.rms_norm(torch.from_numpy(resid), (H,),
                                        weight=torch.from_numpy(gain), eps=eps).numpy()
    assert np.allclose(a["xn"], want, rtol=1e-12, atol=1e-14)
    b = oracle.combine_norm(y, slot_row, w, k, H, expert_norm=True, resid=resid, alpha=0.0,
                            beta=-2.5, gain=gain, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(b["out"] ** 2, axis=1)), 2.5, rtol=1e-13)
    f = b["f"]
    assert np.allclose(b["xn"], -gain * f / np.sqrt(np.mean(f * f, axis=1, keepdims=True)),
                       rtol=1e-12, atol=1e-14)
    c1 = oracle.combine_norm(y, slot_row, w, k, H, resid=resid, alpha=0.7, beta=1.3, gain=gain,
                             eps=0.0)
    c2 = oracle.combine_norm(y, slot_row, w, k, H, resid=resid, alpha=0.7 * 4, beta=1.3 * 4,
                             gain=gain, eps=0.0)
    assert np.allclose(c2["out"], 4 * c1["out"], rtol=1e-13, atol=1e-13)
    assert np.allclose(c2["xn"], c1["xn"], rtol=1e-12, atol=1e-14)


def test_combine_norm_chain_matches_torch_rms_norm():
    """The whole variant composed from torch's RMS norm (float64, CPU): per-row norm of each
    expert output, weighted sum, norm factor of the sum, scaled residual, norm with gain."""
    T, k, H = 5, 4, 48
    rng = np.random.default_rng(25)
    y = rng.standard_normal((T * k, H))
    slot_row = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    resid = rng.standard_normal((T, H))
    gain = rng.uniform(0.5, 1.5, H)
    eps, alpha, beta = 1e-5, 0.9, 1.7
    got = oracle.combine_norm(y, slot_row, w, k, H, expert_norm=True, resid=resid, alpha=alpha,
                              beta=beta, gain=gain, eps=eps)
    rms = torch.nn.functional.rms_norm
    yt = rms(torch.from_numpy(y[slot_row]).reshape(T, k, H), (H,), eps=eps)
    f = (torch.from_numpy(w)[:, :, None] * yt).sum(1)
    out = alpha * torch.from_numpy(resid) + beta * rms(f, (H,), eps=eps)
    xn = rms(out, (H,), weight=torch.from_numpy(gain), eps=eps)
    assert np.allclose(got["f"], f.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(got["out"], out.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(got["xn"], xn.numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- low precision: fp8 (MX) variant
def test_mx_exp_closed_form():
    for j in range(-20, 20):
        assert oracle.mx_exp(2.0 ** j, 8) == j - 8
        assert oracle.mx_exp(2.0 ** j * 1.999, 8) == j - 8
        assert oracle.mx_exp(2.0 ** j * 0.999, 8) == j - 9
    assert oracle.mx_exp(0.0, 8) == -127
    assert oracle.mx_exp(2.0 ** -200, 8) == -127   # clamped
    assert oracle.mx_exp(2.0 ** 200, 8) == 127


def test_e4m3_code_round_trip_and_torch():
    """Every finite code (but -0) round-trips; random values round as torch's float8_e4m3fn
    cast does (to nearest, ties to even) below the saturation point; at or above 448 the code
    saturates."""
    for c in range(256):
        if c in (0x7F, 0xFF, 0x80):
            continue
        assert oracle.e4m3_code(oracle.e4m3(c)) == c, c
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.uniform(-4, 2.3, 2000),
                        [2.0 ** -10, 3 * 2.0 ** -11, 1.0625, 1.1875, 447.9, -0.0009]])
    v = v[np.abs(v) < 448]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_code(x) for x in v], np.uint8)
    zero = (want & 0x7F) == 0          # a negative value rounding to zero: -0 on both sides
    assert np.array_equal(got[~zero], want[~zero])
    assert np.all((got[zero] & 0x7F) == 0)
    # ties to the even mantissa, saturation
    assert oracle.e4m3_code(1.0625) == 0x38 and oracle.e4m3_code(1.1875) == 0x3A
    assert oracle.e4m3_code(448.0) == 0x7E and oracle.e4m3_code(1e6) == 0x7E
    assert oracle.e4m3_code(-500.0) == 0xFE


def test_mx8_quant_is_nearest_on_the_scaled_grid():
    """Brute force over all 254 finite e4m3 codes: each quantised value is a nearest point of the
    block's scaled grid (scale 2^(floor(log2 amax) - 8)); an all-zero block gives zero codes."""
    rng = np.random.default_rng(32)
    v = rng.standard_normal((3, 64)) * np.array([[1e-3], [1.0], [300.0]])
    v[1, 5] = 0.0
    codes, scales = oracle.mx8_quant(v)
    grid = np.array([oracle.e4m3(c) for c in range(256) if c not in (0x7F, 0xFF)])
    deq = oracle.mx8_dequant(codes, scales)
    for r in range(3):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            X = oracle.mx_scale(scales[r, b])
            amax = np.abs(blk).max()
            assert X == 2.0 ** (np.floor(np.log2(amax)) - 8)
            for i in range(32):
                dist = np.abs(grid * X - blk[i]).min()
                assert abs(deq[r, 32 * b + i] - blk[i]) <= dist * (1 + 1e-12)
    z = oracle.mx8_quant(np.zeros((1, 32)))
    assert np.all(z[0] == 0) and z[1][0, 0] == 0


def _tiny_mx():
    sp = dict(T=5, H=128, I=128, E=3, k=2, router="normal", zipf=None)
    L = synth.make_layer(sp, seed=33)
    ex = oracle.Experts(**{n: v.numpy() for n, v in L["experts"].items()})
    return sp, L, ex


def test_nvfp4_to_mxfp8_is_the_quantiser_on_exact_weights():
    """The requantised weights are MXFP8 of the exact NVFP4 weights (row by row), and every
    value is a nearest point of its block's scaled e4m3 grid."""
    sp, L, ex = _tiny_mx()
    mx = oracle.nvfp4_to_mxfp8(ex)
    grid = np.array([oracle.e4m3(c) for c in range(256) if c not in (0x7F, 0xFF)])
    for m in range(3):
        for e in range(ex.E):
            W = oracle.dequant(ex, e, m)
            q, s = (mx.gate_q, mx.up_q, mx.down_q)[m][e], (mx.gate_s, mx.up_s, mx.down_s)[m][e]
            cq, cs = oracle.mx8_quant(W)
            assert np.array_equal(q, cq) and np.array_equal(s, cs)
            Wq = oracle.mx8_weights(mx, e, m)
            for n in range(0, W.shape[0], 19):
                for kk in range(0, W.shape[1], 7):
                    X = oracle.mx_scale(s[n, kk // 32])
                    dist = np.abs(grid * X - W[n, kk]).min()
                    assert abs(Wq[n, kk] - W[n, kk]) <= dist * (1 + 1e-12)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def test_expert_rows_mx_composition_and_planted_mistake():
    """The fp8 expert FFN equals its pinned parts composed with numpy matmuls: MXFP8 x, MXFP8
    weights, SwiGLU, MXFP8 h, down.  Leaving h unquantised (a plausible slip) is caught, and the
    variant stays within its accuracy bar of the exact NVFP4 expert."""
    sp, L, ex = _tiny_mx()
    mx = oracle.nvfp4_to_mxfp8(ex)
    xb = _bits(L["x"])
    tok = np.array([0, 3, 4])
    x = L["x"].double().numpy()[tok]
    xq = oracle.mx8_dequant(*oracle.mx8_quant(x))
    for e in range(ex.E):
        Wg, Wu, Wd = (oracle.mx8_weights(mx, e, m) for m in range(3))
        h = _silu(xq @ Wg.T) * (xq @ Wu.T)
        hq = oracle.mx8_dequant(*oracle.mx8_quant(h))
        want = hq @ Wd.T
        got = oracle.expert_rows_mx(xb, mx, e, tok)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-15)
        slip = h @ Wd.T
        assert not np.allclose(got, slip, rtol=1e-4, atol=0)
        exact = oracle.expert_rows(xb, ex, e, tok)
        assert np.linalg.norm(got - exact) <= 0.15 * np.linalg.norm(exact)
