"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
the whole layer runs on every token; the CPU oracle recomputes a sample of tokens one by one
(routing and FFN are per token, so a sampled token's output is exact), and the grouping arrays
are checked by invariants that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import LOGIT_TOL, check_out, check_routing, oracle_token_out

pytestmark = pytest.mark.gpu

_cache = {}


def _layer(name):
    """Inputs generated on the GPU (as the benchmark does) plus host copies for the oracle."""
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        sp = dict(synth.SPECS[name])
        T = sp["T"] * (4 if sp["T"] == 1 else 1)  # decode: a few pool tokens, one call each
        L = synth.make_layer(sp, seed=0, device="cuda", T=T)
        ex_host = oracle.Experts(**{n: v.cpu().numpy() for n, v in L["experts"].items()})
        _cache[name] = (sp, L, ex_host)
    return _cache[name]


def _run(L, x, k):
    import bit_expert_ffn_amd as moe
    T, H = x.shape
    ex = L.setdefault("_packed", None) or moe.pack_experts(L["experts"])
    L["_packed"] = ex
    E, I = ex["gate_q"].shape[0], ex["gate_q"].shape[1]
    # f16 expert outputs, as the benchmark runs the layer
    buf = moe.LayerBuffers(T, H, I, E, k, device="cuda", y_dtype=torch.float16)
    moe.layer(x, L["w_router"], L["bias"], ex, k, buf)
    torch.cuda.synchronize()
    return buf


def _check_group_invariants(buf, E, k):
    ids = buf.topk_id.cpu().numpy()
    T = ids.shape[0]
    count = buf.count.cpu().numpy()
    offset = buf.offset.cpu().numpy()
    ss = buf.sorted_slot.cpu().numpy()
    sr = buf.slot_row.cpu().numpy()
    active = buf.active.cpu().numpy()
    na = int(buf.n_active.item())
    assert np.array_equal(count, np.bincount(ids.ravel(), minlength=E))
    assert offset[0] == 0 and np.array_equal(np.diff(offset), count) and offset[E] == T * k
    assert np.array_equal(np.sort(ss), np.arange(T * k))
    assert np.array_equal(sr[ss], np.arange(T * k))
    for e in np.nonzero(count)[0]:
        seg = ss[offset[e]:offset[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(ids.ravel()[seg] == e)
    act = [e for e in range(E) if count[e] > 0]
    act.sort(key=lambda e: (-count[e], e))
    assert na == len(act) and list(active[:na]) == act and np.all(active[na:] == -1)
    for t in range(min(T, 64)):
        assert len(set(ids[t].tolist())) == k  # distinct experts per token


def _check_tokens(sp, L, ex_host, buf, tokens, x_all, t_offset=0):
    k = sp["k"]
    xb = x_all.cpu().view(torch.int16).numpy().view(np.uint16)
    wr = L["w_router"].cpu().numpy()
    bias = None if L["bias"] is None else L["bias"].cpu().numpy()
    ref = oracle.layer_tokens(xb, wr, bias, ex_host, k, [t + t_offset for t in tokens])
    g_ids = buf.topk_id.cpu().numpy()[tokens]
    g_w = buf.topk_w.cpu().numpy()[tokens]
    g_logits = buf.logits.cpu().numpy()[tokens]
    assert np.max(np.abs(g_logits - ref["logits"])) <= LOGIT_TOL
    exempt = check_routing(g_ids, g_w, ref["logits"], ref["topk_w"], k)
    r_out = ref["out"].copy()
    for i, ids in exempt.items():
        r_out[i] = oracle_token_out(xb, ex_host, tokens[i] + t_offset, ids, ref["logits"][i])
    g_out = buf.out.cpu().numpy()[tokens]
    mr, ma = check_out(g_out, r_out)
    print("%d token(s) from %d: max_rel %.3e mae %.3e near-ties %d"
          % (len(tokens), tokens[0] + t_offset, mr, ma, len(exempt)))


def test_decode1_full():
    """T=1 calls on pool tokens 0..3 (each call = one benchmark step)."""
    sp, L, ex_host = _layer("decode1")
    print("case decode1 T=1 H=7168 I=2048 E=256 k=8", flush=True)
    for t in range(4):
        x = L["x"][t:t + 1]
        buf = _run(L, x, sp["k"])
        _check_group_invariants(buf, sp["E"], sp["k"])
        _check_tokens(sp, L, ex_host, buf, [0], L["x"], t_offset=t)


def test_decode1_full_single_launch():
    """The benchmark's decode configuration: one call of moe_layer_nvfp4 per token (a single
    persistent kernel), pool tokens 0..3 on one workspace."""
    import bit_expert_ffn_amd as moe
    sp, L, ex_host = _layer("decode1")
    print("case decode1 single launch T=1 H=7168 I=2048 E=256 k=8", flush=True)
    ex = L.setdefault("_packed", None) or moe.pack_experts(L["experts"])
    L["_packed"] = ex
    buf = moe.LayerBuffers(1, sp["H"], sp["I"], sp["E"], sp["k"], device="cuda",
                           y_dtype=torch.float16)
    for t in range(4):
        moe.layer_nvfp4(L["x"][t:t + 1], L["w_router"], L["bias"], ex, sp["k"], buf)
        torch.cuda.synchronize()
        assert not buf.ws[:65536].any().item(), "counters or flags not reset"
        _check_group_invariants(buf, sp["E"], sp["k"])
        _check_tokens(sp, L, ex_host, buf, [0], L["x"], t_offset=t)


def test_decode64_full():
    """Every one of the 64 tokens against the oracle."""
    sp, L, ex_host = _layer("decode64")
    print("case decode64 T=64, all tokens", flush=True)
    buf = _run(L, L["x"], sp["k"])
    _check_group_invariants(buf, sp["E"], sp["k"])
    _check_tokens(sp, L, ex_host, buf, list(range(sp["T"])), L["x"])


def test_decode64_layer_entry():
    _entry_against_four_calls("decode64", [0, 13, 31, 50, 63])


def test_verify128_full():
    """Every one of the 128 tokens against the oracle (Zipf-skewed loads: busy experts on
    several 32-row GEMM tiles)."""
    sp, L, ex_host = _layer("verify128")
    print("case verify128 T=128 I=256 zipf, all tokens", flush=True)
    buf = _run(L, L["x"], sp["k"])
    _check_group_invariants(buf, sp["E"], sp["k"])
    counts = buf.count.cpu().numpy()
    assert counts.max() > 32  # the Zipf bias gives some experts several 32-row tiles
    _check_tokens(sp, L, ex_host, buf, list(range(sp["T"])), L["x"])


def _run_entry(L, x, k):
    """moe_layer_nvfp4 (for 3..128 tokens: the fused routing kernel, then the expert FFN and
    the combine), as the benchmark times the layer at these sizes."""
    import bit_expert_ffn_amd as moe
    T, H = x.shape
    ex = L.setdefault("_packed", None) or moe.pack_experts(L["experts"])
    L["_packed"] = ex
    E, I = ex["gate_q"].shape[0], ex["gate_q"].shape[1]
    buf = moe.LayerBuffers(T, H, I, E, k, device="cuda", y_dtype=torch.float16)
    moe.layer_nvfp4(x, L["w_router"], L["bias"], ex, k, buf)
    torch.cuda.synchronize()
    moe.layer_check(buf.ws)
    return buf


def _entry_against_four_calls(name, sample):
    """The layer entry against the four public calls (checked against the oracle on every
    token above) on every token, and against the oracle directly on a sample of tokens."""
    from parity import route_candidates
    sp, L, ex_host = _layer(name)
    k = sp["k"]
    print("case %s through moe_layer_nvfp4" % name, flush=True)
    be = _run_entry(L, L["x"], k)
    b4 = _run(L, L["x"], k)
    _check_group_invariants(be, sp["E"], k)
    ge, g4 = be.topk_id.cpu().numpy(), b4.topk_id.cpu().numpy()
    diff = np.nonzero((ge != g4).any(1))[0]
    if len(diff):
        xb = L["x"].cpu().view(torch.int16).numpy().view(np.uint16)
        wr = L["w_router"].cpu().numpy()
        bias = None if L["bias"] is None else L["bias"].cpu().numpy()
        lg = oracle.router(xb[diff], wr, bias)
        for i, t in enumerate(diff):
            c = route_candidates(lg[i], k)
            assert tuple(ge[t]) in c and tuple(g4[t]) in c, "token %d: not a near-tie" % t
    same = np.setdiff1d(np.arange(sp["T"]), diff)
    check_out(be.out.cpu().numpy()[same], b4.out.cpu().numpy()[same].astype(np.float64),
              max_rel=1e-4, mae=1e-5)
    _check_tokens(sp, L, ex_host, be, sample, L["x"])


def test_verify128_layer_entry():
    _entry_against_four_calls("verify128", list(range(0, 128, 9)))


def tile_covering_tokens(buf, k, mt=128, n=128):
    """Tokens whose (token, slot) rows land on every row position 0..mt-1 of an expert's
    mt-row GEMM tiles: position p is taken from the expert active[p % n_active], in its tile
    p % (rows // mt), so the positions are spread over experts and over their tiles."""
    count = buf.count.cpu().numpy()
    offset = buf.offset.cpu().numpy()
    ss = buf.sorted_slot.cpu().numpy()
    active = buf.active.cpu().numpy()
    na = int(buf.n_active.item())
    toks = []
    for p in range(mt):
        e = int(active[p % na])
        ntile = max(1, int(count[e]) // mt)
        row = int(offset[e]) + mt * (p % ntile) + p
        assert row < offset[e] + count[e]
        t = int(ss[row]) // k
        if t not in toks:
            toks.append(t)
    rng = np.random.default_rng(0)
    while len(toks) < n:  # seeded extra tokens up to n
        t = int(rng.integers(0, len(ss) // k))
        if t not in toks:
            toks.append(t)
    return sorted(toks)


def test_prefill16k_full():
    """128 tokens whose rows hit every row position of a 128-row GEMM tile (and tiles 0..3 of
    their experts), against the oracle token by token."""
    sp, L, ex_host = _layer("prefill16k")
    print("case prefill16k T=16384", flush=True)
    buf = _run(L, L["x"], sp["k"])
    _check_group_invariants(buf, sp["E"], sp["k"])
    counts = buf.count.cpu().numpy()
    assert counts.min() > 300 and counts.max() < 800
    k = sp["k"]
    toks = tile_covering_tokens(buf, k)
    # the chosen tokens' rows cover every position of a 128-row tile
    sr = buf.slot_row.cpu().numpy()
    offset = buf.offset.cpu().numpy()
    ids = buf.topk_id.cpu().numpy()
    pos = {int(sr[t * k + j] - offset[ids[t, j]]) % 128 for t in toks for j in range(k)}
    assert pos == set(range(128))
    print("comparing %d tokens" % len(toks), flush=True)
    _check_tokens(sp, L, ex_host, buf, toks, L["x"])
