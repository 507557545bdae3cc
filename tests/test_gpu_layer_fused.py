"""GPU parity of moe_layer_nvfp4, the whole layer in one call: for one or two tokens it runs as a
single persistent kernel (router, top-k, grouping, gate/up + SwiGLU, down + combine), whose
blocks wait for each other through counters at the start of the workspace.  Checked against the
CPU oracle on seeded inputs: ids exact (except near-ties), grouping arrays exact, outputs within
the layer's bars; the counters must be back at zero after every call, and repeated calls must
give bit-identical results."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import LOGIT_TOL, check_out, check_routing, experts_np, oracle_token_out

pytestmark = pytest.mark.gpu

SHAPES = {
    "t1_tiny": dict(T=1, H=256, I=128, E=8, k=2, router="normal", zipf=None),
    "t2_small": dict(T=2, H=512, I=384, E=16, k=4, router="normal", zipf=None),
    "t1_odd_experts": dict(T=1, H=1024, I=256, E=37, k=8, router="normal", zipf=None),
    "t2_wide_h": dict(T=2, H=7168, I=256, E=8, k=2, router="normal", zipf=None),
    "t1_one_chunk_i": dict(T=1, H=384, I=128, E=64, k=8, router="uniform", zipf=None),
    "t2_max_slots": dict(T=2, H=256, I=256, E=32, k=16, router="normal", zipf=None),
    "t1_zipf_bias": dict(T=1, H=512, I=256, E=256, k=8, router="normal", zipf=1.1),
    "t2_single_expert": dict(T=2, H=256, I=128, E=1, k=1, router="normal", zipf=None),
    "t1_k32": dict(T=1, H=256, I=128, E=64, k=32, router="normal", zipf=None),
}


def run_fused(L, k, device="cuda", buf=None, ex=None):
    import bit_expert_ffn_amd as moe
    x = L["x"].to(device)
    T, H = x.shape
    if ex is None:
        ex = moe.pack_experts({n: v.to(device) for n, v in L["experts"].items()})
    E, I = ex["gate_q"].shape[0], ex["gate_q"].shape[1]
    if buf is None:
        buf = moe.LayerBuffers(T, H, I, E, k, device=device, y_dtype=torch.float16)
    bias = None if L["bias"] is None else L["bias"].to(device)
    moe.layer_nvfp4(x, L["w_router"].to(device), bias, ex, k, buf)
    torch.cuda.synchronize()
    return buf, ex


def sync_words(buf):
    return buf.ws[:65536].view(torch.int32).cpu().numpy()


def check_against_oracle(L, k, buf):
    N = synth.to_numpy(L)
    exn = experts_np(L["experts"])
    ref = oracle.layer(N["x"], N["w_router"], N["bias"], exn, k)
    ids = buf.topk_id.cpu().numpy()
    assert np.max(np.abs(buf.logits.cpu().numpy() - ref["logits"])) <= LOGIT_TOL
    exempt = check_routing(ids, buf.topk_w.cpu().numpy(), ref["logits"], ref["topk_w"], k)
    r_out = ref["out"].copy()
    if not exempt:
        for name in ("count", "offset", "sorted_slot", "slot_row", "active"):
            assert np.array_equal(getattr(buf, name).cpu().numpy(), ref["group"][name]), name
        assert int(buf.n_active.item()) == ref["group"]["n_active"]
    for t, sel in exempt.items():
        r_out[t] = oracle_token_out(N["x"], exn, t, sel, ref["logits"][t])
    return check_out(buf.out.cpu().numpy(), r_out)


@pytest.mark.parametrize("name", list(SHAPES))
def test_fused_layer_parity(name):
    sp = SHAPES[name]
    print("case fused", name, sp, flush=True)
    L = synth.make_layer(sp, seed=3)
    buf, _ = run_fused(L, sp["k"])
    assert not np.any(sync_words(buf)), "counters or error word not zero after the call"
    mr, ma = check_against_oracle(L, sp["k"], buf)
    print("max_rel %.3e mae %.3e" % (mr, ma))


def test_fused_layer_repeated_calls_bit_identical():
    """Counters reset by each call: back-to-back calls on one workspace, then a different input
    and back again, all bit-identical to the first results."""
    sp = SHAPES["t2_small"]
    print("case fused repeated", sp, flush=True)
    L = synth.make_layer(sp, seed=5)
    buf, ex = run_fused(L, sp["k"])
    first = {n: getattr(buf, n).clone() for n in ("out", "topk_id", "topk_w", "sorted_slot")}
    L2 = dict(L)
    L2["x"] = synth.make_x(sp["T"], sp["H"], seed=6)
    for i in range(6):
        run_fused(L2 if i == 3 else L, sp["k"], buf=buf, ex=ex)
        assert not np.any(sync_words(buf))
        if i != 3:
            for n, v in first.items():
                assert torch.equal(getattr(buf, n), v), (i, n)


def test_fused_matches_four_call_path():
    """The single launch and the four calls agree (combine order differs: not bitwise)."""
    import bit_expert_ffn_amd as moe
    sp = SHAPES["t1_odd_experts"]
    print("case fused vs four calls", sp, flush=True)
    L = synth.make_layer(sp, seed=8)
    buf, ex = run_fused(L, sp["k"])
    T, H = L["x"].shape
    b4 = moe.LayerBuffers(T, H, sp["I"], sp["E"], sp["k"], device="cuda")
    bias = None if L["bias"] is None else L["bias"].cuda()
    moe.layer(L["x"].cuda(), L["w_router"].cuda(), bias, ex, sp["k"], b4)
    torch.cuda.synchronize()
    for n in ("topk_id", "count", "offset", "sorted_slot", "slot_row", "active", "n_active"):
        assert torch.equal(getattr(buf, n), getattr(b4, n)), n
    assert torch.allclose(buf.topk_w, b4.topk_w, atol=1e-6, rtol=0)
    check_out(buf.out.cpu().numpy(), b4.out.cpu().numpy().astype(np.float64), max_rel=1e-5, mae=1e-6)


def test_fused_layer_zero_input_ties():
    """x = 0: all logits equal; ties go to the lower expert id, weights exactly 1/k."""
    sp = dict(T=2, H=256, I=128, E=64, k=8, router="normal", zipf=None)
    print("case fused zero input", sp, flush=True)
    L = synth.make_layer(sp, seed=10)
    L["x"] = torch.zeros_like(L["x"])
    buf, _ = run_fused(L, sp["k"])
    assert buf.topk_id.cpu().tolist() == [list(range(8))] * 2
    assert torch.all(buf.topk_w.cpu() == 1.0 / 8)
    assert torch.all(buf.out.cpu() == 0)


def test_fused_layer_falls_back_for_many_tokens():
    """T above the single-launch limit runs the four calls (y written)."""
    sp = dict(T=5, H=256, I=128, E=8, k=2, router="normal", zipf=None)
    print("case fused entry, four-call path", sp, flush=True)
    L = synth.make_layer(sp, seed=9)
    buf, _ = run_fused(L, sp["k"])
    check_against_oracle(L, sp["k"], buf)


# From three tokens up moe_layer_nvfp4 routes, groups and plans the grouped GEMM's row tiles in
# one persistent kernel (up to 128 tokens; router on the matrix cores), or in separate kernels
# whose one-block grouping also lists the row tiles (above 128 tokens), then runs the expert FFN
# and the combine.  Shapes: few-row kernels with busy experts on the side stream (3 and 12
# tokens), 32-row GEMM tiles (37, 64, 96 and 128 tokens, Zipf bias at 96 and 128, full hidden
# size at 64 and 128), 64-row tiles (600 tokens, separate routing kernels).
FOUR_CALL_SHAPES = {
    "t3_few_rows": dict(T=3, H=512, I=256, E=16, k=4, router="normal", zipf=None),
    "t12_side_stream": dict(T=12, H=256, I=128, E=8, k=4, router="normal", zipf=None),
    "t37_rows32": dict(T=37, H=512, I=256, E=16, k=4, router="normal", zipf=None),
    "t64_h7168": dict(T=64, H=7168, I=256, E=64, k=8, router="uniform", zipf=None),
    "t96_zipf": dict(T=96, H=256, I=256, E=64, k=8, router="normal", zipf=1.1),
    "t128_e256_zipf": dict(T=128, H=7168, I=128, E=256, k=8, router="normal", zipf=1.1),
    "t128_odd_e_k32": dict(T=128, H=384, I=128, E=37, k=32, router="normal", zipf=None),
    "t600_rows64": dict(T=600, H=256, I=256, E=16, k=4, router="normal", zipf=None),
}


def near_tie_tokens(L, a_ids, b_ids, k):
    """Tokens whose ids differ between two runs must be near-ties of the oracle's logits."""
    N = synth.to_numpy(L)
    ref_logits = oracle.router(N["x"], N["w_router"], N["bias"])
    from parity import route_candidates
    bad = np.nonzero((a_ids != b_ids).any(1))[0]
    for t in bad:
        c = route_candidates(ref_logits[t], k)
        assert len(c) > 1 and tuple(a_ids[t]) in c and tuple(b_ids[t]) in c, t
    return set(bad.tolist())


@pytest.mark.parametrize("name", list(FOUR_CALL_SHAPES))
def test_layer_entry_planned_grouping(name):
    """moe_layer_nvfp4 above two tokens: parity with the oracle, and agreement with the four
    public calls made one by one: ids and grouping exact (near-ties aside), routing weights and
    outputs to fp32 summation order (the fused routing kernel sums the logits on the matrix
    cores, the public router on the VALU); bit-identical where both route the same way (600)."""
    import bit_expert_ffn_amd as moe
    sp = FOUR_CALL_SHAPES[name]
    print("case layer entry, planned grouping", name, sp, flush=True)
    L = synth.make_layer(sp, seed=12)
    buf, ex = run_fused(L, sp["k"])
    moe.layer_check(buf.ws)
    assert not np.any(sync_words(buf)), "counters or flags not reset"
    mr, ma = check_against_oracle(L, sp["k"], buf)
    print("oracle: max_rel %.3e mae %.3e" % (mr, ma))
    T, H = L["x"].shape
    b4 = moe.LayerBuffers(T, H, sp["I"], sp["E"], sp["k"], device="cuda", y_dtype=torch.float16)
    bias = None if L["bias"] is None else L["bias"].cuda()
    moe.layer(L["x"].cuda(), L["w_router"].cuda(), bias, ex, sp["k"], b4)
    torch.cuda.synchronize()
    if T > 128:
        for n in ("logits", "topk_id", "topk_w", "count", "offset", "sorted_slot", "slot_row",
                  "active", "n_active", "y", "out"):
            assert torch.equal(getattr(buf, n), getattr(b4, n)), n
        return
    assert torch.allclose(buf.logits, b4.logits, atol=1e-4, rtol=0)
    ties = near_tie_tokens(L, buf.topk_id.cpu().numpy(), b4.topk_id.cpu().numpy(), sp["k"])
    if not ties:
        for n in ("topk_id", "count", "offset", "sorted_slot", "slot_row", "active", "n_active"):
            assert torch.equal(getattr(buf, n), getattr(b4, n)), n
        assert torch.allclose(buf.topk_w, b4.topk_w, atol=2e-6, rtol=0)
        check_out(buf.out.cpu().numpy(), b4.out.cpu().numpy().astype(np.float64),
                  max_rel=1e-4, mae=1e-5)


@pytest.mark.parametrize("T,H,E", [(3, 384, 40), (64, 1024, 72), (128, 7168, 256)])
def test_layer_entry_router_one_hot_exact(T, H, E):
    """x[t] = one-hot at h_t: through the fused routing kernel the logits are row h_t of the
    router weights bit for bit (the three bf16 pieces of each weight add up exactly)."""
    import bit_expert_ffn_amd as moe
    print("case fused routing one-hot T=%d H=%d E=%d" % (T, H, E), flush=True)
    g = torch.Generator().manual_seed(T + H + E)
    sp = dict(T=T, H=H, I=128, E=E, k=2, router="normal", zipf=None)
    L = synth.make_layer(sp, seed=14)
    h_t = torch.randint(0, H, (T,), generator=g)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    x[torch.arange(T), h_t] = 1.0
    L["x"] = x
    wr = (torch.randn((H, E), generator=g) * 0.02).float()
    L["w_router"] = wr
    buf, _ = run_fused(L, 2)
    assert torch.equal(buf.logits.cpu(), wr[h_t])


def test_layer_entry_zero_input_ties():
    """x = 0 through the fused routing kernel: all logits equal, ties go to the lower expert id,
    the weights are exactly 1/k and the output is zero."""
    sp = dict(T=5, H=256, I=128, E=64, k=8, router="normal", zipf=None)
    print("case fused routing zero input", sp, flush=True)
    L = synth.make_layer(sp, seed=15)
    L["x"] = torch.zeros_like(L["x"])
    buf, _ = run_fused(L, sp["k"])
    assert buf.topk_id.cpu().tolist() == [list(range(8))] * 5
    assert torch.all(buf.topk_w.cpu() == 1.0 / 8)
    assert torch.all(buf.out.cpu() == 0)


@pytest.mark.parametrize("name", ["t12_side_stream", "t96_zipf"])
@pytest.mark.parametrize("word", [0, 16])
def test_layer_entry_routing_gives_up_and_recovers(name, word):
    """The fused routing kernel with a barrier that cannot complete (counter A or C preset from
    the host, short spin limit): every block gives up and exits, the counters are reset, the
    error word is set; block 0 leaves a grouping with no active expert and NaN weights, so the
    expert FFN does nothing, the combine stays inside y and out is NaN.  moe_layer_check
    reports it; the next call is correct again, bit for bit."""
    import bit_expert_ffn_amd as moe
    sp = FOUR_CALL_SHAPES[name]
    print("case fused routing give-up", name, "word", word, flush=True)
    L = synth.make_layer(sp, seed=16)
    buf, ex = run_fused(L, sp["k"])
    moe.layer_check(buf.ws)
    first = {n: getattr(buf, n).clone() for n in ("out", "topk_id", "topk_w", "y")}
    words = buf.ws[:65536].view(torch.int32)
    moe.set_layer_spin_limit(buf.ws, 2000)
    words[word] = 1 << 30
    run_fused(L, sp["k"], buf=buf, ex=ex)
    assert torch.isnan(buf.out).all()
    assert int(buf.n_active.item()) == 0
    w = sync_words(buf)
    assert w[48] != 0 and w[49] == 2000
    assert not np.delete(w, [48, 49]).any(), "counters or flags left set"
    with pytest.raises(RuntimeError, match="moe_layer_check"):
        moe.layer_check(buf.ws)
    moe.set_layer_spin_limit(buf.ws, 0)
    run_fused(L, sp["k"], buf=buf, ex=ex)
    moe.layer_check(buf.ws)
    for n, v in first.items():
        assert torch.equal(getattr(buf, n), v), n


# (shape, word): the top-level counter of barrier A (word 0) or C (word 16); with one token and
# k = 8 the kernel's per-XCD mode replaces barrier C by one barrier per group of blocks, whose
# group-0 counter is word 320 (the 256th word after the first flag copy)
GIVE_UP_CASES = [("t1_tiny", 0), ("t1_tiny", 16), ("t2_small", 0), ("t2_small", 16),
                 ("t1_odd_experts", 0), ("t1_odd_experts", 320)]


@pytest.mark.parametrize("name,word", GIVE_UP_CASES)
def test_fused_layer_gives_up_and_recovers(name, word):
    """A barrier that cannot complete, forced from the host: an arrival counter preset far above
    the number of arrivals, so no arrival completes it, with a short spin limit (word 49).  The
    blocks waiting on it must give up and write NaN over their features of out (in the per-XCD
    mode they write NaN into their rows of the partial buffer, and the one group that gives up
    covers every range of features), every block must still make its remaining arrivals (the
    exit counter, or in the per-XCD mode its range counter) and leave the counters and flags
    reset; the error word is set and moe_layer_check reports it and clears it; the next call on
    the same workspace is correct again, bit for bit."""
    import bit_expert_ffn_amd as moe
    sp = SHAPES[name]
    print("case fused give-up", name, "word", word, flush=True)
    L = synth.make_layer(sp, seed=13)
    buf, ex = run_fused(L, sp["k"])
    moe.layer_check(buf.ws)
    first = {n: getattr(buf, n).clone() for n in ("out", "topk_id", "topk_w")}
    words = buf.ws[:65536].view(torch.int32)
    moe.set_layer_spin_limit(buf.ws, 2000)
    words[word] = 1 << 30
    buf.out.fill_(-1.0)
    run_fused(L, sp["k"], buf=buf, ex=ex)  # synchronises: every block has exited
    assert torch.isnan(buf.out).all(), "blocks that gave up must write NaN over their features"
    w = sync_words(buf)
    assert w[48] != 0, "error word not set"
    assert w[49] == 2000
    rest = np.delete(w, [48, 49])
    assert not rest.any(), "counters or flags left set: words %s" % np.nonzero(rest)[0][:8]
    with pytest.raises(RuntimeError, match="moe_layer_check"):
        moe.layer_check(buf.ws)
    w = sync_words(buf)
    assert w[48] == 0 and w[49] == 2000
    moe.set_layer_spin_limit(buf.ws, 0)
    run_fused(L, sp["k"], buf=buf, ex=ex)
    moe.layer_check(buf.ws)
    assert not np.any(sync_words(buf))
    for n, v in first.items():
        assert torch.equal(getattr(buf, n), v), n
