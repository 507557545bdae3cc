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


# From three tokens up moe_layer_nvfp4 runs route, group, expert FFN and combine in turn, and the
# one-block grouping also lists the busy experts' row tiles (the FFN call then skips its own
# planning launch).  Shapes: few-row kernels with busy experts on the side stream (12 tokens),
# 32-row GEMM tiles (37 and 96 tokens, the latter with a Zipf bias), 64-row tiles (600 tokens).
FOUR_CALL_SHAPES = {
    "t12_side_stream": dict(T=12, H=256, I=128, E=8, k=4, router="normal", zipf=None),
    "t37_rows32": dict(T=37, H=512, I=256, E=16, k=4, router="normal", zipf=None),
    "t96_zipf": dict(T=96, H=256, I=256, E=64, k=8, router="normal", zipf=1.1),
    "t600_rows64": dict(T=600, H=256, I=256, E=16, k=4, router="normal", zipf=None),
}


@pytest.mark.parametrize("name", list(FOUR_CALL_SHAPES))
def test_layer_entry_planned_grouping(name):
    """moe_layer_nvfp4 above two tokens: parity with the oracle, and bit-identical results to the
    four public calls made one by one (the same kernels; only the tile plan moves)."""
    import bit_expert_ffn_amd as moe
    sp = FOUR_CALL_SHAPES[name]
    print("case layer entry, planned grouping", name, sp, flush=True)
    L = synth.make_layer(sp, seed=12)
    buf, ex = run_fused(L, sp["k"])
    check_against_oracle(L, sp["k"], buf)
    T, H = L["x"].shape
    b4 = moe.LayerBuffers(T, H, sp["I"], sp["E"], sp["k"], device="cuda", y_dtype=torch.float16)
    bias = None if L["bias"] is None else L["bias"].cuda()
    moe.layer(L["x"].cuda(), L["w_router"].cuda(), bias, ex, sp["k"], b4)
    torch.cuda.synchronize()
    for n in ("topk_id", "topk_w", "count", "offset", "sorted_slot", "slot_row", "active",
              "n_active", "y", "out"):
        assert torch.equal(getattr(buf, n), getattr(b4, n)), n
