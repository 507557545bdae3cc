"""GPU parity of the HIP layer against the CPU oracle on seeded inputs that the oracle finishes
in seconds: the tiny workload, shapes spanning several tiles with ragged tails, edge cases, and
stage-by-stage checks on oracle-made inputs.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (check_out, check_routing, experts_np, gpu_layer, np_buf, oracle_on_selection,
                    tile_major_np, LOGIT_TOL, out_errors)

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": dict(synth.SPECS["tiny"]),
    "ragged_a": dict(T=37, H=512, I=256, E=16, k=4, router="normal", zipf=None),
    "multi_tile": dict(T=200, H=256, I=384, E=32, k=6, router="normal", zipf=None),
    "wide_k": dict(T=5, H=1024, I=128, E=64, k=8, router="normal", zipf=None),
    "max_e": dict(T=64, H=256, I=128, E=256, k=8, router="uniform", zipf=None),
    "single_expert": dict(T=33, H=256, I=256, E=1, k=1, router="normal", zipf=None),
    "dense_k_eq_e": dict(T=6, H=256, I=128, E=8, k=8, router="normal", zipf=None),
    "zipf_skew": dict(T=96, H=256, I=256, E=64, k=8, router="normal", zipf=1.1),
    "one_token": dict(T=1, H=1024, I=256, E=32, k=8, router="normal", zipf=None),
    "two_tokens": dict(T=2, H=512, I=384, E=16, k=4, router="normal", zipf=None),
    "one_token_wide": dict(T=1, H=7168, I=256, E=8, k=2, router="normal", zipf=None),
    # 512 <= T < 2048: 64-row GEMM tiles (32-row below, 128-row from 2048)
    "mid_64_row_tiles": dict(T=600, H=256, I=256, E=16, k=4, router="normal", zipf=None),
    # the prefill configuration at small H and I: T >= 2048 gives 128-row GEMM tiles (with the
    # x -> f16 conversion kernel) and T*k = 16800 > 16384 slots the three-pass grouping
    "prefill_tiles_128": dict(T=2100, H=256, I=256, E=16, k=8, router="normal", zipf=None),
}


def _full_check(L, k, y_dtype=torch.float32):
    """Every output of the layer against the oracle: logits, ids (near-ties aside), all grouping
    arrays bit-exact, every expert-output row y and every token's out.  A near-tie token that
    took the alternative selection is compared with the oracle run on that selection."""
    print("case", L["spec"], "y", y_dtype, flush=True)
    N = synth.to_numpy(L)
    ex = experts_np(L["experts"])
    ref = oracle.layer(N["x"], N["w_router"], N["bias"], ex, k)
    g = np_buf(gpu_layer(L, k, y_dtype))
    assert np.max(np.abs(g["logits"] - ref["logits"])) <= LOGIT_TOL
    exempt = check_routing(g["topk_id"], g["topk_w"], ref["logits"], ref["topk_w"], k)
    _, _, grp, y_ref, out_ref = oracle_on_selection(N["x"], ex, ref, exempt, k)
    for name in ("count", "offset", "sorted_slot", "slot_row", "active"):
        assert np.array_equal(g[name], grp[name]), name
    assert int(g["n_active"][0]) == grp["n_active"]
    check_out(g["y"], y_ref)
    mr, ma = check_out(g["out"], out_ref)
    print("near-ties %d max_rel %.3e mae %.3e" % (len(exempt), mr, ma))
    return mr, ma


@pytest.mark.parametrize("name", list(SHAPES))
def test_layer_parity(name):
    L = synth.make_layer(SHAPES[name], seed=0)
    _full_check(L, SHAPES[name]["k"])


@pytest.mark.parametrize("name", ["ragged_a", "prefill_tiles_128"])
def test_layer_parity_f16_y(name):
    """y in f16, as the benchmark runs the layer."""
    L = synth.make_layer(SHAPES[name], seed=1)
    _full_check(L, SHAPES[name]["k"], torch.float16)


def test_all_rows_to_one_expert():
    sp = dict(T=70, H=256, I=128, E=16, k=2, router="normal", zipf=None)
    L = synth.make_layer(sp, seed=2)
    bias = torch.zeros(16)
    bias[3] = 100.0  # expert 3 is every token's first choice
    L["bias"] = bias
    _full_check(L, 2)


def test_random_code_bytes_cover_every_decode():
    """Every e2m1 code and every finite e4m3 scale code, positive and negative."""
    sp = dict(T=8, H=256, I=128, E=4, k=2, router="normal", zipf=None)
    L = synth.make_layer(sp, seed=3)
    g = torch.Generator().manual_seed(3)
    for n, t in L["experts"].items():
        if n.endswith("_q"):
            t.copy_(torch.randint(0, 256, t.shape, generator=g, dtype=torch.int32).to(torch.uint8))
        elif n.endswith("_s"):
            c = torch.randint(0, 254, t.shape, generator=g, dtype=torch.int32)
            c = torch.where(c >= 127, c + 1, c)  # skip 0x7F and 0xFF (NaN)
            t.copy_(c.to(torch.uint8))
    L["experts"]["ts"].fill_(1.5e-4)
    seen = set(L["experts"]["gate_s"].flatten().tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}
    _full_check(L, 2)


def test_deterministic_bitwise():
    L = synth.make_layer(SHAPES["multi_tile"], seed=4)
    a = np_buf(gpu_layer(L, 6))
    b = np_buf(gpu_layer(L, 6))
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# ---------------------------------------------------------------- stage-by-stage
def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (64, 8, 256), (2048, 8, 256), (2049, 8, 256),
                                   (4096, 8, 256), (16384, 8, 256), (50, 3, 5)])
def test_group_stage_bit_exact(T, k, E):
    """moe_group on seeded ids (one-block path up to 16384 slots, three-pass above)."""
    import bit_expert_ffn_amd as moe
    rng = np.random.default_rng(T + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ref = oracle.group(ids, E)
    ws = torch.zeros(moe.workspace_size(T, 128, 128, E, k), dtype=torch.uint8, device="cuda")
    out = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
           (("count", E), ("offset", E + 1), ("sorted_slot", T * k), ("slot_row", T * k),
            ("active", E), ("n_active", 1))}
    moe.group(_dev_i32(ids), E, out["count"], out["offset"], out["sorted_slot"], out["slot_row"],
              out["active"], out["n_active"], ws)
    torch.cuda.synchronize()
    for n in ("count", "offset", "sorted_slot", "slot_row", "active"):
        assert np.array_equal(out[n].cpu().numpy(), ref[n]), n
    assert int(out["n_active"].item()) == ref["n_active"]


def test_ffn_and_combine_stages_on_oracle_inputs():
    import bit_expert_ffn_amd as moe
    sp = SHAPES["multi_tile"]
    L = synth.make_layer(sp, seed=5)
    N = synth.to_numpy(L)
    ex = experts_np(L["experts"])
    k = sp["k"]
    ids, w = oracle.topk(oracle.router(N["x"], N["w_router"]), k)
    grp = oracle.group(ids, sp["E"])
    y_ref = oracle.ffn(N["x"], ex, grp, k)
    x = L["x"].cuda()
    exd = moe.pack_experts({n: v.cuda() for n, v in L["experts"].items()})
    T, H = x.shape
    ws = torch.zeros(moe.workspace_size(T, H, sp["I"], sp["E"], k), dtype=torch.uint8, device="cuda")
    y = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
    moe.expert_ffn_nvfp4(x, exd, _dev_i32(grp["count"]), _dev_i32(grp["offset"]),
                         _dev_i32(grp["sorted_slot"]), _dev_i32(grp["active"]),
                         _dev_i32([grp["n_active"]]), k, y, ws)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), y_ref)
    # combine alone, on the oracle's y rounded to fp32 and its fp32 weights
    y32 = torch.from_numpy(y_ref.astype(np.float32)).cuda()
    w32 = torch.from_numpy(w.astype(np.float32)).cuda()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.combine(y32, _dev_i32(grp["slot_row"]), w32, out)
    torch.cuda.synchronize()
    ref = oracle.combine(y_ref.astype(np.float32), grp["slot_row"], w.astype(np.float32), k, H)
    mr, ma = out_errors(out.cpu().numpy(), ref)
    assert mr < 1e-6 and ma < 1e-7


def test_route_stage_zero_input_and_ties():
    """x = 0: every logit equals the bias; equal logits go to the lower expert id and the
    weights are exactly 1/k."""
    import bit_expert_ffn_amd as moe
    T, H, E, k = 3, 256, 64, 8
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    wr = torch.randn((H, E), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.zeros(moe.workspace_size(T, H, 128, E, k), dtype=torch.uint8, device="cuda")
    moe.route(x, wr, None, k, ids, w, ws)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [list(range(k))] * T
    assert torch.all(w.cpu() == 1.0 / k)


@pytest.mark.parametrize("T,H,E,k,zipf", [
    (64, 256, 8, 2, None),         # below the matrix-core router: fp32 slices
    (128, 7168, 256, 8, 1.1),      # the verify shape (fp32 slices)
    (512, 256, 8, 2, None),        # smallest token count of the matrix-core router
    (513, 384, 40, 4, None),       # ragged token tile, experts not a multiple of 32 or 64
    (1000, 1024, 256, 8, 1.1),     # Zipf bias, several hidden-dimension slices
    (700, 7168, 256, 8, None),     # full hidden size
])
def test_route_stage_matrix_core(T, H, E, k, zipf):
    """Router around and above the switch to the matrix cores (512 tokens): logits within the
    fp32 reordering tolerance of the oracle's, top-k ids exact except near-ties, weights to fp32
    accuracy."""
    import bit_expert_ffn_amd as moe
    print("case route T=%d H=%d E=%d k=%d zipf=%s" % (T, H, E, k, zipf), flush=True)
    x = synth.make_x(T, H, seed=7)
    wr = synth.make_router(H, E, seed=7)
    bias = synth.make_zipf_bias(E, zipf, seed=7) if zipf else None
    ref_logits = oracle.router(x.view(torch.int16).numpy().view(np.uint16), wr.numpy(),
                               None if bias is None else bias.numpy())
    ref_ids, ref_w = oracle.topk(ref_logits, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.workspace_size(T, H, 128, E, k), dtype=torch.uint8, device="cuda")
    moe.route(x.cuda(), wr.cuda(), None if bias is None else bias.cuda(), k, ids, w, ws,
              logits=logits)
    torch.cuda.synchronize()
    assert np.max(np.abs(logits.cpu().numpy() - ref_logits)) <= LOGIT_TOL
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref_logits, ref_w, k)


@pytest.mark.parametrize("T,H,E", [(8, 384, 40), (600, 1024, 72)])
def test_route_one_hot_rows_exact(T, H, E):
    """x[t] = one-hot at h_t: the logits are row h_t of the router weights, bit for bit (on the
    matrix-core router this needs the three bf16 pieces of every weight to add up exactly)."""
    import bit_expert_ffn_amd as moe
    print("case one-hot route T=%d H=%d E=%d" % (T, H, E), flush=True)
    g = torch.Generator().manual_seed(T + H + E)
    h_t = torch.randint(0, H, (T,), generator=g)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    x[torch.arange(T), h_t] = 1.0
    wr = torch.randn((H, E), generator=g) * 0.02
    k = 2
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.workspace_size(T, H, 128, E, k), dtype=torch.uint8, device="cuda")
    moe.route(x.cuda(), wr.cuda(), None, k, ids, w, ws, logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(logits.cpu(), wr[h_t])


@pytest.mark.parametrize("E,N,K", [(2, 16, 128), (3, 48, 384), (1, 256, 256)])
def test_pack_tile_major_bit_exact(E, N, K):
    import bit_expert_ffn_amd as moe
    g = torch.Generator().manual_seed(E * N + K)
    q = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    s = torch.randint(0, 256, (E, N, K // 16), generator=g, dtype=torch.int32).to(torch.uint8)
    qo, so = moe.nvfp4_pack(q.cuda(), s.cuda())
    torch.cuda.synchronize()
    rq, rs = tile_major_np(q.numpy(), s.numpy())
    assert np.array_equal(qo.cpu().numpy(), rq)
    assert np.array_equal(so.cpu().numpy(), rs)
