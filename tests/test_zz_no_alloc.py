"""moe_layer_nvfp4_noalloc, the allocation-free variant of moe_layer_nvfp4 (for callers that
cannot allocate device memory): its scratch is the library's own per-GPU array, shared by every
call on the GPU.  Through the C ABI, two calls in a row -- the second with a smaller input, so
the scratch holds the first call's contents -- must give exactly what moe_layer_nvfp4 gives on
a fresh zeroed workspace (the same kernels in the same order; the busy-expert chain runs on the
caller's stream instead of a side stream, which changes no arithmetic)."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

# (first call, second call): the four-call path (32-row GEMM tiles; few-row kernels plus the
# busy-expert chain) followed by the single launch, and a full-width decode pair
CASES = {
    "t37_then_t2": (dict(T=37, H=512, I=256, E=16, k=4, router="normal", zipf=None), 2),
    "t12_then_t1": (dict(T=12, H=256, I=128, E=8, k=4, router="normal", zipf=None), 1),
    "t64_then_t1_h7168": (dict(T=64, H=7168, I=2048, E=16, k=8, router="uniform", zipf=None), 1),
    "t2_then_t1_zipf": (dict(T=2, H=1024, I=256, E=64, k=8, router="normal", zipf=1.1), 1),
}
NAMES = ("out", "topk_id", "topk_w", "count", "offset", "sorted_slot", "slot_row", "active",
         "n_active")


def _run(moe, x, L, ex, k, noalloc, y_dtype):
    T, H = x.shape
    E, I = ex["gate_q"].shape[0], ex["gate_q"].shape[1]
    buf = moe.LayerBuffers(T, H, I, E, k, device="cuda", y_dtype=y_dtype)
    buf.out.fill_(7.0)
    buf.y.fill_(7.0)
    if noalloc:
        moe.layer_nvfp4_noalloc(x, L["w_router"], L["bias"], ex, k, buf)
    else:
        moe.layer_nvfp4(x, L["w_router"], L["bias"], ex, k, buf)
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_layer_entry(name):
    import bit_expert_ffn_amd as moe
    sp, t2 = CASES[name]
    print("case noalloc", name, sp, "then T=%d" % t2, flush=True)
    L = synth.make_layer(sp, seed=21, device="cuda")
    ex = moe.pack_experts(L["experts"])
    k = sp["k"]
    for y_dtype in (torch.float16, torch.float32):
        for T in (sp["T"], t2):  # two calls in a row, the second smaller
            x = L["x"][:T]
            want = _run(moe, x, L, ex, k, False, y_dtype)
            got = _run(moe, x, L, ex, k, True, y_dtype)
            assert not torch.isnan(got.out).any()
            for n in NAMES:
                assert torch.equal(getattr(got, n), getattr(want, n)), (T, n)
            if T > 2:  # the four-call path writes y
                assert torch.equal(got.y, want.y), (T, "y")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import bit_expert_ffn_amd as moe
    A = 0x10000  # never dereferenced: the call refuses the shape first
    ex = moe._Experts(A, A, A, A, A, A, A, 256, 7168, 2048)
    assert moe.workspace_size(4096, 7168, 2048, 256, 8) > 16 << 20
    st = moe.lib().moe_layer_nvfp4_noalloc(A, A, None, ctypes.byref(ex), 4096, 8, None, A, A, A,
                                           A, A, A, A, A, A, 1, A, None)
    assert st == -7 and "16 MiB" in moe.status_string(st)
