"""Phase timeline of the persistent kernels inside moe_layer_nvfp4 (a profiling tool).

Needs the profiling library, built beforehand with

    python -m bit_expert_ffn_amd.build --timeline     (-> libmoe_nvfp4_timeline.so)

in which every block of the single-launch layer (one or two tokens) and of the fused routing
kernel (3..128 tokens) records the 100 MHz real-time counter at its phase boundaries.  Usage:

    python -m bit_expert_ffn_amd.timeline WORKLOAD [--calls N]

runs the layer on the seeded inputs of WORKLOAD (decode1 cycles through 64 tokens, as the
benchmark does), after 0.5 s of untimed calls, and prints for each phase boundary the median,
90th percentile and maximum over blocks and calls, in microseconds from the first block's
entry of the same call."""
import argparse
import ctypes
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

LAYER_SMALL = ["entry", "router partials stored", "barrier A passed", "routing published, gate/up starts",
               "gate/up done", "barrier C passed", "h staged", "exit", "logits summed", "first-level ranks",
               "candidate ranks (top-k known)", "first gate/up sets issued", "first down set used",
               "last down set used", "range counter passed"]
LAYER_SMALL_ORDER = [0, 1, 2, 8, 9, 10, 11, 3, 4, 5, 6, 12, 13, 7, 14]
ROUTE_GROUP = ["entry", "router partials stored", "barrier A passed", "top-k done", "barrier C passed",
               "rows placed", "active list sorted", "exit", "router loads issued", "router products done",
               "router sums in LDS"]
ROUTE_GROUP_ORDER = [0, 8, 9, 10, 1, 2, 3, 4, 5, 6, 7]
# blocks that record each slot of the fused routing kernel: all, or the T token blocks, or block 0
ROUTE_GROUP_BLOCKS = ["all", "all", "token", "token", "token", "token", "block 0", "all", "all", "all", "all"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--calls", type=int, default=50)
    ap.add_argument("--per-block", type=int, default=None, metavar="SLOT",
                    help="also print each block's median time at this slot (blocks go round-robin "
                         "to the 8 XCDs, so block b runs on XCD b %% 8), and the per-XCD medians")
    args = ap.parse_args()
    import bit_expert_ffn_amd as moe
    from bit_expert_ffn_amd import build as b
    if not os.path.exists(b.TIMELINE_LIB):
        sys.exit("%s is missing: build it with python -m bit_expert_ffn_amd.build --timeline"
                 % b.TIMELINE_LIB)
    moe.LIB_PATH = b.TIMELINE_LIB  # before the first call into the library
    sys.path.insert(0, ROOT)
    import synth

    dev = torch.device("cuda", 0)
    sp = dict(synth.SPECS[args.workload])
    T = sp["T"]
    if T > 128:
        sys.exit("the persistent kernels run up to 128 tokens")
    pool = 64 if T == 1 else 1
    layer = synth.make_layer(sp, seed=0, device=dev, T=T * pool)
    ex = moe.pack_experts(layer["experts"])
    buf = moe.LayerBuffers(T, sp["H"], sp["I"], sp["E"], sp["k"], device=dev,
                           y_dtype=torch.float16, logits=False)
    calls = [moe.prepare_layer_nvfp4(layer["x"][i * T:(i + 1) * T], layer["w_router"],
                                     layer["bias"], ex, sp["k"], buf) for i in range(pool)]
    L = moe.lib()
    small = T <= 2
    read = L.moe_timeline_layer_small if small else L.moe_timeline_route_group
    read.argtypes = [ctypes.c_void_p]
    read.restype = ctypes.c_int
    names = LAYER_SMALL if small else ROUTE_GROUP

    i = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        for _ in range(8):
            calls[i % pool]()
            i += 1
        torch.cuda.synchronize()
    runs = []
    for _ in range(args.calls):
        for _ in range(4):
            calls[i % pool]()
            i += 1
        torch.cuda.synchronize()
        h = np.zeros((1024, 16), np.uint64)
        if read(ctypes.c_void_p(h.ctypes.data)) != 0:
            sys.exit("reading the timeline failed")
        runs.append(h)
    moe.layer_check(buf.ws)

    G = int((runs[0][:, 0] > 0).sum())  # blocks of the grid (every block stamps its entry)
    rel = []
    for h in runs:
        h = h[:G].astype(np.int64)
        r = (h - h[:, 0].min()) * 0.01
        r[h == 0] = np.nan
        rel.append(r)
    rel = np.stack(rel)  # [calls][blocks][slots]
    print("%s: %s, T=%d, %d blocks, %d calls (us from the first block's entry)" % (
        "layer_small_kernel" if small else "route_group_kernel", args.workload, T, G, args.calls))
    for j in (LAYER_SMALL_ORDER if small else ROUTE_GROUP_ORDER):
        name = names[j]
        who = "all" if small else ROUTE_GROUP_BLOCKS[j]
        v = rel[:, :T, j] if who == "token" else rel[:, :1, j] if who == "block 0" else rel[:, :, j]
        v = v[~np.isnan(v)]
        if v.size:
            label = name if small else "%s (%s)" % (name, "token blocks" if who == "token" else
                                                    "block 0" if who == "block 0" else "all blocks")
            print("  %-44s median %7.2f   p90 %7.2f   max %7.2f" % (
                label, np.median(v), np.percentile(v, 90), v.max()))
    if args.per_block is not None:
        med = np.nanmedian(rel[:, :, args.per_block], axis=0)  # [blocks]
        print("slot %d (%s), median over calls per block:" % (args.per_block, names[args.per_block]))
        for x in range(8):
            v = med[x::8]
            v = v[~np.isnan(v)]
            print("  XCD %d (blocks %d, %d, ...): median %7.2f  max %7.2f" % (x, x, x + 8, np.median(v), v.max()))
        order = np.argsort(-np.nan_to_num(med, nan=-1.0))[:16]
        print("  latest blocks: " + ", ".join("%d (%.2f)" % (b, med[b]) for b in order))


if __name__ == "__main__":
    main()
