"""Comparison rules between the HIP layer and the CPU oracle.

Bars:
  - expert ids bit-exact, except at near-ties: where two neighbouring logits in a token's
    ranking (down to the (k+1)-th) differ by less than NEAR_TIE, the oracle's own ranking with
    that pair swapped is also accepted, and that token's output is checked against the oracle run
    on the swapped selection (the alternative comes from the oracle's logits, never from the GPU);
  - grouping arrays bit-exact;
  - routing weights within W_TOL (absolute), logits within LOGIT_TOL (absolute);
  - layer output: normwise max relative error max|g - r| / max|r| <= MAX_REL and mean absolute
    error <= MAE over all compared outputs.
"""
import numpy as np
import torch

import oracle
import synth

NEAR_TIE = 1e-5
MAX_REL = 2e-2
MAE = 1e-3
# fp32 logits summed in a different order than the oracle's double sum rounded once:
# |error| <~ sqrt(H) * 2^-24 * |running sum|, a few 1e-6 at H = 7168; softmax slope <= 1/4.
LOGIT_TOL = 1e-4
W_TOL = 2e-5


def ranking(logits_row):
    return sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))


def route_candidates(logits_row, k):
    order = ranking(logits_row)
    cands = [tuple(order[:k])]
    lim = min(k, len(order) - 1)
    for i in range(lim):
        if float(logits_row[order[i]]) - float(logits_row[order[i + 1]]) < NEAR_TIE:
            alt = list(order)
            alt[i], alt[i + 1] = alt[i + 1], alt[i]
            cands.append(tuple(alt[:k]))
    return cands


def check_routing(gpu_ids, gpu_w, ref_logits, ref_w, k):
    """Returns {token: alternative ids} for near-tie tokens that took an alternative."""
    exempt = {}
    for t in range(gpu_ids.shape[0]):
        g = tuple(int(v) for v in gpu_ids[t])
        cands = route_candidates(ref_logits[t], k)
        if g == cands[0]:
            assert np.max(np.abs(gpu_w[t] - ref_w[t])) <= W_TOL, (t, gpu_w[t], ref_w[t])
            continue
        assert g in cands[1:], "token %d: GPU ids %s, oracle %s (not a near-tie)" % (t, g, cands[0])
        exempt[t] = g
        l = ref_logits[t, list(g)].astype(np.float64)
        p = np.exp(l - l.max())
        assert np.max(np.abs(gpu_w[t] - p / p.sum())) <= W_TOL
    return exempt


def out_errors(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    d = np.abs(g - r)
    return float(d.max() / max(np.abs(r).max(), 1e-30)), float(d.mean())


def check_out(g, r, max_rel=MAX_REL, mae=MAE):
    mr, ma = out_errors(g, r)
    assert mr <= max_rel and ma <= mae, "max_rel %.3e (bar %.1e), mae %.3e (bar %.1e)" % (mr, max_rel, ma, mae)
    return mr, ma


def selection_weights(ids, logits_row):
    """Softmax over the oracle's logits of a given selection (fp64)."""
    l = logits_row[list(ids)].astype(np.float64)
    p = np.exp(l - l.max())
    return p / p.sum()


def oracle_on_selection(x_bits, ex, ref, exempt, k):
    """The oracle's grouping, expert rows and combine on the selection the comparison accepts:
    the oracle's own ids, except near-tie tokens whose GPU ids are one of the alternatives that
    check_routing derived from the oracle's logits (weights then recomputed from the oracle's
    logits).  Returns (ids, w, grouping, y, out)."""
    ids = ref["topk_id"].copy()
    w = np.array(ref["topk_w"], np.float64)
    for t, sel in exempt.items():
        ids[t] = sel
        w[t] = selection_weights(sel, ref["logits"][t])
    if not exempt:
        return ids, w, ref["group"], ref["y"], ref["out"]
    grp = oracle.group(ids, ex.E)
    y = oracle.ffn(x_bits, ex, grp, k)
    out = oracle.combine(y, grp["slot_row"], w, k, ex.H)
    return ids, w, grp, y, out


def oracle_token_out(x_bits, ex, t, ids, logits_row):
    """Oracle output of token t for a given selection (used for near-tie alternatives)."""
    l = logits_row[list(ids)].astype(np.float64)
    p = np.exp(l - l.max())
    p /= p.sum()
    out = np.zeros(ex.H)
    for j, e in enumerate(ids):
        out += p[j] * oracle.expert_rows(x_bits, ex, e, [t])[0]
    return out


def gpu_layer(L, k, y_dtype=torch.float32, device="cuda"):
    import bit_expert_ffn_amd as moe
    x = L["x"].to(device)
    T, H = x.shape
    ex = moe.pack_experts({n: v.to(device) for n, v in L["experts"].items()})
    E, I = ex["gate_q"].shape[0], ex["gate_q"].shape[1]
    buf = moe.LayerBuffers(T, H, I, E, k, device=device, y_dtype=y_dtype)
    bias = None if L["bias"] is None else L["bias"].to(device)
    moe.layer(x, L["w_router"].to(device), bias, ex, k, buf)
    torch.cuda.synchronize()
    return buf


def np_buf(buf):
    return {n: getattr(buf, n).cpu().numpy() for n in
            ("logits", "topk_id", "topk_w", "count", "offset", "sorted_slot", "slot_row",
             "active", "n_active", "out")} | {"y": buf.y.float().cpu().numpy()}


def tile_major_np(q, s):
    """Reference of the tile-major layout, written from its offset formula (numpy)."""
    E, N, k2 = q.shape
    K = k2 * 2
    qo = np.empty(E * N * K // 2, np.uint8)
    so = np.empty(E * N * K // 16, np.uint8)
    for e in range(E):
        for n in range(N):
            for c in range(K // 128):
                for g in range(4):
                    l = 16 * g + n % 16
                    t = (n // 16) * (K // 128) + c
                    qo[e * N * K // 2 + (t * 64 + l) * 16:][:16] = q[e, n, c * 64 + g * 16:][:16]
                    so[e * N * K // 16 + (t * 64 + l) * 2:][:2] = s[e, n, c * 8 + g * 2:][:2]
    return qo.reshape(q.shape), so.reshape(s.shape)


def experts_np(ex):
    return oracle.Experts(**{k: v.cpu().numpy() for k, v in ex.items()})
