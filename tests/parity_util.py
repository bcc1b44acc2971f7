"""GPU-vs-oracle comparison helpers for the parity tests.

Rules (what the GPU result must satisfy):
  * top-K ids: equal as sets to the oracle's for every token whose fp64
    logit margin z_(K) - z_(K+1) is at least 1e-4 (bit-exact integers);
    tokens below that margin are "flagged" and their output is compared
    against the oracle re-evaluated with the GPU's own expert set.  A router
    on the latent with bf16 activations reads u as the kernel stores it, in
    bf16, while the oracle routes on the exact u: such a token is flagged
    too when its margin is below twice the largest logit shift that
    rounding u can cause (latent_router_shift_bound).
  * counts: equal to the histogram of the GPU's own ids, summing to T*K;
    equal to the oracle's counts once flagged tokens are removed from both.
  * offsets: exclusive prefix sum of counts; token_of/slot_of: the unique
    expert-grouped order (expert id, then token index) of the GPU's ids.
  * outputs: per token, ||out_gpu - out_oracle|| / ||out_oracle|| <= tol
    (2e-2 with bf16 activations, 6e-2 with fp8 expert weights, 1e-4 fp32).
"""
from __future__ import annotations

import numpy as np

MARGIN = 1e-4


def tolerance(spec) -> float:
    if spec.expert_dtype == "fp8_e4m3_rowscale":
        return 6e-2
    if spec.act_dtype == "bf16":
        return 2e-2
    return 1e-4


def latent_router_shift_bound(spec, w_np, x_np, tok, latent):
    """Per token, an upper bound on |z_gpu,e - z_e| over the experts e when
    the router reads the bf16-stored latent: rounding u_c to bf16 (8
    significant bits, relative error <= 2^-8) after an fp32 accumulation
    over d terms (error <= g_d sum_j |W_down[c][j] x_j|, g_n = n 2^-24 /
    (1 - n 2^-24)), then an fp32 accumulation of the logit over l terms.
    A top-K set can only change if the K-th/(K+1)-th margin is below twice
    this bound."""
    import oracle
    def gam(n):
        return n * 2.0 ** -24 / (1.0 - n * 2.0 ** -24)
    Wd = oracle.upcast(w_np["w_down"], spec.act_dtype)
    Wr = np.abs(oracle.upcast(w_np["w_router"], spec.act_dtype))
    X = oracle.upcast(x_np[tok], spec.act_dtype)
    eps = gam(spec.d) * (np.abs(X) @ np.abs(Wd).T)             # [n][l]
    au = np.abs(latent)
    du = 2.0 ** -8 * au + 2.0 * eps                            # |bf16(u_gpu) - u|
    shift = du @ Wr.T + gam(spec.l) * (1.01 * au + du) @ Wr.T  # [n][N]
    return shift.max(axis=1)


def _bf16_latent_router(spec) -> bool:
    return spec.router_on_latent and spec.act_dtype == "bf16" and spec.has_projections


def flag_tokens(spec, w_np, x_np, tok, ref):
    """Tokens whose id set is not compared (see the module rules)."""
    flagged = ref["margin"] < MARGIN
    if _bf16_latent_router(spec):
        b = latent_router_shift_bound(spec, w_np, x_np, tok, ref["latent"])
        flagged |= ref["margin"] < 2.0 * b
    return flagged


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(spec, w_np, x_np, device="cuda:0", layer=None, overlap=None, packed=False):
    """One forward call through the C ABI; packed: with the banded copy of
    the expert weights (latentmoe_pack_expert_weights) as well."""
    import torch
    import mixture_experts_layer_32_amd as pkg
    layer = layer or pkg.LatentMoELayer(spec)
    T = x_np.shape[0]
    dev = pkg.to_device(pkg.pack_gated(dict(w_np, x=x_np)), device)
    if packed:
        dev["experts_packed"] = layer.pack_expert_weights(dev)
    dbg = pkg.debug_buffers(spec, T, device)
    out = layer.forward(dev["x"], dev, debug=dbg, overlap=overlap)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() if v.dtype != torch.bfloat16 else to_f64(v) for k, v in dbg.items()}
    res["out"] = to_f64(out)
    return res, layer


def check_routing_structure(spec, g, T):
    """Integer invariants of the GPU routing that hold at any size."""
    N, K = spec.n_experts, spec.top_k
    idx = g["topk_idx"]
    assert idx.shape == (T, K)
    assert idx.min() >= 0 and idx.max() < N
    srt = np.sort(idx, axis=1)
    assert (np.diff(srt, axis=1) > 0).all(), "duplicate expert in a token's top-k"
    counts = g["expert_counts"].astype(np.int64)
    assert counts.sum() == T * K
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=N))
    off = g["expert_offsets"].astype(np.int64)
    assert off[0] == 0 and np.array_equal(np.diff(off), counts)
    # unique expert-grouped order: by expert id, then token index
    flat_e = idx.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T), K)
    order = np.lexsort((flat_t, flat_e))
    assert np.array_equal(g["token_of"].astype(np.int64), flat_t[order])
    slot = np.empty(T * K, np.int64)
    slot[order] = np.arange(T * K)
    assert np.array_equal(g["slot_of"].reshape(-1).astype(np.int64), slot)


def check_against_oracle(spec, w_np, x_np, g, tokens=None, orc=None, gate_atol=2e-4,
                         logit_atol=None):
    """Compare GPU results for `tokens` (default all) with the fp64 oracle.
    Returns a dict of statistics."""
    import oracle as orc_mod
    orc = orc or orc_mod
    T = x_np.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    ref = orc.forward(spec, w_np, x_np, tokens=tok, want_logits=True, want_latent=True)
    gidx = g["topk_idx"][tok]
    flagged = flag_tokens(spec, w_np, x_np, tok, ref)
    same = (np.sort(gidx, 1) == np.sort(ref["idx"], 1)).all(1)
    bad = ~same & ~flagged
    assert not bad.any(), "top-k ids differ on unflagged tokens %s" % tok[bad][:10].tolist()

    # logits (GPU buffer holds W_r . x without the bias)
    zl = g["logits"][tok].astype(np.float64)
    if spec.has_router_bias:
        zl = zl + w_np["router_bias"].astype(np.float64)[None, :]
    if logit_atol is None:
        logit_atol = 5e-5 if spec.act_dtype == "bf16" else 2e-5
    if _bf16_latent_router(spec):
        # the kernel's logits read the bf16 latent: within the shift bound
        lim = logit_atol + latent_router_shift_bound(spec, w_np, x_np, tok, ref["latent"])
        zdev = np.abs(zl - ref["logits"]).max(axis=1)
        assert (zdev <= lim).all(), "router logits beyond the bf16-latent bound"
    else:
        zerr = np.abs(zl - ref["logits"]).max()
        assert zerr <= logit_atol, "router logits differ by %g" % zerr

    # gates of unflagged tokens, matched by expert id.  A bf16-latent router
    # shifts every logit by at most delta (latent_router_shift_bound); each
    # gate (softmax, or sigmoid normalised over the set) then moves by a
    # factor within [e^-2delta, e^2delta].
    ok = ~flagged
    if ok.any():
        gg = g["topk_gate"][tok][ok].astype(np.float64)
        gi = gidx[ok]
        rg = ref["gate"][ok]
        ri = ref["idx"][ok]
        rel_g = np.zeros(gi.shape[0])
        if _bf16_latent_router(spec):
            delta = latent_router_shift_bound(spec, w_np, x_np, tok, ref["latent"])[ok]
            rel_g = np.expm1(2.0 * delta)
        for r in range(gi.shape[0]):
            m = {int(e): v for e, v in zip(ri[r], rg[r])}
            for j in range(gi.shape[1]):
                want_g = m[int(gi[r, j])]
                assert abs(gg[r, j] - want_g) <= gate_atol + rel_g[r] * want_g, "gate mismatch"

    # outputs; flagged tokens re-evaluated with the GPU's own expert set
    want = ref["out"].copy()
    if flagged.any():
        fr = orc.forward(spec, w_np, x_np, tokens=tok[flagged], forced=gidx[flagged])
        want[flagged] = fr["out"]
    got = g["out"][tok]
    nrm = np.linalg.norm(want, axis=1)
    rel = np.linalg.norm(got - want, axis=1) / np.maximum(nrm, 1e-30)
    tol = tolerance(spec)
    assert np.isfinite(got).all(), "non-finite GPU output"
    assert rel.max() <= tol, "max per-token rel err %.3g > %.3g (token %d)" % (
        rel.max(), tol, tok[int(np.argmax(rel))])
    # latent u when there are projections
    if spec.has_projections and "latent" in g:
        u = g["latent"][tok]
        ur = ref["latent"]
        lrel = np.linalg.norm(u - ur, axis=1) / np.maximum(np.linalg.norm(ur, axis=1), 1e-30)
        assert lrel.max() <= max(tol, 1e-2 if spec.act_dtype == "bf16" else 1e-5), lrel.max()
    # counts over unflagged tokens when every token was evaluated
    if tokens is None:
        N = spec.n_experts
        c_g = np.bincount(g["topk_idx"][~flagged].reshape(-1), minlength=N)
        c_o = np.bincount(ref["idx"][~flagged].reshape(-1), minlength=N)
        assert np.array_equal(c_g, c_o)
    frob = np.linalg.norm(got - want) / np.linalg.norm(want)
    return {"max_rel": float(rel.max()), "frob_rel": float(frob), "flagged": int(flagged.sum()),
            "n": int(len(tok))}


def check_routing_all_tokens(spec, w_np, x_np, g, logit_atol=None):
    """Every token at any size: the oracle's routing alone (fp64 logits,
    (z desc, id asc) top-K, margins) against the GPU's.  The id sets of all
    unflagged tokens are equal; the per-expert counts over the unflagged
    tokens are equal (both bit-exact); the GPU's fp32 logits (W_r x, the
    bias added apart) are within logit_atol of the oracle's.  Returns
    statistics."""
    import oracle
    assert not (spec.router_on_latent and spec.act_dtype == "bf16"), \
        "latent routers on bf16 need the latent; use check_against_oracle"
    T, N = x_np.shape[0], spec.n_experts
    ref = oracle.route(spec, w_np, x_np, want_logits=True)
    gidx = g["topk_idx"]
    flagged = ref["margin"] < MARGIN
    same = (np.sort(gidx, 1) == np.sort(ref["idx"], 1)).all(1)
    bad = ~same & ~flagged
    assert not bad.any(), "top-k ids differ on %d unflagged tokens, e.g. %s" % (
        int(bad.sum()), np.nonzero(bad)[0][:10].tolist())
    c_g = np.bincount(gidx[~flagged].reshape(-1), minlength=N)
    c_o = np.bincount(ref["idx"][~flagged].reshape(-1), minlength=N)
    assert np.array_equal(c_g, c_o), "per-expert counts over unflagged tokens differ"
    zl = g["logits"].astype(np.float64)
    if spec.has_router_bias:
        zl = zl + w_np["router_bias"].astype(np.float64)[None, :]
    if logit_atol is None:
        logit_atol = 5e-5 if spec.act_dtype == "bf16" else 2e-5
    zerr = float(np.abs(zl - ref["logits"]).max())
    assert zerr <= logit_atol, "router logits differ by %g" % zerr
    return {"tokens": int(T), "flagged": int(flagged.sum()), "max_logit_err": zerr,
            "touched_experts": int((c_o > 0).sum())}
