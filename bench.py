"""Benchmark of the Stem prefill hot path on one MI355X.

One step = one attention layer: stem_score (OAM pooling + scoring GEMM), stem_tpd_topk (fused TPD budget +
top-k selection) and bsa_prefill (block-sparse attention over the selected blocks), on seeded synthetic
inputs already resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload llama_128k_bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # dense MFMA TFLOP/s, MI355X
METRIC = "ms/layer + effective TFLOPS (%MFMA peak), 25%-budget prefill at 32K/128K"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def describe(p):
    return (f"{p.name}: {len(p.lens)} request(s) of {'/'.join(str(x) for x in p.lens)} tokens, "
            f"{p.hq} query / {p.hkv} KV heads, head_dim {p.d}, block {p.block}, {p.dtype}, "
            f"{'paged ' + str(p.page_size) + '-token pages, ' if p.paged else ''}"
            f"budget {p.rho_num}/{p.rho_den}, mu {p.mu_num}/{p.mu_den}, beta {p.beta}")


def setup(p, x, dev):
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    kw = {}
    if p.dtype == "fp8":
        kw = dict(q_scale=upload(x["q_scale"]), k_scale=upload(x["k_scale"]), v_scale=upload(x["v_scale"]))
    if p.paged:
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype,
                                 page_table=upload(x["page_table"]), page_size=p.page_size,
                                 num_pages=x["k_pages"].shape[0], **kw)
        k, v = upload(x["k_pages"]), upload(x["v_pages"])
    else:
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, **kw)
        k, v = upload(x["k"]), upload(x["v"])
    q = upload(x["q"])
    return StemPrefill(prob, dev), q, k, v


def visible_pairs(p, words, NB):
    """Causally visible query-key pairs of the selected blocks (from the packed mask)."""
    total = 0
    cb = p.cu_blocks
    for r, L in enumerate(p.lens):
        n = p.nblocks(r)
        sizes = np.array([min(p.block, L - j * p.block) for j in range(n)], dtype=np.int64)
        w = words[:, cb[r]:cb[r + 1]].astype(np.uint32)
        bits = ((w[..., None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(p.hq, n, -1)[:, :, :n].astype(bool)
        bits &= np.tril(np.ones((n, n), dtype=bool))[None]
        off = (bits & ~np.eye(n, dtype=bool)[None]).astype(np.int64) @ sizes  # [hq][n] keys before the diagonal
        diag = bits[:, np.arange(n), np.arange(n)].astype(np.int64) * (sizes * (sizes + 1) // 2)[None]
        total += int((off * sizes[None]).sum() + diag.sum())
    return total


def dense_pairs(p):
    return sum(p.hq * L * (L + 1) // 2 for L in p.lens)


def time_layer(L, q, k, v, p, steps, warmup, torch):
    rho, mu = (p.rho_num, p.rho_den), (p.mu_num, p.mu_den)
    for _ in range(warmup):
        L.forward(q, k, v, p.beta, rho, mu)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        e = evs[s]
        e[0].record()
        L.score(q, k, v, p.beta)
        e[1].record()
        L.select(rho, mu)
        e[2].record()
        L.attend(q, k, v, "selected", True)
        e[3].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in evs])  # ms
    return wall, stage.mean(axis=0), stage[:, 2]


def time_layer_cold(L, q, k, v, p, steps, warmup, torch, dev):
    """The headline protocol: `warmup` untimed steps, then `steps` steps each preceded by overwriting a 1 GiB
    buffer (evicts L2 and the 256 MB MALL; outside the step's events).  Returns the median layer time, the
    per-stage medians, every step's BSA time, and the wall time per step (flush included)."""
    rho, mu = (p.rho_num, p.rho_den), (p.mu_num, p.mu_den)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        L.forward(q, k, v, p.beta, rho, mu)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        scratch.fill_(1)
        e = evs[s]
        e[0].record()
        L.score(q, k, v, p.beta)
        e[1].record()
        L.select(rho, mu)
        e[2].record()
        L.attend(q, k, v, "selected", True)
        e[3].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in evs])  # ms
    layer = stage.sum(axis=1)
    del scratch
    return float(np.median(layer)), np.median(stage, axis=0), stage[:, 2], layer, wall


def stage_bytes(p):
    """Algorithmic HBM bytes of the two selection stages.  Scoring: one read of Q, K and V, the pooled
    q-bar, k-bar, M written once, the causal block scores written once.  Selection: the causal scores read
    once, the mask and the counts written once."""
    eb = {"f32": 4, "bf16": 2, "fp8": 1}[p.dtype]
    nb = [p.nblocks(r) for r in range(len(p.lens))]
    NB = sum(nb)
    words = (max(nb) + 31) // 32
    causal = sum(n * (n + 1) // 2 for n in nb)
    inputs = p.tokens * (p.hq + 2 * p.hkv) * p.d * eb
    pooled = ((p.hq + p.hkv) * p.d + p.hkv) * NB * 4
    scores = p.hq * causal * 4
    return inputs + pooled + scores, scores + p.hq * NB * (words + 1) * 4


def time_bsa(L, q, k, v, mask, reps, torch, inloop=False, expand_v=True):
    L.attend(q, k, v, mask, False, inloop=inloop, expand_v=expand_v)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        L.attend(q, k, v, mask, False, inloop=inloop, expand_v=expand_v)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def fused_vs_two_stage(L, q, k, v, p, torch, reps=10):
    """Fused scoring + selection (stem_score_select) against the two stages run back to back, both warm,
    each timed over `reps` calls; the fused masks are checked against the two-stage ones."""
    rho, mu = (p.rho_num, p.rho_den), (p.mu_num, p.mu_den)
    L.score(q, k, v, p.beta)
    L.select(rho, mu)
    torch.cuda.synchronize()
    ref_mask, ref_counts = L.mask.clone(), L.counts.clone()

    def run(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    two = run(lambda: (L.score(q, k, v, p.beta), L.select(rho, mu)))
    L.mask.zero_()
    fused = run(lambda: L.score_select(q, k, v, p.beta, rho, mu))
    return {"ms": round(fused, 4), "two_stage_ms": round(two, 4), "speedup": round(two / fused, 3),
            "same_mask": bool(torch.equal(ref_mask, L.mask) and torch.equal(ref_counts, L.counts)),
            "score_tensor_bytes_avoided": int(4 * sum(p.hq * p.nblocks(r) * (p.nblocks(r) + 1)
                                                      for r in range(len(p.lens))))}


def measure_other(name, steps, warmup, dev, torch):
    """ms/layer and effective TFLOP/s of another workload (same step: score, select, attend)."""
    import synth

    p = synth.make_problem(name)
    x = synth.make_inputs(p, seed=0)
    L, q, k, v = setup(p, x, dev)
    ms, stage, bsa_each, _, _ = time_layer_cold(L, q, k, v, p, steps, warmup, torch, dev)
    fl = 4 * p.d * visible_pairs(p, L.mask.cpu().numpy().view(np.uint32), L.NB)
    bsa = float(np.mean(bsa_each))
    peak = PEAK[p.dtype]
    out = {"workload": describe(p), "dtype": p.dtype, "ms_per_layer": round(ms, 4),
           "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "pct_of_peak": round(100 * fl / (ms * 1e-3) / 1e12 / peak, 2),
           "stages_ms": [round(float(t), 4) for t in stage], "bsa_tflops": round(fl / (bsa * 1e-3) / 1e12, 2),
           "peak_tflops": peak}
    if max(p.nblocks(r) for r in range(len(p.lens))) <= 2048:
        out["fused_score_select"] = fused_vs_two_stage(L, q, k, v, p, torch)
    if L.bsa_ws.numel() > 0:
        # fp8: bsa_prefill_ws (V expanded to bf16 once per call, expansion included) against bsa_prefill
        # (V converted on every tile visit), warm, same selection
        t_ws = time_bsa(L, q, k, v, "selected", 3, torch)
        t_pv = time_bsa(L, q, k, v, "selected", 3, torch, expand_v=False)
        out["v_expansion"] = {"bsa_prefill_ws_ms": round(t_ws, 4), "bsa_prefill_per_visit_ms": round(t_pv, 4),
                              "speedup": round(t_pv / t_ws, 3), "workspace_bytes": int(L.bsa_ws.numel())}
    return out


def unpack_bits(p, words, r, NB_off):
    """Request r's selection as bool [hq][n][n] (causal part only) from packed mask words."""
    n = p.nblocks(r)
    w = words[:, NB_off:NB_off + n].astype(np.uint32)
    bits = ((w[..., None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(p.hq, n, -1)[:, :, :n].astype(bool)
    return bits & np.tril(np.ones((n, n), dtype=bool))[None]


def selection_stats(p, words, ref_words):
    """Where a selection puts its blocks, and how much of it a reference selection shares."""
    cb = p.cu_blocks
    inter = union = total = sink = diag = local = 0
    dist = 0.0
    for r in range(len(p.lens)):
        n = p.nblocks(r)
        a = unpack_bits(p, words, r, cb[r])
        b = unpack_bits(p, ref_words, r, cb[r])
        inter += int((a & b).sum())
        union += int((a | b).sum())
        ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
        total += int(a.sum())
        sink += int(a[:, :, 0].sum())
        diag += int(a[:, ii == jj].sum())
        local += int(a[:, (ii - jj < 16)].sum())
        dist += float(((ii - jj)[None] * a).sum())
    return {"jaccard_vs_default": round(inter / max(union, 1), 4), "blocks": total,
            "frac_sink_block": round(sink / total, 4), "frac_diagonal": round(diag / total, 4),
            "frac_within_16_blocks": round(local / total, 4), "mean_block_distance": round(dist / total, 2)}


def measure_ablations(L, q, k, v, p, torch, reps=3):
    """The pages' ablation switches on the same inputs: uniform budget (mu = 1), routing only (beta = 0),
    both, and a small beta/mu sweep.  Reports latency and where the selection goes (model accuracy needs
    weights and is out of reach here)."""
    rho = (p.rho_num, p.rho_den)

    def run(beta, mu):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record()
        for _ in range(reps):
            L.score(q, k, v, beta)
            L.select(rho, mu)
        b.record()
        for _ in range(reps):
            L.attend(q, k, v, "selected", True)
        c.record()
        torch.cuda.synchronize()
        words = L.mask.cpu().numpy().view(np.uint32)
        counts = L.counts.cpu().numpy()
        return a.elapsed_time(b) / reps, b.elapsed_time(c) / reps, words, counts

    sel_ms, bsa_ms, ref, _ = run(p.beta, (p.mu_num, p.mu_den))
    res = {}
    variants = [("default", p.beta, (p.mu_num, p.mu_den)), ("uniform_mu1", p.beta, (1, 1)),
                ("routing_only_beta0", 0.0, (p.mu_num, p.mu_den)), ("uniform_and_beta0", 0.0, (1, 1))]
    variants += [(f"beta{b}_mu{m[0]}/{m[1]}", b, m) for b in (0.1, 0.4, 0.8) for m in ((1, 2), (7, 10))]
    n_last = p.nblocks(len(p.lens) - 1)
    for name, beta, mu in variants:
        sel_ms, bsa_ms, words, counts = run(beta, mu)
        fl = 4 * p.d * visible_pairs(p, words, L.NB)
        last = counts[0, p.cu_blocks[-2]:p.cu_blocks[-1]]
        res[name] = {"beta": beta, "mu": f"{mu[0]}/{mu[1]}", "score_select_ms": round(sel_ms, 4),
                     "bsa_ms": round(bsa_ms, 3), "bsa_tflops": round(fl / (bsa_ms * 1e-3) / 1e12, 2),
                     "k_first_uncapped_row": int(last[np.argmax(last < np.arange(1, n_last + 1))]),
                     "k_last_row": int(last[-1]), **selection_stats(p, words, ref)}
    L.score(q, k, v, p.beta)
    L.select(rho, (p.mu_num, p.mu_den))
    torch.cuda.synchronize()
    return res


def measure_naive(L, q, k, v, p, dev, torch, score_ms, fused_ms, samples=4):
    """The naive token-level scoring (sampled queries, softmax, block mass; every step through HBM) on the
    same inputs: its time, its intermediate bytes, and how its selection compares with the pooled one."""
    from block_sparse_attention_oam_amd import _abi

    rho, mu = (p.rho_num, p.rho_den), (p.mu_num, p.mu_den)
    ref = L.mask.cpu().numpy().view(np.uint32).copy()
    nbytes = _abi.naive_workspace_bytes(L.p, samples)
    try:
        nws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    except RuntimeError as e:  # pragma: no cover - memory
        return {"skipped": f"could not allocate {nbytes} bytes: {e}"}
    _abi.stem_naive_score(L.p, q, k, v, p.beta, samples, L.scores, L.ws, nws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(2):
        _abi.stem_naive_score(L.p, q, k, v, p.beta, samples, L.scores, L.ws, nws)
    b.record()
    torch.cuda.synchronize()
    naive_ms = a.elapsed_time(b) / 2
    L.select(rho, mu)
    torch.cuda.synchronize()
    stats = selection_stats(p, L.mask.cpu().numpy().view(np.uint32), ref)
    del nws
    torch.cuda.empty_cache()
    L.score(q, k, v, p.beta)
    L.select(rho, mu)
    torch.cuda.synchronize()
    return {"samples_per_block": samples, "ms": round(naive_ms, 3), "intermediate_bytes": int(nbytes),
            "pooled_score_ms": round(score_ms, 4), "speedup_of_pooled_scoring": round(naive_ms / score_ms, 1),
            "speedup_of_fused_score_select": round(naive_ms / fused_ms, 1),
            "jaccard_with_pooled_selection": stats["jaccard_vs_default"]}


def measure_quantize(dev, torch, reps):
    """The 128K fp8 layer's stage 1 from bf16 activations: stem_quantize_score (amax, quantise + pool,
    score) against stem_score on already-quantised inputs, and the bytes each moves."""
    import synth
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    pb = synth.make_problem("w8a8_128k_fp8", dtype="bf16")
    xb = synth.make_inputs(pb, seed=0)
    q, k, v = upload(xb["q"]), upload(xb["k"]), upload(xb["v"])
    q8, k8, v8 = (torch.empty(t.shape, dtype=torch.uint8, device=dev) for t in (q, k, v))
    qs = torch.empty(pb.hq, dtype=torch.float32, device=dev)
    ks = torch.empty(pb.hkv, dtype=torch.float32, device=dev)
    vs = torch.empty(pb.hkv, dtype=torch.float32, device=dev)
    prob = stem.make_problem(pb.cu_seqlens, pb.hq, pb.hkv, pb.d, pb.block, "fp8", q_scale=qs, k_scale=ks, v_scale=vs)
    L = StemPrefill(prob, dev)

    def run(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_fused = run(lambda: stem.stem_quantize_score(prob, q, k, v, q8, k8, v8, qs, ks, vs, pb.beta, L.scores, L.ws))
    t_score = run(lambda: L.score(q8, k8, v8, pb.beta))
    t_quant = run(lambda: stem.stem_quantize_fp8(prob, q, k, v, q8, k8, v8, qs, ks, vs))

    def unfused():
        stem.stem_quantize_fp8(prob, q, k, v, q8, k8, v8, qs, ks, vs)
        L.score(q8, k8, v8, pb.beta)

    t_unfused = run(unfused)
    bf16_bytes = int(sum(t.numel() * 2 for t in (q, k, v)))
    return {"workload": "w8a8_128k_fp8 from bf16 activations", "quantize_score_ms": round(t_fused, 4),
            "unfused_quantize_then_score_ms": round(t_unfused, 4), "quantize_only_ms": round(t_quant, 4),
            "score_on_fp8_ms": round(t_score, 4), "fusion_speedup": round(t_unfused / t_fused, 3),
            "bf16_bytes_read_twice": bf16_bytes, "fp8_bytes_written": bf16_bytes // 2,
            "note": "unfused: stem_quantize_fp8 (amax pass, then codes) followed by stem_score on the codes"}


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and logical CPU count."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline(p, x, tokens=65536):
    """The oracle's whole pipeline, as it stands, on a bounded sample of the same workload: the first
    `tokens` tokens of request 0 (a request of its own, causal from its first token), KV group 0 and its
    query heads.  Each stage is timed by wall clock: decode (bf16/fp8 bytes to float64) and pooling, block
    scores, TPD budgets and selection, block-sparse attention.  Returns (TFLOP/s, threads, description,
    per-stage seconds); the flop count is 4·d per visible selected pair of the sample's own mask."""
    import oracle
    from tests import stem_cases as sc

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    a, b = sc.request_slices(p)[0]
    T = min(tokens, b - a)
    grp = p.hq // p.hkv
    heads = list(range(grp))  # the query heads of KV group 0
    st = {}
    t = time.perf_counter()
    q = sc.decode_q(p, x, a, a + T, heads)
    k = sc.decode_kv(p, x, 0, "k", [0])[:T]
    v = sc.decode_kv(p, x, 0, "v", [0])[:T]
    qbar = oracle.pool_blocks(q, p.block)
    kbar = oracle.pool_blocks(k, p.block)
    M = oracle.value_log_magnitude(v, p.block)
    st["decode_pool"] = time.perf_counter() - t
    t = time.perf_counter()
    S = oracle.oam_block_scores(qbar, kbar, M, p.beta)
    st["score"] = time.perf_counter() - t
    t = time.perf_counter()
    n = qbar.shape[1]
    budgets = oracle.tpd_budgets(n, p.rho_num, p.rho_den, p.mu_num, p.mu_den)
    mask = oracle.select_all(S, budgets)
    st["budget_select"] = time.perf_counter() - t
    t = time.perf_counter()
    oracle.block_sparse_attention(q, k, v, mask, p.block)
    st["attention"] = time.perf_counter() - t
    # visible selected pairs: full blocks below the diagonal, the causal triangle on it (ragged last block)
    sizes = np.array([min(p.block, T - j * p.block) for j in range(n)], dtype=np.int64)
    vis = 0
    for h in range(len(heads)):
        for i in range(n):
            sel = np.nonzero(mask[h, i, : i + 1])[0]
            vis += int(sizes[i] * sizes[sel[sel < i]].sum())
            if mask[h, i, i]:
                vis += int(sizes[i] * (sizes[i] + 1) // 2)
    dt = sum(st.values())
    desc = (f"the oracle's pipeline on the first {T} tokens of request 0, KV group 0 and its {len(heads)} query "
            f"heads ({n} blocks, {dt:.1f} s)")
    return 4 * p.d * vis / dt / 1e12, threads, desc, {k_: round(v_, 3) for k_, v_ in st.items()}


def traffic_from_profile(src_sha, kernel_src="bsa_bf16.hip"):
    """HBM bytes per BSA launch from the committed PMC summary, if it was taken on the current kernel."""
    name = {"bsa_bf16.hip": "bsa_traffic.json", "bsa_fp8.hip": "bsa_fp8_traffic.json"}.get(kernel_src)
    if name is None:
        return None
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_source_sha256") != src_sha:
        return None
    return d.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_128k_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense run, the density sweep and the other workloads")
    ap.add_argument("--no-other-workloads", action="store_true", help="skip the 32K / fp8 / paged / fp32 lines")
    ap.add_argument("--no-ablations", action="store_true", help="skip the mu = 1 / beta = 0 ablation switches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the library has no multi-GPU path; "
              f"each GPU's share would be this single-GPU kernel on its KV-head group.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    p = synth.make_problem(args.workload)
    log(f"[bench] generating {describe(p)}")
    x = synth.make_inputs(p, seed=0)
    L, q, k, v = setup(p, x, dev)
    log("[bench] timing the layer (cold: 1 GiB overwritten before each step)")
    ms_step, stage_ms, bsa_each, layer_each, wall_step = time_layer_cold(L, q, k, v, p, args.steps, args.warmup,
                                                                         torch, dev)
    log("[bench] warm steps (no eviction)")
    _, warm_stage, _ = time_layer(L, q, k, v, p, args.steps, 1, torch)
    warm_ms = float(np.sum(warm_stage))
    words = L.mask.cpu().numpy().view(np.uint32)
    pairs = visible_pairs(p, words, L.NB)
    flops = 4 * p.d * pairs
    tflops = flops / (ms_step * 1e-3) / 1e12
    bsa_ms = float(np.mean(bsa_each))
    bsa_tflops = flops / (bsa_ms * 1e-3) / 1e12
    peak = PEAK[p.dtype]
    density = pairs / dense_pairs(p)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded; Llama-3-8B-shaped layer, no weights or datasets)",
        "config": {"workload": describe(p), "tokens": p.tokens, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "timing": ("ms_per_step = median over the timed steps of the layer's HIP-event time, each step after "
                   "a 1 GiB buffer was overwritten (cold L2 and MALL); warm = the same steps back to back"),
        "ms_per_step_p10_p90": [round(float(np.percentile(layer_each, 10)), 4),
                                round(float(np.percentile(layer_each, 90)), 4)],
        "wall_ms_per_step_with_eviction": round(wall_step, 4),
        "warm": {"ms_per_step": round(warm_ms, 4), "tflops": round(flops / (warm_ms * 1e-3) / 1e12, 2),
                 "stages_ms": [round(float(t), 4) for t in warm_stage]},
        "stages_ms": {"stem_score": round(float(stage_ms[0]), 4), "stem_tpd_topk": round(float(stage_ms[1]), 4),
                      "bsa_prefill": round(float(stage_ms[2]), 4)},
        "selected_density": round(density, 5),
        "effective_flop_per_layer": flops,
    }
    sb, selb = stage_bytes(p)
    out["scoring_hbm"] = {"algorithmic_bytes": sb, "gbps": round(sb / (stage_ms[0] * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(sb / (stage_ms[0] * 1e-3) / 8e12, 4)}
    out["selection_hbm"] = {"algorithmic_bytes": selb, "gbps": round(selb / (stage_ms[1] * 1e-3) / 1e9, 1),
                            "frac_of_8TBps": round(selb / (stage_ms[1] * 1e-3) / 8e12, 4)}
    # Roofline of the dominant kernel (block-sparse attention): effective flops / average launch time.
    kernel_src = {"bf16": "bsa_bf16.hip", "fp8": "bsa_fp8.hip"}.get(p.dtype, "bsa_fwd.hip")
    src = open(os.path.join(ROOT, "block_sparse_attention_oam_amd", "csrc", kernel_src), "rb").read()
    sha = hashlib.sha256(src).hexdigest()
    out["roofline"] = {"kernel": kernel_src.replace(".hip", "_kernel"), "bound": "mfma", "achieved": round(bsa_tflops, 2), "peak": peak,
                       "unit": "TFLOP/s", "frac": round(bsa_tflops / peak, 4),
                       "traffic": traffic_from_profile(sha, kernel_src), "avg_launch_ms": round(bsa_ms, 4)}
    if not args.no_extras:
        log("[bench] fused scoring + selection")
        out["fused_score_select"] = fused_vs_two_stage(L, q, k, v, p, torch)
        fused_ms = out["fused_score_select"]["ms"]
        if p.dtype == "bf16" and not p.paged:
            log("[bench] naive token-level scoring (comparison path)")
            out["naive_scoring"] = measure_naive(L, q, k, v, p, dev, torch, float(stage_ms[0]), fused_ms)
        log("[bench] dense-causal run of the same kernel")
        dense_ms = time_bsa(L, q, k, v, None, 3, torch)
        dflops = 4 * p.d * dense_pairs(p)
        out["dense"] = {"bsa_ms": round(dense_ms, 3), "tflops": round(dflops / (dense_ms * 1e-3) / 1e12, 2),
                        "sparse_over_dense_latency": round(bsa_ms / dense_ms, 4)}
        log("[bench] density sweep")
        sweep = {}
        for rn in (10, 25, 50, 100):
            L.select((rn, 100), (p.mu_num, p.mu_den))
            torch.cuda.synchronize()
            w2 = L.mask.cpu().numpy().view(np.uint32)
            f2 = 4 * p.d * visible_pairs(p, w2, L.NB)
            t2 = time_bsa(L, q, k, v, L.mask, 3, torch)
            sweep[f"{rn}%"] = {"bsa_ms": round(t2, 3), "tflops": round(f2 / (t2 * 1e-3) / 1e12, 2),
                               "density": round(f2 / (4 * p.d * dense_pairs(p)), 4)}
            if p.dtype == "bf16" and p.d == 128 and p.block == 128 and not p.paged:
                # the same mask through the variant that tests each block's bit inside the loop
                t3 = time_bsa(L, q, k, v, L.mask, 3, torch, inloop=True)
                sweep[f"{rn}%"]["inloop_skip_ms"] = round(t3, 3)
                sweep[f"{rn}%"]["list_speedup_over_inloop"] = round(t3 / t2, 4)
        out["density_sweep"] = sweep
        L.select((p.rho_num, p.rho_den), (p.mu_num, p.mu_den))
        if not args.no_ablations:
            log("[bench] ablation switches (mu = 1, beta = 0, beta/mu sweep)")
            out["ablations"] = measure_ablations(L, q, k, v, p, torch)
        if args.workload == "llama_128k_bf16" and not args.no_other_workloads:
            log("[bench] W8A8 stage 1 from bf16 activations (quantisation fused with pooling)")
            out["w8a8_quantize_score"] = measure_quantize(dev, torch, args.steps)
            torch.cuda.empty_cache()
            others = {}
            for name in ("llama_32k_bf16", "w8a8_128k_fp8", "paged_ragged_bf16", "tiny_f32"):
                log(f"[bench] other workload {name}")
                others[name] = measure_other(name, args.steps, args.warmup, dev, torch)
                torch.cuda.empty_cache()
            out["other_workloads"] = others
    if args.copy_calibration:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(buf)
        dst.copy_(buf)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle on a bounded sample")
        v_cpu, threads, desc, stages = cpu_baseline(p, x)
        out["cpu_baseline"] = {"value": round(v_cpu, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                               "sample": desc, "stages_s": stages, "host": host_cpu()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
