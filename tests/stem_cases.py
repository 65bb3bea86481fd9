"""Shared glue for the parity tests and the benchmark: oracle-side stage results per request and the
comparisons to the GPU results.  Imports the oracle (test infrastructure) and the seeded inputs; the GPU
side goes only through the library's C ABI."""
from __future__ import annotations

import numpy as np

import oracle

# Tolerances stated for BSA outputs given the oracle's mask (bf16 and fp8), and the one derived for the
# fp32 case (fp32 MFMA products and accumulation, exp2 of the scaled logits, fp32 P and V: a few units of
# 2^-24 relative per term; 1e-4 max / 1e-5 mean keeps a wide margin on outputs of magnitude ~1).
TOL = {"bf16": (2e-2, 2e-3), "fp8": (6e-2, 6e-3), "f32": (1e-4, 1e-5)}
TIE_REL = 1e-5  # near-tie window for selection
# LSE bound, derived: the attention kernels round each P to bf16 (relative error <= 2^-9) and their row
# sums add those rounded values, so the sum moves by at most 2^-9 relative and the LSE by at most
# ln(1 + 2^-9) ~ 1.95e-3 (fp32 accumulation adds ~1e-6; the fp32 kernel keeps P in fp32).  1e-2 leaves a
# factor of 5 and still fails an LSE that is off by a visible amount.
LSE_TOL = 1e-2


def request_slices(p):
    cu = p.cu_seqlens
    return [(int(cu[r]), int(cu[r + 1])) for r in range(len(p.lens))]


def decode_q(p, x, a, b, heads=None):
    hs = range(p.hq) if heads is None else heads
    out = np.empty((b - a, len(hs), p.d))
    for c, h in enumerate(hs):
        sc = x["q_scale"][h:h + 1] if p.dtype == "fp8" else None
        out[:, c:c + 1] = oracle.decode(x["q"][a:b, h:h + 1], p.dtype, sc)
    return out


def decode_kv(p, x, r, which, heads=None):
    """Request r's K or V as float64 [L][len(heads)][d]; paged inputs go through the oracle's gather."""
    a, b = request_slices(p)[r]
    L = b - a
    if p.paged:
        raw = oracle.gather_paged(x[which + "_pages"], x["page_table"][r], L)
    else:
        raw = x[which][a:b]
    hs = range(p.hkv) if heads is None else heads
    out = np.empty((L, len(hs), p.d))
    for c, g in enumerate(hs):
        sc = x[which + "_scale"][g:g + 1] if p.dtype == "fp8" else None
        out[:, c:c + 1] = oracle.decode(raw[:, g:g + 1], p.dtype, sc)
    return out


def oracle_stage1(p, x):
    """Per request: (qbar [hq][n][d], kbar [hkv][n][d], M [hkv][n], S [hq][n][n])."""
    res = []
    for r, (a, b) in enumerate(request_slices(p)):
        qbar = np.concatenate([oracle.pool_blocks(decode_q(p, x, a, b, [h]), p.block) for h in range(p.hq)])
        kbar = np.concatenate([oracle.pool_blocks(decode_kv(p, x, r, "k", [g]), p.block) for g in range(p.hkv)])
        M = np.concatenate([oracle.value_log_magnitude(decode_kv(p, x, r, "v", [g]), p.block)
                            for g in range(p.hkv)])
        S = oracle.oam_block_scores(qbar, kbar, M, p.beta)
        res.append((qbar, kbar, M, S))
    return res


def oracle_budgets(p):
    return [oracle.tpd_budgets(p.nblocks(r), p.rho_num, p.rho_den, p.mu_num, p.mu_den) for r in range(len(p.lens))]


def oracle_masks(S_list, budgets):
    return [oracle.select_all(S, k) for S, k in zip(S_list, budgets)]


def unpack_mask(words: np.ndarray, n: int) -> np.ndarray:
    """uint32 words [..., W] -> bool [..., n] (bit j of word j/32)."""
    w = words.astype(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,))[..., :n].astype(bool)


def pack_mask(m: np.ndarray, words: int) -> np.ndarray:
    """bool [..., n] -> int32 words [..., words]."""
    n = m.shape[-1]
    pad = np.zeros(m.shape[:-1] + (words * 32,), dtype=np.uint64)
    pad[..., :n] = m
    pad = pad.reshape(m.shape[:-1] + (words, 32))
    w = (pad << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)
    return w.view(np.int32)


def check_selection(p, S_list, budgets, gpu_words, gpu_counts):
    """Bit-exact selection except in near-tie rows.  Returns the number of near-tie rows that differ."""
    cb = p.cu_blocks
    near_tie_rows = 0
    for r, (S, kk) in enumerate(zip(S_list, budgets)):
        n = len(kk)
        words = gpu_words[:, cb[r]:cb[r + 1]]  # [hq][n][W]
        assert np.array_equal(gpu_counts[:, cb[r]:cb[r + 1]], np.broadcast_to(kk, (p.hq, n))), "budgets differ"
        full = unpack_mask(words, words.shape[-1] * 32)
        for h in range(p.hq):
            for i in range(n):
                row = full[h, i]
                assert not row[i + 1:].any(), f"bits past the diagonal set in row ({h}, {i})"
                got = np.nonzero(row[: i + 1])[0]
                ref = oracle.select_row(S[h, i, : i + 1], int(kk[i]))
                if np.array_equal(got, ref):
                    continue
                s = S[h, i, : i + 1]
                order = np.lexsort((np.arange(i + 1), -s))
                k = int(kk[i])
                sk = s[order[k - 1]]
                sk1 = s[order[k]] if k < i + 1 else -np.inf
                win = TIE_REL * max(abs(sk), abs(sk1))
                assert sk - sk1 < win, f"row ({r}, {h}, {i}) differs outside the tie window"
                assert len(got) == k
                diff = np.setxor1d(got, ref)
                assert np.all(np.abs(s[diff] - sk) <= win), f"row ({r}, {h}, {i}): differing blocks off the tie"
                near_tie_rows += 1
    return near_tie_rows


def oracle_attention(p, x, masks, rows_per_req=None):
    """Oracle BSA outputs.  masks: per-request bool [hq][n][n] (None = dense causal).
    rows_per_req: per request a list of (h, i) or None for all.  Returns per request (O, LSE) with NaN
    where not computed."""
    res = []
    for r, (a, b) in enumerate(request_slices(p)):
        n = p.nblocks(r)
        rows = None if rows_per_req is None else rows_per_req[r]
        need_h = sorted({h for h, _ in rows}) if rows is not None else list(range(p.hq))
        q = np.full((b - a, p.hq, p.d), np.nan)
        q[:, need_h] = decode_q(p, x, a, b, need_h)
        k = decode_kv(p, x, r, "k")
        v = decode_kv(p, x, r, "v")
        m = masks[r] if masks is not None else np.ones((p.hq, n, n), dtype=bool)
        res.append(oracle.block_sparse_attention(q, k, v, m, p.block, rows=rows))
    return res


def compare_attention(p, oracle_res, gpu_out, gpu_lse, rows_per_req=None):
    """Max / mean abs error of the GPU output over the compared rows; LSE max abs error."""
    errs, lerrs = [], []
    for r, ((a, b), (O, lse)) in enumerate(zip(request_slices(p), oracle_res)):
        rows = None if rows_per_req is None else rows_per_req[r]
        if rows is None:
            rows = [(h, i) for h in range(p.hq) for i in range(p.nblocks(r))]
        for h, i in rows:
            t0, t1 = i * p.block, min((i + 1) * p.block, b - a)
            ref = O[t0:t1, h]
            got = gpu_out[a + t0:a + t1, h]
            errs.append(np.abs(got - ref).ravel())
            lref = lse[h, t0:t1]
            lgot = gpu_lse[h, a + t0:a + t1]
            fin = np.isfinite(lref)
            assert np.array_equal(fin, np.isfinite(lgot))
            lerrs.append(np.abs(lgot[fin] - lref[fin]))
    e = np.concatenate(errs)
    le = np.concatenate(lerrs) if lerrs else np.zeros(1)
    return float(e.max()), float(e.mean()), float(le.max() if le.size else 0.0)


def sample_rows(p, r, extra, seed=0, mask=None):
    """Rows (h, i) to check at full size: first/middle/last heads at the first, middle and last blocks;
    the rows around the end of the TPD plan's capped prefix (the last rows with k_i = i + 1 and the first
    ones below it); with `mask` (request r's bool [hq][n][n] selection), the rows where the union of two
    consecutive heads' selections crosses 3/4 of the row's causal blocks (the attention kernel changes
    when it issues its tile loads there); then `extra` random rows."""
    n = p.nblocks(r)
    rng = np.random.default_rng(seed + r)
    hs = sorted({0, p.hq // 2, p.hq - 1})
    is_ = {0, 1 % n, n // 3, n // 2, max(n - 2, 0), n - 1}
    k = oracle.tpd_budgets(n, p.rho_num, p.rho_den, p.mu_num, p.mu_den)
    below = np.nonzero(k < np.arange(1, n + 1))[0]
    if below.size:
        c = int(below[0])  # first row whose budget is below its causal block count
        is_ |= {i for i in (c - 2, c - 1, c, c + 1) if 0 <= i < n}
    rows = {(h, i) for h in hs for i in sorted(is_)}
    if mask is not None and p.hq >= 2:
        for h in (0, (p.hq // 2) & ~1):
            union = (mask[h] | mask[h + 1]).sum(axis=1)
            fits = 4 * union <= 3 * (np.arange(n) + 1)
            flips = np.nonzero(fits[1:] != fits[:-1])[0]
            if flips.size:
                f = int(flips[0]) + 1  # first row on the other side of the switch
                rows |= {(hh, i) for hh in (h, h + 1) for i in (f - 1, f) if 0 <= i < n}
    want = len(rows) + extra
    while len(rows) < want:
        rows.add((int(rng.integers(p.hq)), int(rng.integers(n))))
    return sorted(rows)


def effective_flops(p, masks):
    """4 * d * visible query-key pairs, from per-request bool masks (None = dense causal)."""
    total = 0
    for r, L in enumerate(p.lens):
        n = p.nblocks(r)
        B = p.block
        sizes = np.array([min(B, L - j * B) for j in range(n)], dtype=np.int64)
        if masks is None:
            total += p.hq * L * (L + 1) // 2
            continue
        m = masks[r]
        for i in range(n):
            off = m[:, i, :i].astype(np.int64) @ sizes[:i]  # [hq] keys in earlier selected blocks
            diag = m[:, i, i].astype(np.int64) * (sizes[i] * (sizes[i] + 1) // 2)
            total += int((off * sizes[i] + diag).sum())
    return 4 * p.d * total
