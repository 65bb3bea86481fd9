"""CPU oracle of the Stem sparse-attention prefill path: plain definitions in float64 / exact rationals.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  It shares no code with the HIP library and imports nothing from it.

Sources: the web pages on Tencent Hunyuan's Stem algorithm.  The technical one is "从Stem稀疏注意力看
大模型推理的架构取舍" (developer.cloud.tencent.cn/article/2709440), cited below as [Arch] with its section
titles; the news explainer "腾讯混元 Stem 算法入选 ICML-26" (openai-hub.com/news/599) is [News].

Readings of points the pages leave open (each one is listed, with its reason, in the design notes):
  R1  routing term = attention logit <q, k>/sqrt(d); magnitude term uses the natural log.
  R2  the compact block representation of Q (and of K) is the mean over all valid tokens of the block.
  R3  the block form of log||V_j||_2 is the mean over the block's tokens of ln||v_t||_2.
  R4  no block is forced into the selection (no diagonal or sink rule): selection is plain top-k.
  R5  GQA: scores and selection are per query head; k-bar and M are shared by the heads of a KV group
      (query head h uses KV head h // (Hq/Hkv)).
  R6  TPD runs along the query-block index i, with weights w_i = 1 - (1-mu) i/(n-1).
  R7  TPD total T = round-half-up(rho * n(n+1)/2), clamped to [n, n(n+1)/2]; per-row value
      r_i(x) = min(max(x w_i, 1), i+1) with x solving sum_i r_i(x) = T; integer budgets by rounding the
      prefix sums (k_i = K_i - K_{i-1}, K_i = floor(P_i + 1/2)).
  R8  ties in selection go to the lower block index.
  R9  softmax scale 1/sqrt(d); causal rule key position <= query position inside a request.
  R12 a query row with no visible key has output 0 and LSE = -inf.
  R15 the naive comparison form of the metric samples `samples` queries per block at offsets
      s * (B / samples) (clamped to the request's last token), takes each one's softmax over its visible
      keys, sums the probability mass per key block, averages over the block's samples, and scores
      ln(mean mass) + beta * M[g][j].

Parity pins (tests under `tests/`, marked "not gpu"): every function below is pinned by something other
than itself -- brute-force token-level scores, an independent floating-point bisection of the TPD solve,
a brute-force selection by Python sorting, textbook dense causal attention via torch's CPU SDPA routine at
a 100% budget and with an additive -inf mask, the e4m3fn / bf16 decodes against torch's casts, the fp8
dequantisation against hand-built codes under distinct per-head scales and against torch's decode times
the scale, and the paged gather against the contiguous layout.  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_to_f64", "e4m3fn_table", "fp8_to_f64", "decode", "gather_paged",
    "pool_blocks", "value_log_magnitude", "oam_block_scores", "oam_token_scores",
    "tpd_total", "tpd_solve", "tpd_budgets", "select_row", "select_all",
    "attention_rows", "block_sparse_attention", "dense_causal_attention", "causal_pairs",
    "sampled_query_positions", "naive_block_scores", "e4m3fn_encode", "quantize_fp8_per_head",
]


# ----------------------------------------------------------------------------------------------------
# Input decoding (storage formats -> float64)
# ----------------------------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64: a bf16 value is the fp32 value whose upper 16 bits are `bits`."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def e4m3fn_table() -> np.ndarray:
    """The 256 values of OCP fp8 e4m3fn, from the format's definition.

    Bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.  Exponent 0: subnormal m/8 * 2^-6.
    Exponent 15 with mantissa 7 is NaN (there is no infinity); everything else is (1 + m/8) * 2^(e-7).
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 15 and m == 7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3fn_table()


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Real values (|y| <= 448) -> OCP e4m3fn codes, rounding to the nearest representable value, ties to
    the even code.  Picks, for each value, the nearest entry of the definition table (positive codes
    0x00..0x7E), preferring the even code on a tie."""
    y = np.asarray(y, dtype=np.float64)
    tab = e4m3fn_table()[:0x7F]  # non-negative finite values, increasing with the code
    a = np.abs(y)
    idx = np.searchsorted(tab, a)  # first code with value >= a
    idx = np.clip(idx, 1, 0x7E)
    lo, hi = tab[idx - 1], tab[idx]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (idx % 2 == 0))
    code = np.where(a >= tab[0x7E], 0x7E, np.where(a <= 0, 0, np.where(pick_hi, idx, idx - 1)))
    return (code.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << np.uint8(7))).astype(np.uint8)


def quantize_fp8_per_head(x: np.ndarray, rows=None):
    """W8A8 quantisation of one tensor x [T][H][d] (values exactly representable in fp32), reading R10:
    scale_h = fp32(amax_h / 448) (1 when amax_h = 0), y = fp32(x / scale_h) clamped to +-448, code =
    e4m3fn round-to-nearest-even of y.  Returns (codes uint8 [T][H][d], scale float32 [H]); with `rows`
    (token indices) the scales still come from all of x but only those rows are encoded ([len][H][d])."""
    x = np.asarray(x)
    H = x.shape[1]
    sel = x if rows is None else x[rows]
    codes = np.empty(sel.shape, dtype=np.uint8)
    scale = np.empty(H, dtype=np.float32)
    for h in range(H):
        amax = np.float32(np.abs(x[:, h]).max())
        s = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
        scale[h] = s
        y = (sel[:, h].astype(np.float32) / s).astype(np.float32).astype(np.float64)
        codes[:, h] = e4m3fn_encode(np.clip(y, -448.0, 448.0))
    return codes, scale


def fp8_to_f64(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """e4m3fn codes [..., H, d] times the per-head scale [H] (W8A8 dequantisation)."""
    vals = _E4M3[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scale, dtype=np.float64)[:, None]


def decode(raw: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Stored tensor [..., H, d] -> float64 ('f32' float32, 'bf16' uint16 bits, 'fp8' uint8 codes)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype == "fp8":
        return fp8_to_f64(raw, scale)
    raise ValueError(dtype)


def gather_paged(pages: np.ndarray, table_row: np.ndarray, L: int) -> np.ndarray:
    """Rebuild one request's contiguous KV [L][H][d] from pages [P][page_size][H][d] and its page table row.

    Logical token t lives in physical page table_row[t // page_size] at slot t % page_size ([Arch]
    "HPC-BSA": the operator reads a vLLM-style paged KV cache of fixed-size pages).
    """
    ps = pages.shape[1]
    out = np.empty((L,) + pages.shape[2:], dtype=pages.dtype)
    for t0 in range(0, L, ps):
        t1 = min(t0 + ps, L)
        out[t0:t1] = pages[int(table_row[t0 // ps]), : t1 - t0]
    return out


# ----------------------------------------------------------------------------------------------------
# Stage 1: Output-Aware Metric block scores  ([Arch] "OAM：价值评估" and "HPC-Stem：评估选块，快几十倍")
# ----------------------------------------------------------------------------------------------------
def _blocks(L: int, B: int):
    return [(a, min(a + B, L)) for a in range(0, L, B)]


def pool_blocks(x: np.ndarray, B: int) -> np.ndarray:
    """Compact block representation (reading R2): x [L][H][d] -> mean over each block's tokens, [H][n][d].

    [Arch] "HPC-Stem": because the OAM score is purely additive, the token-level product over sampled Q/K
    can be replaced by per-block compact representations of Q and K and one GEMM.
    """
    L = x.shape[0]
    if L == 0:  # a request with no tokens has no blocks
        return np.zeros((x.shape[1], 0, x.shape[2]))
    out = np.stack([x[a:b].mean(axis=0) for a, b in _blocks(L, B)], axis=1)  # [H][n][d]
    return out


def value_log_magnitude(v: np.ndarray, B: int) -> np.ndarray:
    """Block value-magnitude term (reading R3): M[g][j] = mean over t in block j of ln ||v_{g,t}||_2.

    [Arch] "OAM": the score adds the signal magnitude log||V_j||_2 to the routing relevance.
    """
    L = v.shape[0]
    if L == 0:
        return np.zeros((v.shape[1], 0))
    lognorm = np.log(np.sqrt(np.sum(v * v, axis=-1)))  # [L][H]
    return np.stack([lognorm[a:b].mean(axis=0) for a, b in _blocks(L, B)], axis=1)  # [H][n]


def oam_block_scores(qbar: np.ndarray, kbar: np.ndarray, M: np.ndarray, beta: float) -> np.ndarray:
    """S[h][i][j] = <qbar_{h,i}, kbar_{g,j}>/sqrt(d) + beta * M[g][j] for j <= i; NaN above the diagonal.

    [Arch] "OAM": score = routing relevance (QK^T) + beta * log||V_j||_2, beta = 0.2 on the pages;
    [Arch] "HPC-Stem": all block scores come from one GEMM of the compact representations.
    """
    hq, n, d = qbar.shape
    hkv = kbar.shape[0]
    grp = hq // hkv
    S = np.full((hq, n, n), np.nan)
    tri = np.tril(np.ones((n, n), dtype=bool))
    for h in range(hq):
        g = h // grp
        full = qbar[h] @ kbar[g].T / math.sqrt(d) + beta * M[g][None, :]
        S[h][tri] = full[tri]
    return S


def oam_token_scores(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: float) -> np.ndarray:
    """Token-level OAM score s[h][a][b] = <q_{h,a}, k_{g,b}>/sqrt(d) + beta ln||v_{g,b}||_2, all (a, b).

    Used to pin `oam_block_scores`: the block score equals the mean of s over the block pair (a in I_i,
    b in I_j), the equivalence [Arch] "HPC-Stem" relies on.
    """
    L, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    s = np.empty((hq, L, L))
    for h in range(hq):
        g = h // grp
        for a in range(L):
            for b in range(L):
                s[h, a, b] = float(np.dot(q[a, h], k[b, g])) / math.sqrt(d) + beta * math.log(
                    math.sqrt(float(np.dot(v[b, g], v[b, g]))))
    return s


# ----------------------------------------------------------------------------------------------------
# Stage 2: Token Position Decay budgets  ([Arch] "TPD：优先级排序")
# ----------------------------------------------------------------------------------------------------
def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def tpd_total(n: int, rho_num: int, rho_den: int) -> int:
    """T = round-half-up(rho * C) with C = n(n+1)/2 causal block pairs, clamped to [n, C] (reading R7)."""
    C = causal_pairs(n)
    T = math.floor(Fraction(rho_num, rho_den) * C + Fraction(1, 2))
    return max(n, min(C, T))


def tpd_solve(n: int, T: int, mu: Fraction):
    """Solve sum_i r_i(x) = T exactly.  Returns (x*, [r_i]) as Fractions.

    [Arch] "TPD": the per-position budget decays linearly from k_start at the start to k_end = mu k_start
    at the end, and the total stays that of the uniform allocation (it is redistributed, not increased).
    With w_i = 1 - (1-mu) i/(n-1), row i gets r_i(x) = min(max(x w_i, 1), i+1): at least one block and
    at most the i+1 causal blocks; x = k_start is chosen so the rows add up to T.  F(x) = sum_i r_i(x) is
    continuous, piecewise linear and nondecreasing, so x* is found between two adjacent breakpoints.
    """
    if not (0 < mu <= 1):
        raise ValueError("mu must lie in (0, 1]: with mu = 0 the last row could never reach its share")
    if n == 1:
        return Fraction(1), [Fraction(1)]
    w = [1 - (1 - mu) * Fraction(i, n - 1) for i in range(n)]

    def r(i, x):
        return min(max(x * w[i], Fraction(1)), Fraction(i + 1))

    def F(x):
        return sum(r(i, x) for i in range(n))

    bps = set()
    for i in range(n):
        bps.add(1 / w[i])
        bps.add((i + 1) / w[i])
    bps = sorted(bps)
    # F(0) = n (every row floored at 1); F is flat on [0, bps[0]].
    lo, hi = 0, len(bps) - 1
    if F(bps[0]) >= T:
        x = bps[0]
    elif F(bps[-1]) <= T:
        x = bps[-1]
    else:
        # invariant: F(bps[lo]) < T < F(bps[hi])
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if F(bps[mid]) <= T:
                lo = mid
            else:
                hi = mid
        xa, xb = bps[lo], bps[hi]
        Fa, Fb = F(xa), F(xb)
        x = xa + (T - Fa) * (xb - xa) / (Fb - Fa)
    rs = [r(i, x) for i in range(n)]
    assert sum(rs) == T, (n, T, mu)
    return x, rs


def tpd_budgets(n: int, rho_num: int, rho_den: int, mu_num: int, mu_den: int) -> np.ndarray:
    """Integer per-row budgets k_i (reading R7): k_i = K_i - K_{i-1}, K_i = floor(P_i + 1/2), P_i = sum r.

    Rounding the prefix sums keeps sum_i k_i = T exactly and |k_i - r_i| < 1.  A request with no tokens has
    no rows (empty result).
    """
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    T = tpd_total(n, rho_num, rho_den)
    _, rs = tpd_solve(n, T, Fraction(mu_num, mu_den))
    k = np.empty(n, dtype=np.int64)
    P = Fraction(0)
    Kprev = 0
    for i in range(n):
        P += rs[i]
        K = math.floor(P + Fraction(1, 2))
        k[i] = K - Kprev
        Kprev = K
    return k


# ----------------------------------------------------------------------------------------------------
# Stage 2b: top-k selection  ([Arch] "HPC-Stem": budget generation and selection)
# ----------------------------------------------------------------------------------------------------
def select_row(scores_row: np.ndarray, k: int) -> np.ndarray:
    """The k blocks with the largest scores among j = 0..len-1, ties to the lower j (reading R8)."""
    j = np.arange(len(scores_row))
    order = np.lexsort((j, -np.asarray(scores_row, dtype=np.float64)))
    return np.sort(order[:k])


def select_all(S: np.ndarray, budgets: np.ndarray) -> np.ndarray:
    """Boolean block mask [Hq][n][n]: row (h, i) selects budgets[i] blocks among j <= i."""
    hq, n, _ = S.shape
    mask = np.zeros((hq, n, n), dtype=bool)
    for h in range(hq):
        for i in range(n):
            mask[h, i, select_row(S[h, i, : i + 1], int(budgets[i]))] = True
    return mask


# ----------------------------------------------------------------------------------------------------
# Stage 3: block-sparse attention  ([Arch] "HPC-BSA：跳块零开销的秘密")
# ----------------------------------------------------------------------------------------------------
def attention_rows(q_rows: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                   key_idx: np.ndarray, scale: float):
    """Softmax attention of queries q_rows [m][d] at positions q_pos over keys key_idx (ascending).

    A key is visible to a query when it is in key_idx and its position is <= the query's (reading R9).
    Returns (out [m][d], lse [m]); rows with no visible key give 0 and -inf (reading R12).
    """
    kk = k[key_idx]
    vv = v[key_idx]
    logits = (q_rows @ kk.T) * scale
    logits = np.where(key_idx[None, :] <= q_pos[:, None], logits, -np.inf)
    m = logits.max(axis=1, initial=-np.inf)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(logits - safe_m[:, None])
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, (p @ vv) / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, safe_m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, B: int,
                           scale: float | None = None, rows=None):
    """Block-sparse causal attention of one request.

    q [L][Hq][d], k/v [L][Hkv][d] float64; mask [Hq][n][n] bool (only j <= i is read).  For query block i
    of head h, keys are the tokens of the selected blocks; an unselected block contributes as if all its
    scores were -inf ([Arch] "HPC-BSA").  `rows` optionally restricts the work to (h, i) pairs; the other
    outputs stay NaN.  Returns (O [L][Hq][d], LSE [Hq][L]).
    """
    L, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = -(-L // B)
    O = np.full((L, hq, d), np.nan)
    lse = np.full((hq, L), np.nan)
    todo = rows if rows is not None else [(h, i) for h in range(hq) for i in range(n)]
    for h, i in todo:
        g = h // grp
        a, b = i * B, min((i + 1) * B, L)
        sel = np.nonzero(mask[h, i, : i + 1])[0]
        key_idx = np.concatenate([np.arange(j * B, min((j + 1) * B, L)) for j in sel]) if len(sel) else \
            np.zeros(0, dtype=np.int64)
        o, ls = attention_rows(q[a:b, h], np.arange(a, b), k[:, g], v[:, g], key_idx, scale)
        O[a:b, h] = o
        lse[h, a:b] = ls
    return O, lse


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None):
    """Textbook causal softmax attention of one request in float64 (the 100%-budget special case)."""
    L, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.empty((L, hq, d))
    lse = np.empty((hq, L))
    causal = np.tril(np.ones((L, L), dtype=bool))
    for h in range(hq):
        g = h // grp
        s = np.where(causal, (q[:, h] @ k[:, g].T) * scale, -np.inf)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        O[:, h] = (p @ v[:, g]) / l[:, None]
        lse[h] = m + np.log(l)
    return O, lse


# ----------------------------------------------------------------------------------------------------
# Comparison path: the naive, token-level form of the metric  ([Arch] "HPC-Stem：评估选块，快几十倍", which
# contrasts the one-GEMM scoring with computing attention probabilities token by token and gathering them
# into blocks)
# ----------------------------------------------------------------------------------------------------
def sampled_query_positions(L: int, B: int, samples: int) -> np.ndarray:
    """Reading R15: [n][samples] token positions, block i's sample s at i*B + s*(B/samples), clamped to
    L - 1 (a partial last block repeats its last token)."""
    n = -(-L // B)
    step = B // samples
    return np.array([[min(i * B + s * step, L - 1) for s in range(samples)] for i in range(n)], dtype=np.int64)


def naive_block_scores(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int, beta: float, samples: int,
                       scale: float | None = None, rows=None) -> np.ndarray:
    """Naive block scores of one request (reading R15).

    For block i and head h, each sampled query t takes the softmax of q_t . k_tau * scale over the keys
    tau <= t (KV head g = h // (Hq/Hkv)); the probability mass falling in key block j is summed, averaged
    over the block's samples, and S[h][i][j] = ln(mean mass) + beta * M[g][j] for j <= i (NaN above the
    diagonal).  q [L][Hq][d], k/v [L][Hkv][d] float64.  `rows` optionally restricts the work to (h, i)
    pairs; the other rows stay NaN.
    """
    L, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = -(-L // B)
    M = value_log_magnitude(v, B)
    pos = sampled_query_positions(L, B, samples)
    S = np.full((hq, n, n), np.nan)
    todo = rows if rows is not None else [(h, i) for h in range(hq) for i in range(n)]
    for h, i in todo:
        g = h // grp
        mass = np.zeros(n)
        for t in pos[i]:
            logits = (k[: t + 1, g] @ q[t, h]) * scale
            p = np.exp(logits - logits.max())
            p /= p.sum()
            for j in range(i + 1):
                mass[j] += p[j * B: min((j + 1) * B, t + 1)].sum()
        mass /= samples
        with np.errstate(divide="ignore"):
            S[h, i, : i + 1] = np.log(mass[: i + 1]) + beta * M[g, : i + 1]
    return S
