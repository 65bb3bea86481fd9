"""Pins of the CPU oracle against things other than itself (no GPU).

Each test ties one oracle function to an independent fact: a library routine (torch's dtype casts and its
CPU scaled-dot-product attention), a brute-force computation written differently, a closed form, or an
invariant of the pages' definitions.  A dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


# ------------------------------------------------------------------------------------------ decoding
def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], tab[~nan])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch_cast():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values only
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_to_f64(bits), ref)


def test_synth_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 10.0 ** rng.uniform(-3, 3, 10000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


def test_synth_fp8_cast_matches_definition_encoder():
    """torch's float8 cast (used by synth for speed) agrees with synth's from-definition RNE encoder."""
    rng = np.random.default_rng(3)
    y = rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.7, 20000)
    y = np.concatenate([y, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 240.0, 232.0]])
    y = np.clip(y.astype(np.float32), -448, 448)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    enc = synth.e4m3fn_encode(y.astype(np.float64))
    assert np.array_equal(enc, ref)
    # and decoding what was encoded gives the nearest representable value
    tab = oracle.e4m3fn_table()
    assert np.all(np.abs(tab[enc] - y) <= np.abs(y) * 2.0 ** -4 + 2.0 ** -10)


def test_gather_paged_equals_contiguous():
    p = synth.make_problem("paged_ragged_bf16", lens=(300, 64, 129), hq=4, hkv=2, d=16)
    x = synth.make_inputs(p)
    cu = p.cu_seqlens
    for r, L in enumerate(p.lens):
        got = oracle.gather_paged(x["k_pages"], x["page_table"][r], L)
        assert np.array_equal(got, x["k"][cu[r]:cu[r + 1]])
        got = oracle.gather_paged(x["v_pages"], x["page_table"][r], L)
        assert np.array_equal(got, x["v"][cu[r]:cu[r + 1]])


# ------------------------------------------------------------------------------------------ scores
def _tiny_qkv(L=11, hq=4, hkv=2, d=8, seed=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d)) * rng.lognormal(0, 0.5, (L, hkv, 1))
    return q, k, v


@pytest.mark.parametrize("L,B,hq,hkv,d", [(11, 4, 4, 2, 8), (16, 4, 2, 2, 5), (9, 3, 8, 1, 4)])
def test_block_scores_equal_block_pair_mean_of_token_scores(L, B, hq, hkv, d):
    """The pooled one-GEMM score equals the mean of token-level OAM scores over the block pair."""
    q, k, v = _tiny_qkv(L, hq, hkv, d)
    beta = 0.2
    S = oracle.oam_block_scores(oracle.pool_blocks(q, B), oracle.pool_blocks(k, B),
                                oracle.value_log_magnitude(v, B), beta)
    s = oracle.oam_token_scores(q, k, v, beta)
    n = -(-L // B)
    for h in range(hq):
        for i in range(n):
            for j in range(n):
                blk = s[h, i * B:min(L, (i + 1) * B), j * B:min(L, (j + 1) * B)]
                if j <= i:
                    assert abs(S[h, i, j] - blk.mean()) < 1e-12
                else:
                    assert np.isnan(S[h, i, j])


def test_block_scores_hand_built():
    """Blocks with constant q and k: routing term is one dot product; beta scales ln of the value norm."""
    B, d = 4, 3
    q = np.zeros((8, 1, d)); k = np.zeros((8, 1, d)); v = np.zeros((8, 1, d))
    q[:4, 0] = [1, 2, 3]; q[4:, 0] = [0, 1, 0]
    k[:4, 0] = [2, 0, 1]; k[4:, 0] = [1, 1, 1]
    v[:4, 0] = [math.e ** 2, 0, 0]  # ||v|| = e^2 -> ln = 2
    v[4:, 0] = [0, 0, math.e ** -1]  # ln = -1
    for beta in (0.0, 0.2, 1.0):
        S = oracle.oam_block_scores(oracle.pool_blocks(q, B), oracle.pool_blocks(k, B),
                                    oracle.value_log_magnitude(v, B), beta)
        assert S[0, 0, 0] == pytest.approx(5 / math.sqrt(3) + 2 * beta, abs=1e-14)
        assert S[0, 1, 0] == pytest.approx(0 / math.sqrt(3) + 2 * beta, abs=1e-14)
        assert S[0, 1, 1] == pytest.approx(1 / math.sqrt(3) - 1 * beta, abs=1e-14)


def test_block_scores_gqa_head_mapping():
    """Query head h reads KV head h // (Hq/Hkv) (consecutive grouping)."""
    B, d, hq, hkv = 2, 2, 4, 2
    q = np.zeros((2, hq, d)); q[:, :, 0] = 1.0
    k = np.zeros((2, hkv, d)); k[:, 0, 0] = 1.0; k[:, 1, 0] = 3.0
    v = np.ones((2, hkv, d))
    S = oracle.oam_block_scores(oracle.pool_blocks(q, B), oracle.pool_blocks(k, B),
                                oracle.value_log_magnitude(v, B), 0.0)
    assert [S[h, 0, 0] * math.sqrt(d) for h in range(hq)] == pytest.approx([1, 1, 3, 3])


# ------------------------------------------------------------------------------------------ budgets
def _float_bisect_x(n, T, mu):
    """Independent float64 solve of sum_i min(max(x w_i, 1), i+1) = T by bisection."""
    w = 1.0 - (1.0 - mu) * np.arange(n) / (n - 1)
    i1 = np.arange(n) + 1.0

    def F(x):
        return np.minimum(np.maximum(x * w, 1.0), i1).sum()

    lo, hi = 0.0, float(n) / mu + n + 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if F(mid) < T:
            lo = mid
        else:
            hi = mid
    x = 0.5 * (lo + hi)
    return x, np.minimum(np.maximum(x * w, 1.0), i1)


def test_tpd_total_closed_forms():
    assert oracle.tpd_total(32, 25, 100) == 132  # 0.25 * 528
    assert oracle.tpd_total(1024, 25, 100) == 131200  # 0.25 * 524800
    assert oracle.tpd_total(1024, 10, 100) == 52480
    assert oracle.tpd_total(3, 1, 4) == 3  # 1.5 rounds to 2, clamped up to n = 3
    assert oracle.tpd_total(5, 1, 3) == 5  # 15/3 = 5
    assert oracle.tpd_total(7, 1, 8) == 7  # 28/8 = 3.5 -> 4, clamped to n
    assert oracle.tpd_total(10, 3, 10) == 17  # 16.5 rounds half up to 17
    assert oracle.tpd_total(4, 1, 1) == 10


@pytest.mark.parametrize("n,rho", [(2, (1, 2)), (7, (1, 4)), (32, (25, 100)), (64, (10, 100)),
                                   (100, (37, 100)), (256, (25, 100)), (33, (90, 100)), (513, (1, 100))])
@pytest.mark.parametrize("mu", [(7, 10), (1, 1), (1, 2), (1, 100), (1, 3)])
def test_tpd_budget_invariants(n, rho, mu):
    T = oracle.tpd_total(n, *rho)
    x, rs = oracle.tpd_solve(n, T, Fraction(*mu))
    k = oracle.tpd_budgets(n, *rho, *mu)
    idx = np.arange(n)
    assert int(k.sum()) == T
    assert np.all(k >= 1) and np.all(k <= idx + 1)
    assert all(abs(int(k[i]) - rs[i]) < 1 for i in range(n))
    # independent float bisection lands on the same per-row values
    if n > 1:
        xf, rf = _float_bisect_x(n, T, mu[0] / mu[1])
        assert np.allclose([float(r) for r in rs], rf, atol=1e-7 * n)
    # rows that are neither capped nor floored follow one line: r_i = x (1 - (1-mu) i/(n-1))
    mu_f = Fraction(*mu)
    for i in range(n):
        if 1 < rs[i] < i + 1:
            assert rs[i] == x * (1 - (1 - mu_f) * Fraction(i, n - 1))
    # the line's end value is mu times its start value (k_end = mu * k_start)
    if n > 1 and 1 < rs[-1] < n:
        assert rs[-1] == mu_f * x


@pytest.mark.parametrize("n,rho,T,k_start,dense_rows", [
    (32, 25, 132, 5.247, 5), (256, 25, 8224, 41.477, 40), (512, 25, 32832, 82.881, 79),
    (1024, 10, 52480, 62.460, 61), (1024, 25, 131200, 165.688, 158), (1024, 50, 262400, 373.538, 337)])
def test_tpd_against_an_independent_exact_computation(n, rho, T, k_start, dense_rows):
    """Totals, line start k_start* (to 3 decimals) and the number of leading rows whose integer budget is
    their whole causal row (k_i = i + 1), from a separate exact computation made when the workloads were
    planned (mu = 7/10); at n = 1024 and 25% the line also ends at k_end* = 115.982."""
    assert oracle.tpd_total(n, rho, 100) == T
    x, rs = oracle.tpd_solve(n, T, Fraction(7, 10))
    assert abs(float(x) - k_start) < 5e-4
    k = oracle.tpd_budgets(n, rho, 100, 7, 10)
    full = k == np.arange(1, n + 1)
    assert int(full.sum()) == dense_rows and bool(full[:dense_rows].all())
    if (n, rho) == (1024, 25):
        assert abs(float(rs[-1]) - 115.982) < 5e-4


def test_tpd_full_budget_is_dense_and_min_budget_is_one_per_row():
    for n in (1, 2, 5, 40):
        assert np.array_equal(oracle.tpd_budgets(n, 1, 1, 7, 10), np.arange(1, n + 1))
        assert np.array_equal(oracle.tpd_budgets(n, 0, 1, 7, 10), np.ones(n, dtype=np.int64))


def test_tpd_rejects_mu_zero():
    with pytest.raises(ValueError):
        oracle.tpd_budgets(8, 1, 2, 0, 1)


def test_tpd_uniform_when_mu_is_one():
    n = 200
    k = oracle.tpd_budgets(n, 25, 100, 1, 1)
    T = oracle.tpd_total(n, 25, 100)
    assert int(k.sum()) == T
    x, rs = oracle.tpd_solve(n, T, Fraction(1))
    unc = [i for i in range(n) if rs[i] < i + 1]
    assert len({rs[i] for i in unc}) == 1  # one common value past the capped head rows
    assert all(int(k[i]) in (math.floor(x), math.ceil(x)) for i in unc)


def test_tpd_decays_linearly_from_start_to_end():
    """n = 1024, 25%: the budget line falls from k_start to 0.7 k_start across the rows."""
    n = 1024
    k = oracle.tpd_budgets(n, 25, 100, 7, 10)
    T = oracle.tpd_total(n, 25, 100)
    x, rs = oracle.tpd_solve(n, T, Fraction(7, 10))
    assert rs[-1] == Fraction(7, 10) * x
    capped = sum(1 for i in range(n) if rs[i] == i + 1)
    assert 100 < capped < 200  # rows whose line value exceeds their i+1 causal blocks
    assert k[-1] < k[capped + 1]
    assert abs(int(k[-1]) - 0.7 * float(x)) < 1


# ------------------------------------------------------------------------------------------ selection
def test_select_row_against_python_sort_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(300):
        m = int(rng.integers(1, 70))
        s = rng.integers(-4, 5, size=m).astype(np.float64) * 0.5  # many exact ties
        if trial % 3 == 0:
            s = rng.standard_normal(m)
        kk = int(rng.integers(1, m + 1))
        brute = sorted(sorted(range(m), key=lambda j: (-s[j], j))[:kk])
        assert list(oracle.select_row(s, kk)) == brute


def test_select_all_equal_scores_takes_lowest_indices():
    S = np.zeros((1, 6, 6))
    mask = oracle.select_all(S, np.array([1, 1, 2, 2, 3, 3]))
    assert [list(np.nonzero(mask[0, i])[0]) for i in range(6)] == [[0], [0], [0, 1], [0, 1], [0, 1, 2],
                                                                   [0, 1, 2]]


# ------------------------------------------------------------------------------------------ attention
def _sdpa(q, k, v, attn_mask=None, causal=False):
    """torch CPU scaled_dot_product_attention in float64, heads expanded for GQA."""
    L, hq, d = q.shape
    grp = hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()
    kt = torch.from_numpy(np.repeat(k, grp, axis=1)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.repeat(v, grp, axis=1)).permute(1, 0, 2).contiguous()
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("L,B,hq,hkv,d", [(50, 8, 4, 2, 16), (64, 16, 8, 1, 8), (7, 4, 2, 2, 4), (1, 4, 1, 1, 4)])
def test_full_budget_equals_textbook_dense_attention(L, B, hq, hkv, d):
    q, k, v = _tiny_qkv(L, hq, hkv, d, seed=L)
    n = -(-L // B)
    mask = np.ones((hq, n, n), dtype=bool)
    O, lse = oracle.block_sparse_attention(q, k, v, mask, B)
    ref = _sdpa(q, k, v, causal=True)
    assert np.max(np.abs(O - ref)) < 1e-12
    Od, lsed = oracle.dense_causal_attention(q, k, v)
    assert np.max(np.abs(Od - ref)) < 1e-12
    # LSE against an explicit logsumexp of the causal logits
    grp = hq // hkv
    for h in range(hq):
        s = (q[:, h] @ k[:, h // grp].T) / math.sqrt(d)
        s = np.where(np.tril(np.ones((L, L), dtype=bool)), s, -np.inf)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
        assert np.max(np.abs(lse[h] - ref_lse)) < 1e-12


def test_random_block_mask_equals_additive_neg_inf_mask():
    """Skipped blocks act as -inf scores: compare with SDPA under an additive block mask."""
    L, B, hq, hkv, d = 45, 8, 4, 2, 16
    q, k, v = _tiny_qkv(L, hq, hkv, d, seed=9)
    n = -(-L // B)
    rng = np.random.default_rng(10)
    mask = rng.random((hq, n, n)) < 0.5
    mask[:, :, 0] = True  # keep every query row non-empty for the SDPA comparison
    O, lse = oracle.block_sparse_attention(q, k, v, mask, B)
    add = np.full((hq, L, L), -np.inf)
    for h in range(hq):
        for t in range(L):
            for s_ in range(t + 1):
                if mask[h, t // B, s_ // B]:
                    add[h, t, s_] = 0.0
    ref = _sdpa(q, k, v, attn_mask=add)
    assert np.max(np.abs(O - ref)) < 1e-12


def test_empty_row_gives_zero_output_and_neg_inf_lse():
    L, B = 16, 4
    q, k, v = _tiny_qkv(L, 2, 1, 4, seed=11)
    mask = np.ones((2, 4, 4), dtype=bool)
    mask[1, 2, :] = False
    O, lse = oracle.block_sparse_attention(q, k, v, mask, B)
    assert np.all(O[8:12, 1] == 0) and np.all(np.isneginf(lse[1, 8:12]))
    assert np.all(np.isfinite(O[:, 0]))


def test_rows_subset_matches_full_run():
    L, B = 40, 8
    q, k, v = _tiny_qkv(L, 4, 2, 8, seed=12)
    mask = np.random.default_rng(13).random((4, 5, 5)) < 0.6
    mask[:, :, 0] = True
    O, lse = oracle.block_sparse_attention(q, k, v, mask, B)
    Os, lses = oracle.block_sparse_attention(q, k, v, mask, B, rows=[(3, 4), (0, 2)])
    assert np.array_equal(Os[32:40, 3], O[32:40, 3]) and np.array_equal(lses[0, 16:24], lse[0, 16:24])
    assert np.isnan(Os[0, 1, 0])


# ------------------------------------------------------------------------------------ naive comparator
def test_naive_sampled_positions():
    pos = oracle.sampled_query_positions(300, 64, 4)
    assert pos.tolist()[0] == [0, 16, 32, 48]
    assert pos.tolist()[-1] == [256, 272, 288, 299]  # the partial last block repeats its last token


def test_naive_scores_uniform_keys_closed_form():
    """All keys equal: every softmax is uniform over the t + 1 visible keys, so the mass of block j is
    |block j within [0, t]| / (t + 1) (beta = 0 isolates the routing term)."""
    rng = np.random.default_rng(1)
    L, B, S = 200, 32, 4
    q = rng.normal(size=(L, 2, 8))
    k = np.tile(rng.normal(size=(1, 1, 8)), (L, 1, 1))
    v = rng.normal(size=(L, 1, 8))
    got = oracle.naive_block_scores(q, k, v, B, 0.0, S)
    pos = oracle.sampled_query_positions(L, B, S)
    n = -(-L // B)
    for i in range(n):
        for j in range(i + 1):
            want = np.mean([max(0, min((j + 1) * B, t + 1) - j * B) / (t + 1) for t in pos[i]])
            assert abs(got[0, i, j] - math.log(want)) < 1e-12
            assert abs(got[1, i, j] - math.log(want)) < 1e-12


def test_naive_scores_mass_sums_to_one():
    """Probability conservation: for each row the block masses (exp of score minus beta M) add up to 1."""
    rng = np.random.default_rng(2)
    L, B = 333, 32
    q, k, v = rng.normal(size=(L, 4, 16)), rng.normal(size=(L, 2, 16)), rng.normal(size=(L, 2, 16))
    S = oracle.naive_block_scores(q, k, v, B, 0.3, 8)
    M = oracle.value_log_magnitude(v, B)
    for h in range(4):
        for i in range(S.shape[1]):
            assert abs(np.exp(S[h, i, : i + 1] - 0.3 * M[h // 2, : i + 1]).sum() - 1.0) < 1e-12


def test_naive_scores_against_masked_softmax_over_the_full_matrix():
    """Brute force by another route: the full token-level logit matrix, an additive causal mask, torch's
    softmax, then block sums of the sampled rows."""
    rng = np.random.default_rng(3)
    L, B, S, hq, hkv, d = 150, 16, 2, 4, 2, 8
    q, k, v = rng.normal(size=(L, hq, d)), rng.normal(size=(L, hkv, d)), rng.normal(size=(L, hkv, d))
    got = oracle.naive_block_scores(q, k, v, B, 0.5, S)
    M = oracle.value_log_magnitude(v, B)
    pos = oracle.sampled_query_positions(L, B, S)
    n = -(-L // B)
    for h in range(hq):
        g = h // (hq // hkv)
        logits = torch.tensor(q[:, h] @ k[:, g].T / math.sqrt(d))
        logits = logits.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        P = torch.softmax(logits, dim=1).numpy()
        pad = np.zeros((L, n * B))
        pad[:, :L] = P
        mass = pad.reshape(L, n, B).sum(axis=2)  # [t][j]
        for i in range(n):
            want = np.log(mass[pos[i]].mean(axis=0)[: i + 1]) + 0.5 * M[g, : i + 1]
            assert np.max(np.abs(got[h, i, : i + 1] - want)) < 1e-12


# ------------------------------------------------------------------------------------ W8A8 quantisation
def test_e4m3fn_encoder_matches_torch_cast_including_midpoints():
    rng = np.random.default_rng(0)
    tab = oracle.e4m3fn_table()[:0x7F]
    mids = ((tab[1:] + tab[:-1]) / 2).astype(np.float32)
    y = np.concatenate([rng.uniform(-448, 448, 50000).astype(np.float32), rng.normal(0, 0.01, 5000).astype(np.float32),
                        mids, -mids, tab.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0])])
    got = oracle.e4m3fn_encode(y.astype(np.float64))
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_quantize_fp8_per_head_closed_forms():
    """amax maps to the largest code (448); the scale is amax/448 in fp32; half the amax maps to 224
    (representable); decoding the codes times the scale stays within half a quantum of x."""
    rng = np.random.default_rng(5)
    x = rng.normal(size=(64, 3, 16)).astype(np.float32).astype(np.float64)
    x[7, 1, 3] = 12.5  # head 1's amax
    x[9, 1, 4] = -6.25  # half of it, negative
    codes, scale = oracle.quantize_fp8_per_head(x)
    assert scale[1] == np.float32(np.float32(12.5) / np.float32(448.0))
    assert codes[7, 1, 3] == 0x7E and codes[9, 1, 4] == (0x80 | 0x76)  # 448 = 1.75*2^8, 224 = 1.75*2^7
    back = oracle.fp8_to_f64(codes, scale)
    for h in range(3):
        # the dequantised value is within half a quantum of x, in x's own units: the quantum of y = x/scale
        # (2^-3 of y's binade, 2^-9 below the normal range) times the head's scale
        y = x[:, h] / float(scale[h])
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))), -6).astype(np.int64)
        spacing = np.ldexp(1.0, np.minimum(e, 8) - 3) * float(scale[h])
        assert np.all(np.abs(back[:, h] - x[:, h]) <= spacing / 2 * (1 + 1e-9))


def test_fp8_dequantisation_applies_each_heads_own_scale():
    """W8A8 dequantisation ([Arch] "答案不在算法里", W8A8-FP8): value = e4m3fn(code) * scale[head].
    Hand-built codes with exact values (0x38 = 1.0, 0xB0 = -0.5, 0x7E = 448, 0x01 = 2^-9) under three
    distinct per-head scales: dividing by the scale, dropping it or taking another head's scale all fail."""
    scale = np.array([0.5, 2.0, 3.0], dtype=np.float32)
    codes = np.zeros((2, 3, 4), dtype=np.uint8)
    codes[:, :, 0] = 0x38
    codes[:, :, 1] = 0xB0
    codes[:, :, 2] = 0x7E
    codes[:, :, 3] = 0x01
    back = oracle.fp8_to_f64(codes, scale)
    unit = np.array([1.0, -0.5, 448.0, 2.0 ** -9])
    for t in range(2):
        for h in range(3):
            assert np.array_equal(back[t, h], unit * float(scale[h])), (t, h)
    # a single head slice with its own one-element scale array, as the tests pass it
    assert np.array_equal(oracle.fp8_to_f64(codes[:, 2:3], scale[2:3])[0, 0], unit * 3.0)


def test_fp8_dequantisation_matches_torch_decode_times_scale():
    """Random codes of every finite value, four heads with unrelated scales: the oracle's dequantisation
    equals torch's float8_e4m3fn decode multiplied by the head's scale, exactly (both are exact in
    float64)."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(257, 4, 16), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11  # NaN codes aside
    scale = np.array([1.5e-3, 0.75, 7.0, 2.0 ** -20], dtype=np.float32)
    got = oracle.fp8_to_f64(codes, scale)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = dec * scale.astype(np.float64)[None, :, None]
    assert np.array_equal(got, want)
