"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Small cases (several tiles, ragged tails, GQA 1/4/8, paged with 16/32/64-token pages, fp32/bf16/fp8,
external masks with empty rows) are checked on every output; the full-size workloads are checked on all
budgets and selections and on sampled attention rows.  Selections must be bit-exact except in near-tie rows
(k-th and (k+1)-th oracle scores within 1e-5 relative); attention given the oracle's mask must meet the
max/mean abs tolerances of its dtype.
"""
import math
import sys

import numpy as np
import pytest

import synth
import oracle
from tests import stem_cases as sc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_oam_amd as stem  # noqa: F401  (fails loudly if libstem.so is missing)

    stem.lib()
    return torch.device("cuda:0")


def _run(p, x, dev, masks_for_bsa=None, dense=False):
    """Run the three stages on the GPU.  masks_for_bsa: per-request bool masks to feed bsa_prefill
    (the oracle's); None uses the GPU's own selection.  Returns a dict of host arrays."""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    kw = {}
    if p.dtype == "fp8":
        kw = dict(q_scale=upload(x["q_scale"]), k_scale=upload(x["k_scale"]), v_scale=upload(x["v_scale"]))
    if p.paged:
        pt = upload(x["page_table"])
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, page_table=pt,
                                 page_size=p.page_size, num_pages=x["k_pages"].shape[0], **kw)
        k, v = upload(x["k_pages"]), upload(x["v_pages"])
    else:
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, **kw)
        k, v = upload(x["k"]), upload(x["v"])
    q = upload(x["q"])
    L = StemPrefill(prob, dev)
    L.score(q, k, v, p.beta)
    L.select((p.rho_num, p.rho_den), (p.mu_num, p.mu_den))
    res = {}
    qb, kb, M = L.pooled()
    torch.cuda.synchronize()
    res["qbar"], res["kbar"], res["M"] = qb.cpu().numpy(), kb.cpu().numpy(), M.cpu().numpy()
    res["scores"] = L.scores.cpu().numpy()
    res["words"] = L.mask.cpu().numpy().view(np.uint32)
    res["counts"] = L.counts.cpu().numpy()
    if masks_for_bsa is not None:
        full = np.zeros((p.hq, L.NB, L.words), dtype=np.int32)
        cb = p.cu_blocks
        for r, m in enumerate(masks_for_bsa):
            full[:, cb[r]:cb[r + 1]] = sc.pack_mask(m, L.words)
        ext = upload(full)
        L.attend(q, k, v, mask=ext)
    else:
        L.attend(q, k, v, mask=None if dense else "selected")
    torch.cuda.synchronize()
    res["out"] = L.out.float().cpu().numpy().astype(np.float64)
    res["lse"] = L.lse.cpu().numpy().astype(np.float64)
    res["NB"] = L.NB
    return res


def _check_stage1(p, g, ref):
    cb = p.cu_blocks
    worst_s = 0.0
    for r, (qbar, kbar, M, S) in enumerate(ref):
        if S.shape[1] == 0:  # an empty request: no blocks
            continue
        sl = slice(cb[r], cb[r + 1])
        assert np.max(np.abs(g["qbar"][:, sl] - qbar)) < 1e-5
        assert np.max(np.abs(g["kbar"][:, sl] - kbar)) < 1e-5
        assert np.max(np.abs(g["M"][:, sl] - M)) < 1e-5
        n = S.shape[1]
        tri = np.tril(np.ones((n, n), dtype=bool))
        gs = g["scores"][:, sl, :n]
        err = np.abs(gs - S)[:, tri] / np.maximum(1.0, np.abs(S[:, tri]))
        worst_s = max(worst_s, float(err.max()))
    assert worst_s < 2e-6, worst_s  # well inside the 1e-5 selection tie window
    return worst_s


SMALL = [
    ("tiny_f32", {}),
    ("tiny_f32", dict(lens=(1000,), hq=4, hkv=1)),
    ("llama_32k_bf16", dict(lens=(1000,), hq=8, hkv=2)),
    ("llama_32k_bf16", dict(lens=(300, 1, 129, 700), hq=4, hkv=4)),
    ("llama_32k_bf16", dict(lens=(777,), hq=8, hkv=1, d=64)),
    ("llama_32k_bf16", dict(lens=(640,), hq=4, hkv=2, block=64)),
    ("llama_32k_bf16", dict(lens=(1500,), hq=4, hkv=1, rho_num=50, mu_num=1, mu_den=1)),
    ("llama_32k_bf16", dict(lens=(1100, 2000), hq=8, hkv=2, beta=0.0)),
    ("llama_32k_bf16", dict(lens=(3000,), hq=4, hkv=1, beta=0.0, mu_num=1, mu_den=1)),
    ("w8a8_128k_fp8", dict(lens=(1000,), hq=8, hkv=2)),
    ("w8a8_128k_fp8", dict(lens=(200, 513), hq=4, hkv=1, d=64)),
    ("paged_ragged_bf16", dict(lens=(300, 64, 700), hq=4, hkv=2)),
    ("paged_ragged_bf16", dict(lens=(257, 1000), hq=4, hkv=1, page_size=16)),
    ("paged_ragged_bf16", dict(lens=(129, 500), hq=2, hkv=2, page_size=32, dtype="fp8")),
    ("llama_32k_bf16", dict(lens=(300, 0, 129), hq=4, hkv=2)),  # an empty request inside a batch
    ("paged_ragged_bf16", dict(lens=(0, 200, 0, 64), hq=2, hkv=1)),
    ("w8a8_128k_fp8", dict(lens=(0, 700), hq=4, hkv=2)),
    # an odd number of query heads per KV head: one head per workgroup, with pages of 64 and of 16 tokens
    ("paged_ragged_bf16", dict(lens=(300, 700), hq=3, hkv=1)),
    ("paged_ragged_bf16", dict(lens=(257, 1000), hq=3, hkv=3, page_size=16)),
    # fp8 with two query heads per workgroup over pages of 64 and of 32 tokens
    ("paged_ragged_bf16", dict(lens=(300, 700), hq=4, hkv=2, dtype="fp8")),
    ("paged_ragged_bf16", dict(lens=(129, 500), hq=8, hkv=2, page_size=32, dtype="fp8")),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_small_case_all_outputs(dev, name, over):
    p = synth.make_problem(name, **over)
    _log(f"[case] {name} {over}")
    x = synth.make_inputs(p, seed=0)
    ref1 = sc.oracle_stage1(p, x)
    budgets = sc.oracle_budgets(p)
    masks = sc.oracle_masks([s for *_, s in ref1], budgets)
    g = _run(p, x, dev, masks_for_bsa=masks)
    worst = _check_stage1(p, g, ref1)
    ties = sc.check_selection(p, [s for *_, s in ref1], budgets, g["words"], g["counts"])
    ora = sc.oracle_attention(p, x, masks)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"])
    tmax, tmean = sc.TOL[p.dtype]
    _log(f"  score rel err {worst:.2e}, near-tie rows {ties}, out max {mx:.2e} mean {mean:.2e}, lse {lerr:.2e}")
    assert mx <= tmax and mean <= tmean
    assert lerr <= sc.LSE_TOL


def _random_problem(seed):
    """A seeded random small problem over the supported space: dtype, head_dim and block cycle with the
    seed (so that the twelve cases cover each kernel), the rest is drawn: GQA ratio, 1-3 requests (some
    empty, some shorter than a block), contiguous or paged K/V (pages of 16-96 tokens, also ones that do
    not divide the block), budget, mu and beta."""
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "fp8", "bf16", "f32"][seed % 4]
    block = [128, 128, 64][seed % 3]
    d = 64 if seed % 5 == 2 else 128
    hq, hkv = [(2, 1), (3, 1), (4, 1), (4, 2), (6, 2), (8, 2), (2, 2), (6, 3)][rng.integers(8)]
    nreq = int(rng.integers(1, 4))
    lens = []
    for _ in range(nreq):
        u = rng.random()
        lens.append(0 if u < 0.1 else int(rng.integers(1, 200)) if u < 0.4 else int(rng.integers(200, 1500)))
    if sum(lens) == 0:
        lens[0] = 333
    mu = [(7, 10), (1, 1), (1, 2)][rng.integers(3)]
    over = dict(lens=tuple(lens), hq=hq, hkv=hkv, d=d, block=block, dtype=dtype,
                rho_num=int(rng.choice([10, 25, 50, 100])), beta=float(rng.choice([0.2, 0.0, 0.5])),
                mu_num=mu[0], mu_den=mu[1])
    if seed % 5 in (1, 3):
        over.update(paged=True, page_size=int(rng.choice([16, 32, 48, 64, 96])))
    return synth.make_problem("llama_32k_bf16", **over)


@pytest.mark.parametrize("seed", range(12))
def test_random_small_problem_all_outputs(dev, seed):
    """Every output of the three stages against the oracle on a seeded random problem."""
    p = _random_problem(seed)
    _log(f"[random {seed}] lens {p.lens} hq {p.hq} hkv {p.hkv} d {p.d} block {p.block} {p.dtype} "
         f"paged {p.paged}/{p.page_size} rho {p.rho_num}% mu {p.mu_num}/{p.mu_den} beta {p.beta}")
    x = synth.make_inputs(p, seed=seed)
    ref1 = sc.oracle_stage1(p, x)
    budgets = sc.oracle_budgets(p)
    masks = sc.oracle_masks([s for *_, s in ref1], budgets)
    g = _run(p, x, dev, masks_for_bsa=masks)
    _check_stage1(p, g, ref1)
    ties = sc.check_selection(p, [s for *_, s in ref1], budgets, g["words"], g["counts"])
    ora = sc.oracle_attention(p, x, masks)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"])
    tmax, tmean = sc.TOL[p.dtype]
    _log(f"  near-tie rows {ties}, out max {mx:.2e} mean {mean:.2e}, lse {lerr:.2e}")
    assert mx <= tmax and mean <= tmean
    assert lerr <= sc.LSE_TOL


def test_plain_c_program_runs_the_path(dev, tmp_path):
    """A C99 program (tests/c_abi_pipeline.c) built with gcc against stem.h and the HIP runtime's C API
    runs stem_score, stem_tpd_topk and bsa_prefill on seeded inputs; its selection and outputs are
    checked against the oracle like the Python binding's."""
    import os
    import subprocess
    from block_sparse_attention_oam_amd import _abi

    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.dirname(_abi.LIB_PATH)
    exe = str(tmp_path / "c_abi_pipeline")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I" + os.path.join(root, "include"), os.path.join(here, "c_abi_pipeline.c"), "-L" + libdir,
                        "-lstem", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + libdir, "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    p = synth.make_problem("llama_32k_bf16", lens=(1100,), hq=4, hkv=2)
    x = synth.make_inputs(p, seed=11)
    for name in ("q", "k", "v"):
        np.ascontiguousarray(x[name]).tofile(str(tmp_path / (name + ".bin")))
    _log("[c pipeline] 1100 tokens, 4 query / 2 KV heads")
    r = subprocess.run([exe, str(tmp_path), "1100", "4", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    n = p.nblocks(0)
    words = np.fromfile(str(tmp_path / "mask.bin"), dtype=np.uint32).reshape(p.hq, n, (n + 31) // 32)
    counts = np.fromfile(str(tmp_path / "counts.bin"), dtype=np.int32).reshape(p.hq, n)
    bits = np.fromfile(str(tmp_path / "out.bin"), dtype=np.uint16).reshape(1100, p.hq, p.d)
    out = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lse = np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).reshape(p.hq, 1100).astype(np.float64)
    ref1 = sc.oracle_stage1(p, x)
    budgets = sc.oracle_budgets(p)
    sc.check_selection(p, [s for *_, s in ref1], budgets, words, counts)
    gmask = sc.unpack_mask(words, n) & np.tril(np.ones((n, n), dtype=bool))[None]
    ora = sc.oracle_attention(p, x, [gmask])
    mx, mean, lerr = sc.compare_attention(p, ora, out, lse)
    _log(f"  out max {mx:.2e} mean {mean:.2e} lse {lerr:.2e}")
    assert mx <= 2e-2 and mean <= 2e-3 and lerr <= sc.LSE_TOL


@pytest.mark.parametrize("name,over", [SMALL[0], SMALL[2], SMALL[3], SMALL[9], SMALL[11]],
                         ids=["f32", "bf16", "bf16-one-head-per-workgroup", "fp8", "paged"])
def test_dense_mode_matches_textbook_attention(dev, name, over):
    """mask = NULL runs dense causal attention: the 100%-budget special case of the oracle."""
    p = synth.make_problem(name, **over)
    x = synth.make_inputs(p, seed=1)
    g = _run(p, x, dev, dense=True)
    ora = sc.oracle_attention(p, x, None)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"])
    _log(f"[dense] {name}: out max {mx:.2e} mean {mean:.2e} lse {lerr:.2e}")
    tmax, tmean = sc.TOL[p.dtype]
    assert mx <= tmax and mean <= tmean and lerr <= sc.LSE_TOL


LARGE = [("llama_32k_bf16", dict(lens=(1000, 300), hq=4, hkv=2)),
         ("llama_32k_bf16", dict(lens=(700,), hq=3, hkv=1)),
         ("w8a8_128k_fp8", dict(lens=(1000, 300), hq=4, hkv=2)),
         ("tiny_f32", dict(lens=(600,), hq=4, hkv=2))]


@pytest.mark.parametrize("factor", [2.0, 4.0, 8.0])
@pytest.mark.parametrize("name,over,dense", [(n, o, False) for n, o in LARGE] + [(*LARGE[0], True)],
                         ids=["bf16", "bf16-one-head-per-workgroup", "fp8", "f32", "bf16-dense"])
def _bf16_round(a):
    """float64 -> nearest bf16 value (through float32, ties to even), as float64."""
    u = np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_p_model_error(p, x, masks, ora):
    """Max abs error, against the oracle, of a model of the kernels' rounding (test-side, not part of the
    oracle): float64 attention whose softmax weights P are rounded to bf16 before they weight V and before
    they are summed, with the output rounded to bf16.  Only the reference point of the exponentials differs
    from the kernels (the row max here), which changes which way each P rounds but not by how much."""
    worst = 0.0
    grp = p.hq // p.hkv
    scale = 1.0 / math.sqrt(p.d)
    for r, (a, b) in enumerate(sc.request_slices(p)):
        L, n = b - a, p.nblocks(r)
        if L == 0:
            continue
        q, k, v = sc.decode_q(p, x, a, b), sc.decode_kv(p, x, r, "k"), sc.decode_kv(p, x, r, "v")
        m = masks[r] if masks is not None else np.ones((p.hq, n, n), dtype=bool)
        O = ora[r][0]
        for h in range(p.hq):
            for i in range(n):
                t0, t1 = i * p.block, min((i + 1) * p.block, L)
                sel = np.nonzero(m[h, i, : i + 1])[0]
                if not len(sel):
                    continue
                kid = np.concatenate([np.arange(j * p.block, min((j + 1) * p.block, L)) for j in sel])
                lg = q[t0:t1, h] @ k[kid, h // grp].T * scale
                lg = np.where(kid[None, :] <= np.arange(t0, t1)[:, None], lg, -np.inf)
                P = _bf16_round(np.exp(lg - lg.max(axis=1, keepdims=True)))
                o = _bf16_round((P @ v[kid, h // grp]) / P.sum(axis=1, keepdims=True))
                worst = max(worst, float(np.abs(o - O[t0:t1, h]).max()))
    return worst


@pytest.mark.parametrize("factor", [2.0, 4.0, 8.0])
@pytest.mark.parametrize("name,over,dense", [(n, o, False) for n, o in LARGE] + [(*LARGE[0], True)],
                         ids=["bf16", "bf16-one-head-per-workgroup", "fp8", "f32", "bf16-dense"])
def test_large_logits_take_the_rebase_path(dev, name, over, dense, factor):
    """Q and K scaled by an exact power of two, so every logit grows by factor^2 (at 8: logits up to ~200,
    row spreads of ~40 in natural units): rows get peaked and later keys outgrow the softmax reference
    taken from a row's first keys by more than the kernels allow, which sends them through their rebase
    path.

    Bound, computed: the logits are exact fp32 sums of exact products, so their size adds no error; what
    peaked rows expose is the bf16 rounding of each P and of the output.  A float64 model with exactly
    those roundings (_bf16_p_model_error) gives the error they cause on these inputs; the kernel must stay
    within 1.5x of it (it rounds other P values, since its exponentials start from another reference, so
    its maximum is another draw of the same size) or within the dtype's tolerance, whichever is larger.
    The fp32 path keeps P in fp32; its logits' rounding is relative, so its tolerance grows with them
    (factor^2)."""
    p = synth.make_problem(name, **over)
    _log(f"[large logits] {name} {over} x{factor} dense={dense}")
    x = synth.make_inputs(p, seed=6)
    f = np.float32(factor)
    if p.dtype == "fp8":  # the codes stay, the per-head scales grow
        x["q_scale"] = x["q_scale"] * f
        x["k_scale"] = x["k_scale"] * f
    elif p.dtype == "bf16":  # exact: a power of two moves the exponent only
        for key in ("q", "k"):
            x[key] = synth.bf16_bits((x[key].astype(np.uint32) << 16).view(np.float32) * f)
    else:
        x["q"], x["k"] = x["q"] * f, x["k"] * f
    if dense:
        masks = None
        g = _run(p, x, dev, dense=True)
    else:
        ref1 = sc.oracle_stage1(p, x)
        masks = sc.oracle_masks([s for *_, s in ref1], sc.oracle_budgets(p))
        g = _run(p, x, dev, masks_for_bsa=masks)
    ora = sc.oracle_attention(p, x, masks)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"])
    tmax, tmean = sc.TOL[p.dtype]
    if p.dtype == "f32":
        model, bound = 0.0, tmax * factor ** 2
    else:
        model = _bf16_p_model_error(p, x, masks, ora)
        bound = max(tmax, 1.5 * model)
    _log(f"  out max {mx:.2e} (bf16-P model {model:.2e}, bound {bound:.2e}) mean {mean:.2e} lse {lerr:.2e}")
    assert mx <= bound and mean <= tmean and lerr <= sc.LSE_TOL


def test_end_to_end_gpu_selection_feeds_attention(dev):
    p = synth.make_problem("llama_32k_bf16", lens=(1200, 333), hq=8, hkv=2)
    x = synth.make_inputs(p, seed=2)
    g = _run(p, x, dev)
    cb = p.cu_blocks
    gmasks = [sc.unpack_mask(g["words"][:, cb[r]:cb[r + 1]], p.nblocks(r)) for r in range(len(p.lens))]
    for m in gmasks:
        m &= np.tril(np.ones(m.shape[1:], dtype=bool))[None]
    ora = sc.oracle_attention(p, x, gmasks)
    mx, mean, _ = sc.compare_attention(p, ora, g["out"], g["lse"])
    assert mx <= 2e-2 and mean <= 2e-3


def test_external_mask_with_empty_rows_and_skipped_diagonal(dev):
    p = synth.make_problem("llama_32k_bf16", lens=(900, 260), hq=4, hkv=2)
    x = synth.make_inputs(p, seed=3)
    rng = np.random.default_rng(4)
    masks = []
    for r in range(len(p.lens)):
        n = p.nblocks(r)
        m = rng.random((p.hq, n, n)) < 0.4
        m[0, :, :] = False  # head 0: every row empty
        m[1, np.arange(n), np.arange(n)] = False  # head 1: diagonal never selected
        m[2, :, :] = True  # head 2: dense, plus bits past the diagonal that must be ignored
        masks.append(m)
    g = _run(p, x, dev, masks_for_bsa=masks)
    tri = [m & np.tril(np.ones(m.shape[1:], dtype=bool))[None] for m in masks]
    ora = sc.oracle_attention(p, x, tri)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"])
    assert mx <= 2e-2 and mean <= 2e-3
    a, b = sc.request_slices(p)[0]
    assert np.all(g["out"][a:b, 0] == 0) and np.all(np.isneginf(g["lse"][0, a:b]))


def test_repeated_runs_are_bitwise_identical(dev):
    p = synth.make_problem("llama_32k_bf16", lens=(2000,), hq=8, hkv=2)
    x = synth.make_inputs(p, seed=5)
    g1 = _run(p, x, dev)
    g2 = _run(p, x, dev)
    for key in ("scores", "words", "counts", "out", "lse"):
        a, b = g1[key], g2[key]
        if key == "scores":
            n = p.nblocks(0)
            tri = np.tril(np.ones((n, n), dtype=bool))
            a, b = a[:, :, :n][:, tri], b[:, :, :n][:, tri]
        assert np.array_equal(a, b, equal_nan=True), key


# ------------------------------------------------------------------------------------ full-size workloads
FULL = ["tiny_f32", "llama_32k_bf16", "llama_128k_bf16", "w8a8_128k_fp8", "paged_ragged_bf16"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(dev, name):
    """All budgets and selections bit-exact (tie window aside); attention on sampled rows with the oracle's
    mask; the dense mode on sampled rows."""
    p = synth.make_problem(name)
    _log(f"[full] {name}: generating inputs")
    x = synth.make_inputs(p, seed=0)
    _log(f"[full] {name}: oracle scores and selection")
    ref1 = sc.oracle_stage1(p, x)
    S_list = [s for *_, s in ref1]
    budgets = sc.oracle_budgets(p)
    masks = sc.oracle_masks(S_list, budgets)
    _log(f"[full] {name}: GPU run")
    g = _run(p, x, dev, masks_for_bsa=masks)
    worst = _check_stage1(p, g, ref1)
    ties = sc.check_selection(p, S_list, budgets, g["words"], g["counts"])
    rows = [sc.sample_rows(p, r, 12, mask=masks[r]) if p.lens[r] > 4096 else None for r in range(len(p.lens))]
    _log(f"[full] {name}: oracle attention on sampled rows")
    ora = sc.oracle_attention(p, x, masks, rows)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"], rows)
    _log(f"[full] {name}: score rel {worst:.2e}, near-tie rows {ties}, out max {mx:.2e} mean {mean:.2e}, "
         f"lse {lerr:.2e}")
    tmax, tmean = sc.TOL[p.dtype]
    assert mx <= tmax and mean <= tmean and lerr <= sc.LSE_TOL


# ------------------------------------------------------------------------------------ W8A8 quantising stage 1
def _quantize_and_reference(p8, xb, dev):
    """stem_quantize_score on bf16 inputs, and stem_score on the codes and scales it produced."""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    q, k, v = upload(xb["q"]), upload(xb["k"]), upload(xb["v"])
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    v8 = torch.empty(v.shape, dtype=torch.uint8, device=dev)
    qs = torch.empty(p8.hq, dtype=torch.float32, device=dev)
    ks = torch.empty(p8.hkv, dtype=torch.float32, device=dev)
    vs = torch.empty(p8.hkv, dtype=torch.float32, device=dev)
    prob = stem.make_problem(p8.cu_seqlens, p8.hq, p8.hkv, p8.d, p8.block, "fp8", q_scale=qs, k_scale=ks, v_scale=vs)
    L1 = StemPrefill(prob, dev)
    L1.scores.fill_(float("nan"))
    stem.stem_quantize_score(prob, q, k, v, q8, k8, v8, qs, ks, vs, p8.beta, L1.scores, L1.ws)
    L2 = StemPrefill(prob, dev)
    L2.scores.fill_(float("nan"))
    L2.score(q8, k8, v8, p8.beta)
    torch.cuda.synchronize()
    return L1, L2, (q8, k8, v8), (qs, ks, vs)


@pytest.mark.parametrize("over", [dict(lens=(1000,), hq=8, hkv=2), dict(lens=(200, 513), hq=4, hkv=1, d=64),
                                  dict(lens=(2000, 300), hq=8, hkv=8, block=64)])
def test_quantize_score_codes_scales_and_pooling(dev, over):
    """Codes and scales bit-exact against the oracle's quantisation; pooled tensors and scores bit-exact
    against stem_score run on those codes."""
    pb = synth.make_problem("w8a8_128k_fp8", dtype="bf16", **over)
    p8 = synth.make_problem("w8a8_128k_fp8", **over)
    xb = synth.make_inputs(pb, seed=4)
    L1, L2, codes, scales = _quantize_and_reference(p8, xb, dev)
    for name, c, s_ in (("q", codes[0], scales[0]), ("k", codes[1], scales[1]), ("v", codes[2], scales[2])):
        want_c, want_s = oracle.quantize_fp8_per_head(oracle.bf16_to_f64(xb[name]))
        assert np.array_equal(s_.cpu().numpy(), want_s), name
        assert np.array_equal(c.cpu().numpy(), want_c), name
    for t1, t2 in zip(L1.pooled(), L2.pooled()):
        assert torch.equal(t1, t2)
    n = max(p8.nblocks(r) for r in range(len(p8.lens)))
    tri = torch.tril(torch.ones(n, n, dtype=torch.bool, device=dev))
    for r in range(len(p8.lens)):
        nr = p8.nblocks(r)
        a = L1.scores[:, p8.cu_blocks[r]:p8.cu_blocks[r + 1], :nr][:, tri[:nr, :nr]]
        b = L2.scores[:, p8.cu_blocks[r]:p8.cu_blocks[r + 1], :nr][:, tri[:nr, :nr]]
        assert torch.equal(a, b)


@pytest.mark.parametrize("over", [dict(lens=(1000,), hq=8, hkv=2), dict(lens=(200, 513), hq=4, hkv=1, d=64)])
def test_quantize_fp8_alone_matches_oracle_and_fused_stage(dev, over):
    """stem_quantize_fp8 (no pooling): scales and codes bit-exact against the oracle's quantisation and
    equal to stem_quantize_score's; stem_score on them gives stem_quantize_score's scores."""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    pb = synth.make_problem("w8a8_128k_fp8", dtype="bf16", **over)
    p8 = synth.make_problem("w8a8_128k_fp8", **over)
    xb = synth.make_inputs(pb, seed=5)
    L1, _, codes, scales = _quantize_and_reference(p8, xb, dev)
    q, k, v = upload(xb["q"]), upload(xb["k"]), upload(xb["v"])
    c2 = [torch.full(t.shape, 0xAB, dtype=torch.uint8, device=dev) for t in (q, k, v)]
    s2 = [torch.full((n,), float("nan"), dtype=torch.float32, device=dev) for n in (p8.hq, p8.hkv, p8.hkv)]
    prob = stem.make_problem(p8.cu_seqlens, p8.hq, p8.hkv, p8.d, p8.block, "fp8", q_scale=s2[0], k_scale=s2[1],
                             v_scale=s2[2])
    stem.stem_quantize_fp8(prob, q, k, v, *c2, *s2)
    L3 = StemPrefill(prob, dev)
    L3.scores.fill_(float("nan"))
    L3.score(*c2, p8.beta)
    torch.cuda.synchronize()
    for name, c, s_, cf, sf in zip("qkv", c2, s2, codes, scales):
        want_c, want_s = oracle.quantize_fp8_per_head(oracle.bf16_to_f64(xb[name]))
        assert np.array_equal(s_.cpu().numpy(), want_s), name
        assert np.array_equal(c.cpu().numpy(), want_c), name
        assert torch.equal(c, cf) and torch.equal(s_, sf), name
    for r in range(len(p8.lens)):
        nr = p8.nblocks(r)
        tri = torch.tril(torch.ones(nr, nr, dtype=torch.bool, device=dev))
        a = L1.scores[:, p8.cu_blocks[r]:p8.cu_blocks[r + 1], :nr][:, tri]
        b = L3.scores[:, p8.cu_blocks[r]:p8.cu_blocks[r + 1], :nr][:, tri]
        assert torch.equal(a, b)


@pytest.mark.timeout(600)
def test_quantize_score_full_size_128k(dev):
    """The 128K fp8 layer from its bf16 activations: scales bit-exact, codes bit-exact on sampled token
    rows, pooled tensors and scores bit-exact against stem_score on the produced codes."""
    pb = synth.make_problem("w8a8_128k_fp8", dtype="bf16")
    p8 = synth.make_problem("w8a8_128k_fp8")
    _log("[quant] 128K: generating bf16 inputs")
    xb = synth.make_inputs(pb, seed=0)
    L1, L2, codes, scales = _quantize_and_reference(p8, xb, dev)
    rows = np.random.default_rng(0).choice(p8.tokens, 512, replace=False)
    for name, c, s_ in (("q", codes[0], scales[0]), ("k", codes[1], scales[1]), ("v", codes[2], scales[2])):
        want_c, want_s = oracle.quantize_fp8_per_head(oracle.bf16_to_f64(xb[name]), rows=rows)
        assert np.array_equal(s_.cpu().numpy(), want_s), name
        assert np.array_equal(c.cpu().numpy()[rows], want_c), name
    for t1, t2 in zip(L1.pooled(), L2.pooled()):
        assert torch.equal(t1, t2)
    n = p8.nblocks(0)
    tri = torch.tril(torch.ones(n, n, dtype=torch.bool, device=dev))
    assert torch.equal(L1.scores[:, :, :n][:, tri], L2.scores[:, :, :n][:, tri])


# ------------------------------------------------------------------------------------ fused scoring + selection
def _layer(p, x, dev):
    """The problem descriptor, a StemPrefill and the device inputs of a synthetic workload."""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    kw = {}
    if p.dtype == "fp8":
        kw = dict(q_scale=upload(x["q_scale"]), k_scale=upload(x["k_scale"]), v_scale=upload(x["v_scale"]))
    if p.paged:
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, page_table=upload(x["page_table"]),
                                 page_size=p.page_size, num_pages=x["k_pages"].shape[0], **kw)
        k, v = upload(x["k_pages"]), upload(x["v_pages"])
    else:
        prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, **kw)
        k, v = upload(x["k"]), upload(x["v"])
    return StemPrefill(prob, dev), upload(x["q"]), k, v


def _fused_vs_two_stage(p, x, dev):
    """Masks and counts from stem_score + stem_tpd_topk and from stem_score_select on the same inputs."""
    L, q, k, v = _layer(p, x, dev)
    rho, mu = (p.rho_num, p.rho_den), (p.mu_num, p.mu_den)
    L.score(q, k, v, p.beta)
    L.select(rho, mu)
    m1, c1 = L.mask.clone(), L.counts.clone()
    L.mask.fill_(-1)
    L.counts.fill_(-1)
    L.ws.zero_()
    L.score_select(q, k, v, p.beta, rho, mu)
    torch.cuda.synchronize()
    return L, m1, c1


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_fused_score_select_equals_two_stage(dev, name, over):
    p = synth.make_problem(name, **over)
    x = synth.make_inputs(p, seed=0)
    L, m1, c1 = _fused_vs_two_stage(p, x, dev)
    assert torch.equal(L.mask, m1) and torch.equal(L.counts, c1)


def test_fused_score_select_matches_oracle(dev):
    p = synth.make_problem("llama_32k_bf16", lens=(1500, 700), hq=8, hkv=2)
    x = synth.make_inputs(p, seed=9)
    ref1 = sc.oracle_stage1(p, x)
    S_list = [s for *_, s in ref1]
    budgets = sc.oracle_budgets(p)
    L, _, _ = _fused_vs_two_stage(p, x, dev)
    sc.check_selection(p, S_list, budgets, L.mask.cpu().numpy().view(np.uint32), L.counts.cpu().numpy())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama_32k_bf16", "llama_128k_bf16", "w8a8_128k_fp8", "paged_ragged_bf16"])
def test_fused_score_select_full_size(dev, name):
    p = synth.make_problem(name)
    _log(f"[fused] {name}")
    x = synth.make_inputs(p, seed=0)
    L, m1, c1 = _fused_vs_two_stage(p, x, dev)
    assert torch.equal(L.mask, m1) and torch.equal(L.counts, c1)


def test_scoring_beyond_2048_blocks_and_batch_independence(dev):
    """stem_score has no 2048-block limit (only the fused selection and masked attention do): a batch whose
    longest request has 2100 blocks, every score against the oracle; and its second request, scored again
    alone, gives the same scores bit for bit (a request's scores do not depend on its batch)."""
    p = synth.make_problem("llama_32k_bf16", lens=(2100 * 64, 1000 * 64 - 7), hq=2, hkv=1, d=64, block=64)
    x = synth.make_inputs(p, seed=3)
    L, q, k, v = _layer(p, x, dev)
    L.scores.fill_(float("nan"))
    L.score(q, k, v, p.beta)
    torch.cuda.synchronize()
    qb, kb, M = L.pooled()
    g = {"qbar": qb.cpu().numpy(), "kbar": kb.cpu().numpy(), "M": M.cpu().numpy(), "scores": L.scores.cpu().numpy()}
    _log("[scores > 2048 blocks] oracle")
    _check_stage1(p, g, sc.oracle_stage1(p, x))
    t0 = p.lens[0]
    p2 = synth.make_problem("llama_32k_bf16", lens=(p.lens[1],), hq=2, hkv=1, d=64, block=64)
    x2 = dict(x, q=x["q"][t0:], k=x["k"][t0:], v=x["v"][t0:])
    L2, q2, k2, v2 = _layer(p2, x2, dev)
    L2.scores.fill_(float("nan"))
    L2.score(q2, k2, v2, p2.beta)
    torch.cuda.synchronize()
    n2, cb = p2.nblocks(0), p.cu_blocks[1]
    tri = torch.tril(torch.ones(n2, n2, dtype=torch.bool, device=dev))
    assert torch.equal(L2.scores[:, :n2, :n2][:, tri], L.scores[:, cb:cb + n2, :n2][:, tri])


# ------------------------------------------------------------------------------------ fp8: V expanded once
def _expanded_vs_per_visit(p, x, dev, dense=False):
    """Attention of an fp8 problem through bsa_prefill (V converted on every tile visit) and through
    bsa_prefill_ws (V expanded to bf16 once), on the GPU's own selection (or dense)."""
    L, q, k, v = _layer(p, x, dev)
    L.score(q, k, v, p.beta)
    L.select((p.rho_num, p.rho_den), (p.mu_num, p.mu_den))
    mask = None if dense else "selected"
    L.attend(q, k, v, mask, expand_v=False)
    o1, l1 = L.out.clone(), L.lse.clone()
    L.out.fill_(float("nan"))
    L.lse.fill_(float("nan"))
    L.bsa_ws.fill_(0xFF)
    L.attend(q, k, v, mask, expand_v=True)
    torch.cuda.synchronize()
    return L, v, o1, l1


FP8_CASES = [
    dict(lens=(1000,), hq=8, hkv=2),                                 # two heads per workgroup
    dict(lens=(700, 129), hq=3, hkv=1),                              # one head per workgroup
    dict(lens=(300, 700), hq=4, hkv=2, paged=True, page_size=64),    # pages of 64 tokens
    dict(lens=(129, 500), hq=8, hkv=2, paged=True, page_size=32),    # smaller pages
    dict(lens=(1, 65, 128, 200), hq=2, hkv=1),                       # requests shorter than a sub-tile
]


@pytest.mark.parametrize("over", FP8_CASES, ids=[f"fp8-{i}" for i in range(len(FP8_CASES))])
@pytest.mark.parametrize("dense", [False, True], ids=["selected", "dense"])
def test_fp8_expanded_v_is_bit_identical_to_per_visit_conversion(dev, over, dense):
    """The bf16 expansion equals torch's e4m3fn decode, and the attention on it reproduces bsa_prefill's
    outputs and LSE bit for bit (both give the MFMAs the same bf16 V tile)."""
    p = synth.make_problem("w8a8_128k_fp8", **over)
    x = synth.make_inputs(p, seed=4)
    L, v, o1, l1 = _expanded_vs_per_visit(p, x, dev, dense)
    assert L.bsa_ws.numel() == 2 * v.numel()
    dec = v.view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16).flatten()
    assert torch.equal(L.bsa_ws.view(torch.int16), dec)
    assert torch.equal(L.out.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(L.lse, l1)


@pytest.mark.timeout(600)
def test_fp8_expanded_v_full_size_128k(dev):
    p = synth.make_problem("w8a8_128k_fp8")
    _log("[fp8 expanded V] w8a8_128k_fp8")
    x = synth.make_inputs(p, seed=0)
    L, v, o1, l1 = _expanded_vs_per_visit(p, x, dev)
    assert torch.equal(L.out.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(L.lse, l1)


@pytest.mark.parametrize("hq,hkv", [(3, 3), (2, 1)], ids=["one-head-per-workgroup", "two-heads-per-workgroup"])
def test_fused_score_select_beyond_1024_blocks(dev, hq, hkv):
    """Rows of 1025-2048 blocks take the fused kernel's widest register layout (32 slots per lane), with one
    query head per workgroup (odd group size) or two: masks and counts equal to the two-stage path's, and
    every budget and selection against the oracle."""
    p = synth.make_problem("llama_32k_bf16", lens=(1300 * 64 - 5,), hq=hq, hkv=hkv, d=64, block=64)
    x = synth.make_inputs(p, seed=12)
    L, m1, c1 = _fused_vs_two_stage(p, x, dev)
    assert torch.equal(L.mask, m1) and torch.equal(L.counts, c1)
    ref1 = sc.oracle_stage1(p, x)
    sc.check_selection(p, [s for *_, s in ref1], sc.oracle_budgets(p), L.mask.cpu().numpy().view(np.uint32),
                       L.counts.cpu().numpy())


# ------------------------------------------------------------------------------------ naive comparison path
def _naive_gpu(p, x, dev, samples):
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd import _abi
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype)
    q, k, v = upload(x["q"]), upload(x["k"]), upload(x["v"])
    L = StemPrefill(prob, dev)
    nws = torch.empty(_abi.naive_workspace_bytes(prob, samples), dtype=torch.uint8, device=dev)
    L.scores.fill_(float("nan"))
    _abi.stem_naive_score(prob, q, k, v, p.beta, samples, L.scores, L.ws, nws)
    L.select((p.rho_num, p.rho_den), (p.mu_num, p.mu_den))
    torch.cuda.synchronize()
    del nws
    return L


@pytest.mark.parametrize("lens,hq,hkv,d,block,samples", [
    ((1000,), 4, 2, 128, 128, 4), ((300, 1, 129, 700), 4, 4, 128, 128, 1),
    ((777,), 8, 1, 64, 64, 8), ((2000,), 2, 1, 128, 128, 128), ((640, 513), 4, 2, 128, 64, 16)])
def test_naive_scores_match_oracle(dev, lens, hq, hkv, d, block, samples):
    """The naive token-level scores (sampled queries, softmax, block mass) against the oracle's, and the
    TPD selection made from them."""
    p = synth.make_problem("llama_32k_bf16", lens=lens, hq=hq, hkv=hkv, d=d, block=block)
    x = synth.make_inputs(p, seed=21)
    L = _naive_gpu(p, x, dev, samples)
    gs = L.scores.cpu().numpy()
    cb = p.cu_blocks
    S_list = []
    worst = 0.0
    for r, (a, b) in enumerate(sc.request_slices(p)):
        q = sc.decode_q(p, x, a, b)
        k = sc.decode_kv(p, x, r, "k")
        v = sc.decode_kv(p, x, r, "v")
        S = oracle.naive_block_scores(q, k, v, p.block, p.beta, samples)
        n = S.shape[1]
        tri = np.tril(np.ones((n, n), dtype=bool))
        worst = max(worst, float(np.max(np.abs(gs[:, cb[r]:cb[r + 1], :n][:, tri] - S[:, tri]))))
        S_list.append(S)
    _log(f"[naive] {lens} samples {samples}: max abs score error {worst:.2e}")
    assert worst < 2e-4
    sc.check_selection(p, S_list, sc.oracle_budgets(p), L.mask.cpu().numpy().view(np.uint32),
                       L.counts.cpu().numpy())


@pytest.mark.timeout(600)
def test_naive_scores_full_size_32k_sampled_rows(dev):
    """At the 32K workload (4 samples per block) on sampled rows: each checked row's scores against the
    oracle's."""
    p = synth.make_problem("llama_32k_bf16")
    x = synth.make_inputs(p, seed=0)
    L = _naive_gpu(p, x, dev, 4)
    gs = L.scores.cpu().numpy()
    q = sc.decode_q(p, x, 0, p.lens[0])
    k = sc.decode_kv(p, x, 0, "k")
    v = sc.decode_kv(p, x, 0, "v")
    rows = [(0, 0), (3, 17), (9, 128), (17, 200), (31, 255), (30, 254)]
    S = oracle.naive_block_scores(q, k, v, p.block, p.beta, 4, rows=rows)
    for h, i in rows:
        err = np.max(np.abs(gs[h, i, : i + 1] - S[h, i, : i + 1]))
        assert err < 2e-4, (h, i, err)


# ------------------------------------------------------------------------------------ in-loop skip variant
def _inloop_vs_list(p, x, dev, mask_dev=None):
    """Run bsa_prefill and bsa_prefill_inloop on the same mask (the GPU's own selection by default);
    return (list out, list lse, in-loop out, in-loop lse) as device tensors."""
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload
    import block_sparse_attention_oam_amd as stem

    prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype)
    k, v, q = upload(x["k"]), upload(x["v"]), upload(x["q"])
    L = StemPrefill(prob, dev)
    L.score(q, k, v, p.beta)
    L.select((p.rho_num, p.rho_den), (p.mu_num, p.mu_den))
    m = L.mask if mask_dev is None else mask_dev
    L.attend(q, k, v, m)
    o1, l1 = L.out.clone(), L.lse.clone()
    L.out.fill_(7.0)
    L.lse.fill_(7.0)
    L.attend(q, k, v, m, inloop=True)
    torch.cuda.synchronize()
    return L, o1, l1, L.out.clone(), L.lse.clone()


@pytest.mark.parametrize("lens,hq,hkv,rho", [((1000,), 8, 2, 25), ((300, 1, 129, 700), 4, 4, 10),
                                             ((2000,), 4, 1, 100)])
def test_inloop_variant_equals_list_variant_and_oracle(dev, lens, hq, hkv, rho):
    """The skip test inside the loop visits the same blocks in the same order: outputs are identical to
    bsa_prefill's, and both match the oracle."""
    p = synth.make_problem("llama_32k_bf16", lens=lens, hq=hq, hkv=hkv, rho_num=rho)
    x = synth.make_inputs(p, seed=11)
    L, o1, l1, o2, l2 = _inloop_vs_list(p, x, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cb = p.cu_blocks
    words = L.mask.cpu().numpy().view(np.uint32)
    gm = [sc.unpack_mask(words[:, cb[r]:cb[r + 1]], p.nblocks(r)) & np.tril(np.ones((p.nblocks(r),) * 2, bool))[None]
          for r in range(len(p.lens))]
    ora = sc.oracle_attention(p, x, gm)
    mx, mean, lerr = sc.compare_attention(p, ora, o2.float().cpu().numpy().astype(np.float64),
                                          l2.cpu().numpy().astype(np.float64))
    assert mx <= 2e-2 and mean <= 2e-3 and lerr <= sc.LSE_TOL


def test_inloop_variant_external_mask_with_empty_rows(dev):
    p = synth.make_problem("llama_32k_bf16", lens=(900, 260), hq=4, hkv=2)
    x = synth.make_inputs(p, seed=3)
    rng = np.random.default_rng(12)
    NB = sum(p.nblocks(r) for r in range(len(p.lens)))
    words = rng.integers(0, 2 ** 32, size=(p.hq, NB, 1), dtype=np.uint64).astype(np.uint32)
    words[0] = 0          # head 0: every row empty
    words[2] = 0xFFFFFFFF  # head 2: dense plus bits past the diagonal
    from block_sparse_attention_oam_amd.layer import upload

    _, o1, l1, o2, l2 = _inloop_vs_list(p, x, dev, upload(words.view(np.int32)))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.timeout(600)
def test_inloop_variant_full_size_128k(dev):
    p = synth.make_problem("llama_128k_bf16")
    _log("[inloop] 128K: generating inputs")
    x = synth.make_inputs(p, seed=0)
    _, o1, l1, o2, l2 = _inloop_vs_list(p, x, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------------------------ ablation switches
ABLATIONS = [dict(mu_num=1, mu_den=1), dict(beta=0.0), dict(beta=0.0, mu_num=1, mu_den=1),
             dict(beta=0.8, mu_num=1, mu_den=2)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("over", ABLATIONS, ids=["uniform_mu1", "beta0", "uniform_beta0", "beta0.8_mu0.5"])
def test_ablation_switches_full_size_32k(dev, over):
    """The pages' ablations (uniform budget, routing-only score) at the 32K workload: every budget and
    selection against the oracle, attention on sampled rows."""
    p = synth.make_problem("llama_32k_bf16", **over)
    _log(f"[ablation] {over}")
    x = synth.make_inputs(p, seed=0)
    ref1 = sc.oracle_stage1(p, x)
    S_list = [s for *_, s in ref1]
    budgets = sc.oracle_budgets(p)
    if p.mu_num == p.mu_den:
        b = budgets[0]
        uncapped = b < np.arange(1, len(b) + 1)
        assert np.ptp(b[uncapped]) <= 1  # uniform: every uncapped row gets the same budget up to rounding
    masks = sc.oracle_masks(S_list, budgets)
    g = _run(p, x, dev, masks_for_bsa=masks)
    worst = _check_stage1(p, g, ref1)
    ties = sc.check_selection(p, S_list, budgets, g["words"], g["counts"])
    rows = [sc.sample_rows(p, 0, 8, mask=masks[0])]
    ora = sc.oracle_attention(p, x, masks, rows)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"], rows)
    _log(f"  score rel {worst:.2e}, near-tie rows {ties}, out max {mx:.2e} mean {mean:.2e}, lse {lerr:.2e}")
    tmax, tmean = sc.TOL[p.dtype]
    assert mx <= tmax and mean <= tmean and lerr <= sc.LSE_TOL


# ------------------------------------------------------------------------------------ maximum sizes
@pytest.mark.timeout(900)
def test_longest_request_the_masked_kernels_take(dev):
    """2048 blocks in one request (262144 tokens, the masked attention kernels' limit), 2 query heads: every
    budget and selection against the oracle, attention on sampled rows, and the fused selection equal to
    the two-stage one."""
    p = synth.make_problem("llama_128k_bf16", lens=(2048 * 128,), hq=2, hkv=1)
    _log("[max] 2048 blocks: generating inputs")
    x = synth.make_inputs(p, seed=6)
    ref1 = sc.oracle_stage1(p, x)
    S_list = [s for *_, s in ref1]
    budgets = sc.oracle_budgets(p)
    masks = sc.oracle_masks(S_list, budgets)
    g = _run(p, x, dev, masks_for_bsa=masks)
    _check_stage1(p, g, ref1)
    ties = sc.check_selection(p, S_list, budgets, g["words"], g["counts"])
    rows = [sc.sample_rows(p, 0, 6, mask=masks[0])]
    ora = sc.oracle_attention(p, x, masks, rows)
    mx, mean, lerr = sc.compare_attention(p, ora, g["out"], g["lse"], rows)
    _log(f"[max] near-tie rows {ties}, out max {mx:.2e} mean {mean:.2e}, lse {lerr:.2e}")
    assert mx <= 2e-2 and mean <= 2e-3 and lerr <= sc.LSE_TOL
    L, m1, c1 = _fused_vs_two_stage(p, x, dev)
    assert torch.equal(L.mask, m1) and torch.equal(L.counts, c1)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama_128k_bf16", "w8a8_128k_fp8"], ids=["bf16", "fp8"])
def test_dense_mode_beyond_16384_blocks(dev, name):
    """Dense causal attention (no mask) of one request of 16400 blocks (2,099,200 tokens), two query heads
    of one KV head: the rows of blocks 16383, 16384 and 16399, which see keys in blocks past 2^14, against
    the oracle.  (Masked calls stop at 2048 blocks; the dense walk has no such limit.)"""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    p = synth.make_problem(name, lens=(16400 * 128,), hq=2, hkv=1)
    _log(f"[dense 16400 blocks] {name}: generating inputs")
    x = synth.make_inputs(p, seed=8)
    kw = {}
    if p.dtype == "fp8":
        kw = dict(q_scale=upload(x["q_scale"]), k_scale=upload(x["k_scale"]), v_scale=upload(x["v_scale"]))
    prob = stem.make_problem(p.cu_seqlens, p.hq, p.hkv, p.d, p.block, p.dtype, **kw)
    q, k, v = upload(x["q"]), upload(x["k"]), upload(x["v"])
    L = StemPrefill(prob, dev)
    _log(f"[dense 16400 blocks] {name}: GPU run")
    L.attend(q, k, v, mask=None)
    torch.cuda.synchronize()
    rows = [(0, 16383), (1, 16384), (0, 16399), (1, 16399)]
    out = np.empty(L.out.shape, dtype=np.float64)
    lse = np.full(L.lse.shape, np.nan)
    for h, i in rows:
        sl = slice(i * p.block, (i + 1) * p.block)
        out[sl, h] = L.out[sl, h].float().cpu().numpy()
        lse[h, sl] = L.lse[h, sl].cpu().numpy()
    del q, k, v, L
    torch.cuda.empty_cache()
    n = p.nblocks(0)
    _log(f"[dense 16400 blocks] {name}: oracle rows")
    ora = sc.oracle_attention(p, x, [np.broadcast_to(np.bool_(True), (p.hq, n, n))], [rows])
    mx, mean, lerr = sc.compare_attention(p, ora, out, lse, [rows])
    _log(f"  out max {mx:.2e} mean {mean:.2e} lse {lerr:.2e}")
    tmax, tmean = sc.TOL[p.dtype]
    assert mx <= tmax and mean <= tmean and lerr <= sc.LSE_TOL


# ------------------------------------------------------------------------------------ budgets on the device
BUDGET_SWEEP = [(n, rho, mu) for n in (1, 2, 3, 5, 12, 31, 32, 33, 64, 65, 100, 255, 256, 1000, 1024, 2048, 4096)
                for rho in ((25, 100), (10, 100), (50, 100), (100, 100), (1, 100), (1, 3))
                for mu in ((7, 10), (1, 1), (1, 2), (1, 100))]


def test_device_budgets_and_exact_ties_match_oracle(dev):
    """stem_tpd_topk on all-equal scores: counts are the TPD budgets (exact integers) and every row selects
    its k lowest block indices (ties go to the lower index).  Ragged batches exercise per-request plans."""
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import upload

    groups = {}
    for n, rho, mu in BUDGET_SWEEP:
        groups.setdefault((rho, mu), []).append(n)
    for (rho, mu), ns in groups.items():
        for batch in (ns[:9], ns[9:]):
            lens = [64 * n for n in batch]
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            prob = stem.make_problem(cu, 1, 1, 64, 64, "f32")
            NB, mx = stem.block_counts(prob)
            W = (mx + 31) // 32
            scores = torch.zeros((1, NB, mx), dtype=torch.float32, device=dev)
            mask = torch.full((1, NB, W), -1, dtype=torch.int32, device=dev)
            counts = torch.zeros((1, NB), dtype=torch.int32, device=dev)
            stem.stem_tpd_topk(prob, scores, rho, mu, mask, counts)
            torch.cuda.synchronize()
            c = counts.cpu().numpy()[0]
            words = mask.cpu().numpy()[0].view(np.uint32)
            off = 0
            for n in batch:
                ref = oracle.tpd_budgets(n, *rho, *mu)
                assert np.array_equal(c[off:off + n], ref), (n, rho, mu)
                bits = sc.unpack_mask(words[off:off + n], W * 32)
                want = np.arange(W * 32)[None, :] < ref[:, None]
                assert np.array_equal(bits, want), (n, rho, mu)
                off += n
