"""Host-side tests of the C-ABI library (no GPU): loading, exported symbols, the budget arithmetic shared
with the selection kernel, workspace sizing, and every argument-validation error path.

Calls here either touch no device memory (host helpers) or are built to fail validation, which happens on
the host before any HIP call; fake device addresses are never dereferenced.
"""
import ctypes
import os
import random
import re
import subprocess

import numpy as np
import pytest

import block_sparse_attention_oam_amd as stem
from block_sparse_attention_oam_amd import _abi
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stem.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_compiles_as_c99():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_plain_c_program_uses_the_abi(tmp_path):
    """A C99 program (tests/c_abi_consumer.c) compiled with gcc against the header, linked against the
    library: host-only entry points and host-side validation, called from C."""
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libstem.so is not built")
    exe = str(tmp_path / "c_abi_consumer")
    libdir = os.path.dirname(_abi.LIB_PATH)
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_consumer.c")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), src, "-L", libdir,
                        "-lstem", "-Wl,-rpath," + libdir, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer ok" in r.stdout


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(stem.EXPORTS)
    L = stem.lib()
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", stem.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared) <= exported


def _declared_prototypes():
    """{name: (return type text, [parameter type texts])} from the header (comments stripped)."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"^\s*((?:const\s+)?[a-z_0-9]+\s*\*?)\s*([a-z_0-9]+)\s*\(([^)]*)\)\s*;", src, flags=re.M):
        ret, name, params = m.group(1), m.group(2), m.group(3).strip()
        args = [] if params in ("", "void") else [a.strip() for a in params.split(",")]
        protos[name] = (re.sub(r"\s+", " ", ret).strip(), args)
    return protos


def _ctype_of(text):
    """The ctypes type a C parameter or return type must map to (pointers of any kind: void pointer or a
    ctypes pointer / structure pointer)."""
    t = re.sub(r"\b(const|struct)\b", "", text)
    if "*" in t:
        return "pointer"
    base = t.split()[0] if t.split() else t
    return {"int": ctypes.c_int, "int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "size_t": ctypes.c_size_t,
            "float": ctypes.c_float, "double": ctypes.c_double}[base]


def test_binding_signatures_match_the_header():
    """Every declared function: the binding's argument count and the scalar argument and return types agree
    with the prototype (pointer parameters are pointers on both sides)."""
    protos = _declared_prototypes()
    assert set(protos) == set(stem.EXPORTS)
    L = stem.lib()
    for name, (ret, args) in protos.items():
        f = getattr(L, name)
        assert len(f.argtypes) == len(args), (name, len(f.argtypes), args)
        for want_text, got in zip(args, f.argtypes):
            want = _ctype_of(want_text.rsplit(" ", 1)[0] if " " in want_text and "*" not in want_text.rsplit(" ", 1)[1] else want_text)
            if want == "pointer":
                assert got is ctypes.c_void_p or issubclass(got, ctypes._Pointer) or got is ctypes.c_char_p, (name, want_text, got)
            else:
                assert ctypes.sizeof(got) == ctypes.sizeof(want) and got._type_ == want._type_, (name, want_text, got)
        want_ret = _ctype_of(ret)
        if want_ret == "pointer":
            assert f.restype in (ctypes.c_char_p, ctypes.c_void_p), (name, ret, f.restype)
        else:
            assert f.restype is not None and ctypes.sizeof(f.restype) == ctypes.sizeof(want_ret), (name, ret, f.restype)


def test_status_strings():
    L = stem.lib()
    for s, name in [(0, "STEM_OK"), (-1, "STEM_E_INVALID_ARG"), (-2, "STEM_E_UNSUPPORTED"),
                    (-3, "STEM_E_WORKSPACE"), (-4, "STEM_E_HIP")]:
        assert L.stem_status_string(s).decode() == name


@pytest.mark.parametrize("n", [1, 2, 3, 5, 16, 32, 64, 100, 256, 511, 1024])
@pytest.mark.parametrize("rho", [(0, 1), (1, 100), (10, 100), (25, 100), (50, 100), (1, 1), (2, 7)])
@pytest.mark.parametrize("mu", [(7, 10), (1, 1), (1, 2), (1, 100), (699, 1000)])
def test_budget_arithmetic_matches_oracle(n, rho, mu):
    got = stem.stem_tpd_budgets_host(n, *rho, *mu)
    ref = oracle.tpd_budgets(n, *rho, *mu)
    assert np.array_equal(got, ref)


def test_budget_arithmetic_random_sweep():
    rnd = random.Random(7)
    for _ in range(150):
        n = rnd.randint(1, 900)
        rho = (rnd.randint(0, 100), 100)
        mu = (rnd.randint(1, 20), 20)
        assert np.array_equal(stem.stem_tpd_budgets_host(n, *rho, *mu), oracle.tpd_budgets(n, *rho, *mu))


def test_budget_argument_errors():
    for args in [(0, 1, 4, 7, 10), (8, -1, 4, 7, 10), (8, 5, 4, 7, 10), (8, 1, 0, 7, 10), (8, 1, 4, 0, 10),
                 (8, 1, 4, 11, 10), (8, 1, 4, 7, 0), (40000, 1, 4, 7, 10 ** 6)]:
        with pytest.raises(stem.StemError) as e:
            stem.stem_tpd_budgets_host(*args)
        assert e.value.status in (_abi.STEM_E_INVALID_ARG, _abi.STEM_E_UNSUPPORTED)


# ------------------------------------------------------------------------------------------------ problems
def _prob(**kw):
    base = dict(cu_seqlens=[0, 1000, 3000], hq=8, hkv=2, head_dim=128, block=128, dtype="bf16")
    base.update(kw)
    return stem.make_problem(**base)


def test_block_counts_and_workspace_layout():
    p = _prob()
    nb, mx = stem.block_counts(p)
    assert (nb, mx) == (8 + 16, 16)
    oq, ok, om = stem.workspace_layout(p)
    qb = 8 * nb * 128 * 4
    kb = 2 * nb * 128 * 4
    mb = 2 * nb * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert (oq, ok, om) == (0, al(qb), al(qb) + al(kb))
    assert stem.workspace_bytes(p) == al(qb) + al(kb) + al(mb)
    p64 = _prob(cu_seqlens=[0, 65], block=64, head_dim=64, dtype="f32", hq=2, hkv=2)
    assert stem.block_counts(p64) == (2, 2)


class _FakeTensor:
    """Stands in for a device tensor in calls that must fail validation: address and shape only."""

    def __init__(self, addr=0x10000, shape=(1,), elem=4):
        self._a, self.shape, self._e = addr, shape, elem

    def data_ptr(self):
        return self._a

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return self._e


BAD_PROBLEMS = [
    (dict(cu_seqlens=[0]), "num_reqs"),
    (dict(cu_seqlens=[1, 10]), "cu_seqlens[0]"),
    (dict(cu_seqlens=[0, 10, 5]), "decreases"),
    (dict(cu_seqlens=[0, 0]), "empty"),
    (dict(hq=6, hkv=4), "hq % hkv"),
    (dict(hq=0), "hq"),
    (dict(head_dim=96), "head_dim"),
    (dict(block=32), "block"),
    (dict(dtype=7), "dtype"),
    (dict(dtype="fp8"), "scale"),
    (dict(cu_seqlens=list(range(0, 258))), "num_reqs"),
]


@pytest.mark.parametrize("kw,msg", BAD_PROBLEMS)
def test_invalid_problem_is_rejected_by_every_entry_point(kw, msg):
    p = _prob(**kw)
    T = _FakeTensor
    calls = [
        lambda: stem.block_counts(p),
        lambda: stem.workspace_layout(p),
        lambda: stem.stem_score(p, T(), T(), T(), 0.2, T(shape=(1, 1, 64)), T(shape=(1 << 30,), elem=1), stream=0),
        lambda: stem.stem_score_noalloc(p, T(), T(), T(), 0.2, T(shape=(1, 1, 64)), stream=0),
        lambda: stem.stem_tpd_topk(p, T(shape=(1, 1, 64)), (1, 4), (7, 10), T(shape=(1, 1, 2)), T(), stream=0),
        lambda: stem.bsa_prefill(p, T(), T(), T(), None, T(), stream=0),
        lambda: _abi.bsa_prefill_inloop(p, T(), T(), T(), T(shape=(8, 24, 1)), T(), stream=0),
        lambda: stem.bsa_prefill_ws(p, T(), T(), T(), None, T(), ws=T(shape=(1 << 30,), elem=1), stream=0),
        lambda: stem.bsa_workspace_bytes(p),
        lambda: stem.stem_score_select(p, T(), T(), T(), 0.2, (1, 4), (7, 10), T(shape=(1, 1, 2)), T(),
                                       T(shape=(1 << 30,), elem=1), stream=0),
    ]
    for c in calls:
        with pytest.raises(stem.StemError) as e:
            c()
        assert e.value.status in (_abi.STEM_E_INVALID_ARG, _abi.STEM_E_UNSUPPORTED)
        assert msg in str(e.value)
    assert stem.lib().stem_workspace_bytes(p.ref) == 0


def test_paged_descriptor_errors():
    pt = _FakeTensor(shape=(2, 16))
    for kw, msg in [(dict(page_size=0), "page_size"), (dict(page_size=24), "page_size"),
                    (dict(page_size=64, num_pages=0), "num_pages"),
                    (dict(page_size=64, num_pages=10, page_table=_FakeTensor(shape=(2, 4))), "page_table_stride")]:
        args = dict(page_table=pt, num_pages=10)
        args.update(kw)
        p = _prob(**args)
        with pytest.raises(stem.StemError) as e:
            stem.block_counts(p)
        assert msg in str(e.value)


def test_call_argument_errors():
    p = _prob()  # NB = 24, max_n = 16
    T = _FakeTensor
    ws_need = stem.workspace_bytes(p)
    cases = [
        (lambda: stem.stem_score(p, T(), T(), T(), 0.2, T(shape=(8, 24, 15)), T(shape=(ws_need,), elem=1), stream=0),
         "score_row_stride"),
        (lambda: stem.stem_score(p, T(), T(), T(), 0.2, T(shape=(8, 24, 16)), T(shape=(ws_need - 1,), elem=1),
                                 stream=0), "workspace"),
        (lambda: stem.stem_score(p, T(addr=0x10008), T(), T(), 0.2, T(shape=(8, 24, 16)),
                                 T(shape=(ws_need,), elem=1), stream=0), "aligned"),
        (lambda: stem.stem_score(p, T(), T(), T(), float("nan"), T(shape=(8, 24, 16)), T(shape=(ws_need,), elem=1),
                                 stream=0), "beta"),
        (lambda: stem.stem_tpd_topk(p, T(shape=(8, 24, 16)), (1, 4), (7, 10), T(shape=(8, 24, 0)), T(), stream=0),
         "mask_row_words"),
        (lambda: stem.stem_tpd_topk(p, T(shape=(8, 24, 16)), (5, 4), (7, 10), T(shape=(8, 24, 1)), T(), stream=0),
         "rho"),
        (lambda: stem.stem_tpd_topk(p, T(shape=(8, 24, 16)), (1, 4), (0, 10), T(shape=(8, 24, 1)), T(), stream=0),
         "mu"),
        (lambda: stem.bsa_prefill(p, T(), T(), T(), T(shape=(8, 24, 0)), T(), stream=0), "mask_row_words"),
        (lambda: stem.bsa_prefill(p, T(), T(), T(), None, T(), softmax_scale=float("inf"), stream=0),
         "softmax_scale"),
        (lambda: stem.bsa_prefill(p, T(), T(), T(), None, None, stream=0), "non-NULL"),
    ]
    for c, msg in cases:
        with pytest.raises(stem.StemError) as e:
            c()
        assert msg in str(e.value), str(e.value)


def test_inloop_variant_argument_errors():
    """The in-loop skip comparison variant validates like bsa_prefill, needs a mask and supports only the
    main production shape."""
    from block_sparse_attention_oam_amd import _abi as A

    T = _FakeTensor
    p = _prob()
    with pytest.raises(stem.StemError) as e:
        A.bsa_prefill_inloop(p, T(), T(), T(), None, T(), stream=0)
    assert "needs a mask" in str(e.value)
    with pytest.raises(stem.StemError) as e:
        A.bsa_prefill_inloop(p, T(), T(), T(), T(shape=(8, 24, 0)), T(), stream=0)
    assert "mask_row_words" in str(e.value)
    for kw in (dict(dtype="f32"), dict(head_dim=64), dict(block=64),
               dict(dtype="fp8", q_scale=T(), k_scale=T(), v_scale=T())):
        q = _prob(**kw)
        nb, mx = stem.block_counts(q)
        with pytest.raises(stem.StemError) as e:
            A.bsa_prefill_inloop(q, T(), T(), T(), T(shape=(8, nb, (mx + 31) // 32)), T(), stream=0)
        assert e.value.status == A.STEM_E_UNSUPPORTED, (kw, str(e.value))


def test_score_select_argument_errors():
    """The fused scoring + selection entry point validates the union of stem_score's and stem_tpd_topk's
    arguments (no score tensor) and supports requests of up to 2048 blocks."""
    T = _FakeTensor
    p = _prob()  # NB = 24, max_n = 16
    need = stem.workspace_bytes(p)
    ws = T(shape=(need,), elem=1)
    ok = dict(q=T(), k=T(), v=T(), beta=0.2, rho=(1, 4), mu=(7, 10), mask=T(shape=(8, 24, 1)), counts=T(), ws=ws)
    cases = [
        (dict(q=None), "non-NULL"),
        (dict(mask=None), "non-NULL"),
        (dict(counts=None), "non-NULL"),
        (dict(ws=T(shape=(need - 1,), elem=1)), "workspace"),
        (dict(beta=float("nan")), "beta"),
        (dict(mask=T(shape=(8, 24, 0))), "mask_row_words"),
        (dict(rho=(5, 4)), "rho"),
        (dict(mu=(0, 10)), "mu"),
        (dict(v=T(addr=0x10008)), "aligned"),
    ]
    for kw, msg in cases:
        a = dict(ok)
        a.update(kw)
        with pytest.raises(stem.StemError) as e:
            stem.stem_score_select(p, a["q"], a["k"], a["v"], a["beta"], a["rho"], a["mu"], a["mask"], a["counts"],
                                   a["ws"], stream=0)
        assert msg in str(e.value), (kw, str(e.value))
    big = _prob(cu_seqlens=[0, 2049 * 128])
    nb, mx = stem.block_counts(big)
    with pytest.raises(stem.StemError) as e:
        stem.stem_score_select(big, T(), T(), T(), 0.2, (1, 4), (7, 10), T(shape=(8, nb, (mx + 31) // 32)), T(),
                               T(shape=(stem.workspace_bytes(big),), elem=1), stream=0)
    assert e.value.status == _abi.STEM_E_UNSUPPORTED


def test_noalloc_scoring_validation_and_scratch_limit():
    """stem_score_noalloc validates like stem_score and rejects, on the host, a problem whose pooled tensors
    exceed the static scratch (STEM_SCRATCH_BYTES in the header)."""
    T = _FakeTensor
    src = open(HEADER).read()
    m = re.search(r"#define STEM_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == _abi.SCRATCH_BYTES
    p = _prob()  # NB = 24, max_n = 16
    for call, msg in [
        (lambda: stem.stem_score_noalloc(p, T(), T(), T(), 0.2, T(shape=(8, 24, 15)), stream=0), "score_row_stride"),
        (lambda: stem.stem_score_noalloc(p, T(), T(), T(), float("nan"), T(shape=(8, 24, 16)), stream=0), "beta"),
        (lambda: stem.stem_score_noalloc(p, T(addr=0x10008), T(), T(), 0.2, T(shape=(8, 24, 16)), stream=0),
         "aligned"),
        (lambda: stem.stem_score_noalloc(p, None, T(), T(), 0.2, T(shape=(8, 24, 16)), stream=0), "non-NULL"),
    ]:
        with pytest.raises(stem.StemError) as e:
            call()
        assert msg in str(e.value), str(e.value)
    # 32 query / 8 KV heads, head_dim 128: 3271 blocks fit in 64 MiB, 3272 do not
    for nb, fits in ((3271, True), (3272, False)):
        q = _prob(cu_seqlens=[0, nb * 128], hq=32, hkv=8, head_dim=128, block=128)
        assert (stem.workspace_bytes(q) <= _abi.SCRATCH_BYTES) == fits
    big = _prob(cu_seqlens=[0, 3272 * 128], hq=32, hkv=8, head_dim=128, block=128)
    with pytest.raises(stem.StemError) as e:
        stem.stem_score_noalloc(big, T(), T(), T(), 0.2, T(shape=(32, 3272, 3272)), stream=0)
    assert e.value.status == _abi.STEM_E_UNSUPPORTED and "static scratch" in str(e.value)


def test_quantize_fp8_argument_errors():
    """The quantise-only entry point describes an fp8 layer with contiguous K/V and needs every buffer."""
    T = _FakeTensor
    f8 = dict(dtype="fp8", q_scale=T(), k_scale=T(), v_scale=T())
    p = _prob(**f8)
    args = [T() for _ in range(9)]
    with pytest.raises(stem.StemError) as e:
        stem.stem_quantize_fp8(_prob(), *args, stream=0)
    assert e.value.status == _abi.STEM_E_UNSUPPORTED
    with pytest.raises(stem.StemError) as e:
        stem.stem_quantize_fp8(_prob(page_table=T(shape=(2, 64)), page_size=64, num_pages=40, **f8), *args, stream=0)
    assert e.value.status == _abi.STEM_E_UNSUPPORTED
    for bad, msg in ((3, "non-NULL"), (7, "non-NULL")):
        a = list(args)
        a[bad] = None
        with pytest.raises(stem.StemError) as e:
            stem.stem_quantize_fp8(p, *a, stream=0)
        assert msg in str(e.value)
    a = list(args)
    a[4] = T(addr=0x10008)
    with pytest.raises(stem.StemError) as e:
        stem.stem_quantize_fp8(p, *a, stream=0)
    assert "aligned" in str(e.value)


def test_bsa_workspace_bytes_and_argument_errors():
    """bsa_prefill_ws needs 2 bytes per V element (the bf16 expansion) for fp8 at d = 128, B = 128 --
    contiguous: tokens x hkv x d, paged: the whole pool -- and no workspace otherwise; a missing, short or
    misaligned workspace is refused before anything is enqueued."""
    T = _FakeTensor
    f8 = dict(dtype="fp8", q_scale=T(), k_scale=T(), v_scale=T())
    p = _prob(**f8)
    need = 3000 * 2 * 128 * 2
    assert stem.bsa_workspace_bytes(p) == need
    pp = _prob(page_table=T(shape=(2, 64)), page_size=64, num_pages=70, **f8)
    assert stem.bsa_workspace_bytes(pp) == 70 * 64 * 2 * 128 * 2
    assert stem.bsa_workspace_bytes(_prob()) == 0
    assert stem.bsa_workspace_bytes(_prob(dtype="f32")) == 0
    assert stem.bsa_workspace_bytes(_prob(head_dim=64, **f8)) == 0
    for ws, status, msg in ((None, _abi.STEM_E_WORKSPACE, "workspace"),
                            (T(shape=(need - 1,), elem=1), _abi.STEM_E_WORKSPACE, "workspace"),
                            (T(addr=0x10008, shape=(need,), elem=1), _abi.STEM_E_INVALID_ARG, "aligned")):
        with pytest.raises(stem.StemError) as e:
            stem.bsa_prefill_ws(p, T(), T(), T(), None, T(), ws=ws, stream=0)
        assert e.value.status == status and msg in str(e.value), str(e.value)
    # the other checks of bsa_prefill come first
    with pytest.raises(stem.StemError) as e:
        stem.bsa_prefill_ws(p, T(), T(), T(), T(shape=(8, 24, 0)), T(), ws=None, stream=0)
    assert "mask_row_words" in str(e.value)


def test_last_error_is_cleared_by_a_successful_call():
    with pytest.raises(stem.StemError):
        stem.block_counts(_prob(hq=3, hkv=2))
    assert stem.lib().stem_last_error().decode() != ""
    stem.block_counts(_prob())
    assert stem.lib().stem_last_error().decode() == ""
