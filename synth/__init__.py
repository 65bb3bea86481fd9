"""Seeded synthetic inputs for the Stem prefill path (shared by the oracle tests and the GPU path).

This module only *draws* inputs and stores them in the byte formats the library reads (fp32, bf16, OCP
fp8 e4m3fn plus per-head fp32 scales, contiguous or paged KV).  It holds none of the method's arithmetic:
no pooling, scoring, budgets, selection or attention.

Distributions (the workloads of "Tencent Hunyuan Stem", page developer.cloud.tencent.cn/article/2709440,
sections "HPC-Stem" and "HPC-BSA": 128K-context prefill of an FP8 production model; shapes follow a
Llama-3-8B attention layer):

* Q and K rows: N(0, 1)/sqrt(8) per coordinate, plus a shared rank-4 component R_g[t] = z_{g,t} U_g^T added
  to KV head g and to every query head of group g.  U_g (d x 4) has orthonormal columns (QR of a Gaussian
  matrix); z_{g,t} is an AR(1) process along the tokens of each request with unit stationary variance and
  phi = exp(-1/256), so the shared direction survives block mean-pooling.
* V rows: v_t = lambda_t * eps_t with eps ~ N(0, I_d), lambda_t ~ LogNormal(0, 0.5) per (token, KV head).
* Sinks (when enabled): K rows at positions 0..3 of every request and KV head are set to 16 * U_g[:, 0].
* bf16 rounding is round-to-nearest-even of the fp32 draws.  fp8 inputs quantise the bf16 values per head
  with scale = amax|x| / 448 and round-to-nearest-even e4m3fn codes (saturating at +-448).
* Paged KV: 64-token pages; physical pages are placed by a seeded permutation, and request r's logical page
  p maps to perm[sum of earlier requests' page counts + p].

Draw order from numpy's default_rng(SeedSequence(seed)): Q, K, V eps, V lambda, U (all groups), AR(1)
innovations (all groups, packed tokens), page permutation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.signal import lfilter

__all__ = ["Problem", "CONFIGS", "make_problem", "make_inputs", "bf16_bits", "e4m3fn_encode"]


@dataclass(frozen=True)
class Problem:
    """Shape and method parameters of one workload (plain data)."""

    name: str
    lens: tuple
    hq: int
    hkv: int
    d: int
    block: int
    dtype: str  # "f32" | "bf16" | "fp8"
    sinks: bool = True
    paged: bool = False
    page_size: int = 64
    rho_num: int = 25  # budget fraction rho = rho_num / rho_den of the causal blocks
    rho_den: int = 100
    mu_num: int = 7  # TPD end/start ratio mu = mu_num / mu_den
    mu_den: int = 10
    beta: float = 0.2

    @property
    def tokens(self) -> int:
        return int(sum(self.lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)

    def nblocks(self, r: int) -> int:
        return -(-int(self.lens[r]) // self.block)

    @property
    def cu_blocks(self) -> np.ndarray:
        nb = [self.nblocks(r) for r in range(len(self.lens))]
        return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)

    def with_(self, **kw) -> "Problem":
        d = dict(self.__dict__)
        d.update(kw)
        if "lens" in kw:
            d["lens"] = tuple(int(x) for x in kw["lens"])
        return Problem(**d)


# The five workloads: tiny fp32 MHA case, 32K and 128K bf16 GQA layers, fp8 128K layer, paged ragged batch.
CONFIGS = {
    "tiny_f32": Problem("tiny_f32", (2048,), 2, 2, 64, 64, "f32", sinks=False),
    "llama_32k_bf16": Problem("llama_32k_bf16", (32768,), 32, 8, 128, 128, "bf16"),
    "llama_128k_bf16": Problem("llama_128k_bf16", (131072,), 32, 8, 128, 128, "bf16"),
    "w8a8_128k_fp8": Problem("w8a8_128k_fp8", (131072,), 64, 8, 128, 128, "fp8"),
    "paged_ragged_bf16": Problem("paged_ragged_bf16", (8192, 32768, 65536, 131072), 32, 8, 128, 128,
                                 "bf16", paged=True, page_size=64),
}


def make_problem(name: str, **overrides) -> Problem:
    return CONFIGS[name].with_(**overrides) if overrides else CONFIGS[name]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Real values -> OCP e4m3fn codes (uint8), round to nearest even, saturating at +-448.

    e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6);
    0x7F/0xFF are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(y), 448.0)
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)  # floor(log2 a), clamped to the subnormal exponent
    quantum = np.ldexp(1.0, e - 3)
    m = np.rint(a / quantum)  # half to even
    val = m * quantum  # exactly representable in e4m3fn (or 2^(e+1), still representable)
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = (val > 0) & (e2 >= -6)
    mant_n = np.where(normal, val / np.ldexp(1.0, np.where(normal, e2, 0) - 3) - 8.0, 0.0)
    code_n = ((e2 + 7) << 3).astype(np.int64) + mant_n.astype(np.int64)
    code_s = np.rint(val / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s).astype(np.uint8)
    return code | sign


def _ar1(innov: np.ndarray, phi: float) -> np.ndarray:
    """AR(1) along axis 0 with unit stationary variance: z_0 = e_0, z_t = phi z_{t-1} + sqrt(1-phi^2) e_t."""
    if innov.shape[0] == 0:  # an empty request
        return innov.astype(np.float64)
    c = math.sqrt(1.0 - phi * phi)
    z = lfilter([c], [1.0, -phi], innov.astype(np.float64), axis=0)
    # lfilter's first output is c*e_0; rescale the start so z_0 = e_0 (stationary start), then propagate.
    z0 = innov[0].astype(np.float64)
    # z_t(true) = z_t(lfilter) + phi^t (z0 - c e0)
    corr = z0 - c * innov[0].astype(np.float64)
    decay = phi ** np.arange(innov.shape[0], dtype=np.float64)
    z += decay[:, None] * corr[None, :]
    return z


def _draw_fp32(p: Problem, rng: np.random.Generator):
    T, hq, hkv, d = p.tokens, p.hq, p.hkv, p.d
    s8 = np.float32(1.0 / math.sqrt(8.0))
    q = rng.standard_normal((T, hq, d), dtype=np.float32)
    q *= s8
    k = rng.standard_normal((T, hkv, d), dtype=np.float32)
    k *= s8
    v = rng.standard_normal((T, hkv, d), dtype=np.float32)
    lam = rng.lognormal(0.0, 0.5, size=(T, hkv)).astype(np.float32)
    v *= lam[:, :, None]
    U = np.empty((hkv, d, 4), dtype=np.float64)
    for g in range(hkv):
        U[g] = np.linalg.qr(rng.standard_normal((d, 4)))[0]
    innov = rng.standard_normal((T, hkv * 4))
    phi = math.exp(-1.0 / 256.0)
    cu = p.cu_seqlens
    group = hq // hkv
    for r in range(len(p.lens)):
        a, b = int(cu[r]), int(cu[r + 1])
        z = _ar1(innov[a:b], phi).reshape(b - a, hkv, 4)
        for g in range(hkv):
            Rg = (z[:, g, :] @ U[g].T).astype(np.float32)  # [L, d]
            k[a:b, g, :] += Rg
            q[a:b, g * group:(g + 1) * group, :] += Rg[:, None, :]
            if p.sinks:
                ns = min(4, b - a)
                k[a:a + ns, g, :] = (16.0 * U[g][:, 0]).astype(np.float32)
    return q, k, v


def _quant_fp8_per_head(x: np.ndarray):
    """x [T][H][d] fp32 (bf16-valued) -> (codes uint8 [T][H][d], scale fp32 [H]), scale = amax/448 per head.

    The cast is torch's CPU float -> float8_e4m3fn conversion (round to nearest even); inputs are clamped
    to +-448 first, so its out-of-range behaviour never applies.
    """
    import torch

    H = x.shape[1]
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(H, dtype=np.float32)
    for h in range(H):
        xh = torch.from_numpy(np.ascontiguousarray(x[:, h, :]))
        amax = float(xh.abs().max())
        s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
        scale[h] = s
        y = (xh / torch.tensor(s, dtype=torch.float32)).clamp_(-448.0, 448.0)
        codes[:, h, :] = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _page(p: Problem, x: np.ndarray, perm: np.ndarray):
    """Scatter contiguous [T][H][d] rows into 64-token pages [P][ps][H][d] and build the page table."""
    ps = p.page_size
    npages = [-(-int(L) // ps) for L in p.lens]
    P = int(sum(npages))
    pages = np.zeros((P, ps) + x.shape[1:], dtype=x.dtype)
    table = np.full((len(p.lens), max(npages)), -1, dtype=np.int32)
    cu = p.cu_seqlens
    off = 0
    for r, L in enumerate(p.lens):
        for lp in range(npages[r]):
            phys = int(perm[off + lp])
            table[r, lp] = phys
            t0 = int(cu[r]) + lp * ps
            t1 = min(t0 + ps, int(cu[r + 1]))
            pages[phys, : t1 - t0] = x[t0:t1]
        off += npages[r]
    return pages, table


def make_inputs(p: Problem, seed: int = 0) -> dict:
    """Draw the inputs of problem `p` and return them in the library's storage formats.

    Keys: q, k, v (contiguous storage: float32 / uint16 bf16 bits / uint8 e4m3fn codes), q_scale,
    k_scale, v_scale (fp8 only, float32 per head), k_pages, v_pages, page_table (paged only),
    cu_seqlens (int32).
    """
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    q, k, v = _draw_fp32(p, rng)
    out = {"problem": p, "cu_seqlens": p.cu_seqlens}
    if p.dtype == "f32":
        out.update(q=q, k=k, v=v)
    elif p.dtype == "bf16":
        out.update(q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v))
    elif p.dtype == "fp8":
        out["q"], out["q_scale"] = _quant_fp8_per_head(_bf16_value(bf16_bits(q)))
        del q
        out["k"], out["k_scale"] = _quant_fp8_per_head(_bf16_value(bf16_bits(k)))
        out["v"], out["v_scale"] = _quant_fp8_per_head(_bf16_value(bf16_bits(v)))
    else:
        raise ValueError(f"unknown dtype {p.dtype}")
    if p.paged:
        npages = sum(-(-int(L) // p.page_size) for L in p.lens)
        perm = rng.permutation(npages)
        out["k_pages"], out["page_table"] = _page(p, out["k"], perm)
        out["v_pages"], _ = _page(p, out["v"], perm)
    return out
