"""One attention layer's Stem prefill: allocates device buffers with torch and calls the three C entry points.

torch is used only for device memory and the stream; all arithmetic runs in libstem.so's kernels.
"""
from __future__ import annotations

import torch

from . import _abi


def upload(arr, device="cuda"):
    """Host NumPy array (float32 / uint16 bf16 bits / uint8 fp8 codes / int32) -> device tensor, same bytes."""
    import numpy as np

    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class StemPrefill:
    """Buffers and calls of one layer.  q/k/v are device tensors in the library's layouts."""

    def __init__(self, problem: _abi.Problem, device="cuda"):
        self.p = problem
        c = problem.c
        self.NB, self.max_n = _abi.block_counts(problem)
        self.tokens = int(problem.cu_seqlens[-1])
        self.words = (self.max_n + 31) // 32
        self.device = device
        self.ws = torch.empty(_abi.workspace_bytes(problem), dtype=torch.uint8, device=device)
        self.scores = torch.empty((c.hq, self.NB, self.max_n), dtype=torch.float32, device=device)
        self.mask = torch.empty((c.hq, self.NB, self.words), dtype=torch.int32, device=device)
        self.counts = torch.empty((c.hq, self.NB), dtype=torch.int32, device=device)
        out_dtype = torch.float32 if c.dtype == _abi.DTYPES["f32"] else torch.bfloat16
        self.out = torch.empty((self.tokens, c.hq, c.head_dim), dtype=out_dtype, device=device)
        self.lse = torch.empty((c.hq, self.tokens), dtype=torch.float32, device=device)
        # attention workspace: V's bf16 expansion for fp8 problems, empty otherwise
        self.bsa_ws = torch.empty(_abi.bsa_workspace_bytes(problem), dtype=torch.uint8, device=device)

    def pooled(self):
        """Views of the workspace: (qbar [hq][NB][d], kbar [hkv][NB][d], M [hkv][NB])."""
        c = self.p.c
        oq, ok, om = _abi.workspace_layout(self.p)
        f = self.ws.view(torch.float32) if self.ws.numel() % 4 == 0 else None
        qb = f[oq // 4: oq // 4 + c.hq * self.NB * c.head_dim].view(c.hq, self.NB, c.head_dim)
        kb = f[ok // 4: ok // 4 + c.hkv * self.NB * c.head_dim].view(c.hkv, self.NB, c.head_dim)
        M = f[om // 4: om // 4 + c.hkv * self.NB].view(c.hkv, self.NB)
        return qb, kb, M

    def score(self, q, k, v, beta=0.2, stream=None):
        _abi.stem_score(self.p, q, k, v, beta, self.scores, self.ws, stream)

    def select(self, rho=(25, 100), mu=(7, 10), stream=None):
        _abi.stem_tpd_topk(self.p, self.scores, rho, mu, self.mask, self.counts, stream)

    def score_select(self, q, k, v, beta=0.2, rho=(25, 100), mu=(7, 10), stream=None):
        """Pooling, scoring and selection fused (no score tensor); fills mask and counts."""
        _abi.stem_score_select(self.p, q, k, v, beta, rho, mu, self.mask, self.counts, self.ws, stream)

    def attend(self, q, k, v, mask="selected", lse=True, softmax_scale=0.0, stream=None, inloop=False,
               expand_v=True):
        """inloop=True runs the comparison variant that tests the mask inside the loop.  fp8 problems run
        bsa_prefill_ws (V expanded to bf16 once per call) unless expand_v=False (bsa_prefill: V converted
        per tile visit); the outputs are the same."""
        m = self.mask if isinstance(mask, str) and mask == "selected" else mask
        lse_t = self.lse if lse else None
        if inloop:
            _abi.bsa_prefill_inloop(self.p, q, k, v, m, self.out, lse_t, softmax_scale, stream)
        elif expand_v and self.bsa_ws.numel() > 0:
            _abi.bsa_prefill_ws(self.p, q, k, v, m, self.out, lse_t, softmax_scale, self.bsa_ws, stream)
        else:
            _abi.bsa_prefill(self.p, q, k, v, m, self.out, lse_t, softmax_scale, stream)

    def forward(self, q, k, v, beta=0.2, rho=(25, 100), mu=(7, 10), stream=None, fused=True):
        """Score, select, attend.  fused: scoring and selection in one kernel (no score tensor; the same
        masks) where the library supports it (up to 2048 blocks per request), else the two stages."""
        if fused and self.max_n <= 2048:
            self.score_select(q, k, v, beta, rho, mu, stream)
        else:
            self.score(q, k, v, beta, stream)
            self.select(rho, mu, stream)
        self.attend(q, k, v, "selected", True, 0.0, stream)
        return self.out
