"""Stem sparse-attention prefill on AMD Instinct MI355X (gfx950): OAM block scoring, fused TPD top-k
selection and block-sparse flash attention, as a C-ABI library (libstem.so) with a thin Python binding."""
from ._abi import (  # noqa: F401
    DTYPES, EXPORTS, LIB_PATH, Problem, StemError, block_counts, bsa_prefill, lib, make_problem,
    stem_score, stem_score_select, stem_tpd_budgets_host, stem_tpd_topk, workspace_bytes, workspace_layout,
    bsa_prefill_inloop, stem_quantize_score, stem_naive_score, naive_workspace_bytes, stem_score_noalloc,
    stem_quantize_fp8, bsa_workspace_bytes, bsa_prefill_ws,
)
