"""The no-allocation scoring entry point (stem_score_noalloc: pooled tensors in the library's static
per-device scratch) against stem_score with a caller workspace, through the C ABI: the same kernels, so
the block scores must be identical, on consecutive calls whose later problems are smaller than the first
(the scratch keeps the previous call's contents)."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CALLS = [
    ("llama_32k_bf16", {}),                                                  # 32 heads x 256 blocks
    ("paged_ragged_bf16", dict(lens=(300, 64, 700), hq=4, hkv=2, dtype="fp8")),  # smaller, paged fp8
    ("llama_32k_bf16", dict(lens=(300, 1, 129, 700), hq=4, hkv=4)),          # smaller, ragged
]


def test_noalloc_scoring_equals_workspace_scoring_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_oam_amd as stem
    from block_sparse_attention_oam_amd.layer import StemPrefill, upload

    dev = torch.device("cuda:0")
    for name, over in CALLS:
        p = synth.make_problem(name, **over)
        _log(f"[no-alloc] {name} {over}")
        x = synth.make_inputs(p, seed=13)
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
        q = upload(x["q"])
        L = StemPrefill(prob, dev)
        L.scores.fill_(float("nan"))
        L.score(q, k, v, p.beta)
        ref = L.scores.clone()
        L.scores.fill_(float("nan"))
        stem.stem_score_noalloc(prob, q, k, v, p.beta, L.scores)
        torch.cuda.synchronize()
        for r in range(len(p.lens)):
            n = p.nblocks(r)
            if n == 0:
                continue
            tri = torch.tril(torch.ones(n, n, dtype=torch.bool, device=dev))
            sl = slice(int(p.cu_blocks[r]), int(p.cu_blocks[r + 1]))
            a = ref[:, sl, :n][:, tri]
            b = L.scores[:, sl, :n][:, tri]
            assert not torch.isnan(a).any()
            assert torch.equal(a, b), (name, over, r)
        _log(f"  {p.hq} heads, {L.NB} blocks: scores identical")
