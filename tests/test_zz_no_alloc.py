"""The allocation-free attention entry point (br_attn_fwd_noalloc) against br_attn_fwd.

Both run the same plan and kernels, so the outputs and log-sum-exps must agree bit for bit.
Two calls in a row share the library's one per-GPU workspace; the second is smaller, so
stale contents of the first call must not leak into it.  A table whose plan exceeds the
library's workspace is rejected on the host before any GPU work.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import workloads
from gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else \
        t.contiguous().view(torch.int32).cpu().numpy()


def _compare(w, what):
    log(f"[gpu] no-alloc {what}: T={w.total_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim}")
    dev = upload(w)
    ref, ref_lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True)
    out = torch.empty_like(dev["Q"])
    lse = torch.empty_like(ref_lse)
    br.attn_fwd_noalloc(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, out, lse=lse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(out), _bits(ref), err_msg=f"{what}: output")
    np.testing.assert_array_equal(_bits(lse), _bits(ref_lse), err_msg=f"{what}: lse")


def test_noalloc_matches_attn_fwd_twice_shrinking():
    # first call: the worked shape (several split-key chunks for the query rows); second: tiny
    _compare(workloads.make("worked", 0), "worked")
    _compare(workloads.make("tiny", 1), "tiny after worked")


def test_noalloc_rejects_oversized_plan():
    # a batch whose split-key partials exceed the scratch size
    prompts = [(32, [128] * 100, 32)] * 16
    so, sp, _, _ = workloads.segment_tables(prompts)
    T = int(so[-1])
    dims = br.make_dims(len(prompts), 32, 8, 128, T)
    assert br.attn_workspace_bytes(dims, so, sp) > br.NOALLOC_SCRATCH_BYTES
    Q = torch.zeros((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((T, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(br.BlockRankError) as ei:
        br.attn_fwd_noalloc(Q, K, K, so, sp, torch.empty_like(Q))
    assert ei.value.status == 2  # BR_ERR_UNSUPPORTED
