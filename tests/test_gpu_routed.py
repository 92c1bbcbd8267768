"""GPU parity of top-B routed attention (br_attn_routed_fwd) against the fp64 oracle, on seeded
inputs, through the C ABI."""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import check_attn, dev_bf16, log, upload
from pins import random_prompts

pytestmark = pytest.mark.gpu


def _keep_lists(rng, prompts, mode):
    kp, kk = [0], []
    for (_, lens, _) in prompts:
        n = len(lens)
        if mode == "all":
            ks = list(range(n))
        elif mode == "none":
            ks = []
        else:
            ks = rng.sample(range(n), rng.randint(1, n))
        rng.shuffle(ks)
        kk += ks
        kp.append(len(kk))
    return np.array(kp), np.array(kk, dtype=np.int64)


CASES = [(0, 4, 1, 64, "some"), (1, 32, 8, 128, "some"), (2, 8, 2, 128, "none"), (3, 16, 2, 64, "some"),
         (4, 8, 8, 128, "all")]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_G{c[1] // c[2]}_d{c[3]}_{c[4]}" for c in CASES])
def test_routed_parity(case):
    seed, hq, hkv, d, mode = case
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=2, p_max=70, n_max=9, l_max=250, q_max=140, p_min=1)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 900 + seed)
    kp, kk = _keep_lists(rng, prompts, mode)
    log(f"[routed parity] seed={seed} Hq={hq} Hkv={hkv} d={d} keep={kk.tolist()}")
    dev = upload(w)
    out, lse = br.attn_routed(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, kp, kk, lse=True)
    torch.cuda.synchronize()
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, kp, kk)
    rows = np.nonzero(~dropped)[0]
    O_ref, lse_ref = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, kp, kk, rows)
    check_attn(out, O_ref, rows=rows, what=f"routed {case}")
    l = lse.cpu().numpy().astype(np.float64)[rows]
    assert (np.abs(l - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max() <= 1e-3
    # dropped documents' rows are left as they were (zero-filled by the wrapper)
    if dropped.any():
        assert torch.count_nonzero(out[torch.as_tensor(np.nonzero(dropped)[0], device=out.device)]) == 0


def test_routed_keep_all_is_bit_identical_to_prompt_kernel():
    w = workloads.make("worked", 0)
    dev = upload(w)
    n = w.num_docs
    log("[routed parity] worked prompt, every document kept")
    a = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
    b = br.attn_routed(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, [0, n], np.arange(n)[::-1].copy())
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_routed_top_b_from_readout():
    """The routing step end to end on the worked prompt: readout scores -> order -> keep the top
    32 documents -> routed attention; checked against the oracle on sampled rows."""
    w = workloads.make("worked", 1)
    dev = upload(w)
    scores = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    order = br.sort_docs(scores, w.doc_ptr)
    keep = order[:32].cpu().numpy().astype(np.int64)
    log(f"[routed parity] worked prompt, top-32 documents {keep[:8].tolist()}...")
    out = br.attn_routed(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, [0, 32], keep)
    torch.cuda.synchronize()
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, [0, 32], keep)
    offs = [int(x) for x in w.segment_offsets]
    rows = np.r_[np.arange(offs[-2], offs[-1]), np.nonzero(~dropped)[0][::37]]
    O_ref, _ = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, [0, 32], keep, rows)
    check_attn(out, O_ref, rows=rows, what="top-32 routed")
