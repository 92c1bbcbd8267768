"""GPU parity of top-B routed attention (br_attn_routed_fwd) against the fp64 oracle, on seeded
inputs, through the C ABI."""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import ORDER_GAP, check_attn, dev_bf16, log, upload
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


def _oracle_top_b(w, B):
    """The oracle's own readout and rank choose the kept documents (inputs to both sides)."""
    s_ref, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    order = orc.rank(s_ref, w.doc_ptr)
    return s_ref, order[:B].astype(np.int64)


def _check_gpu_top_b(w, dev, s_ref, keep, B):
    """The GPU's readout -> order picks the same top-B set wherever the oracle's B-th and (B+1)-th
    scores are separated by more than the order tolerance."""
    scores = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    order = br.sort_docs(scores, w.doc_ptr)
    torch.cuda.synchronize()
    srt = np.sort(s_ref)[::-1]
    if len(srt) > B and srt[B - 1] - srt[B] > ORDER_GAP:
        assert set(order[:B].cpu().numpy().tolist()) == set(keep.tolist()), "GPU top-B set differs"


def test_routed_top_b_from_readout():
    """The routing step end to end on the worked prompt: readout scores -> order -> keep the top
    32 documents -> routed attention; checked against the oracle on sampled rows."""
    w = workloads.make("worked", 1)
    dev = upload(w)
    s_ref, keep = _oracle_top_b(w, 32)
    _check_gpu_top_b(w, dev, s_ref, keep, 32)
    log(f"[routed parity] worked prompt, top-32 documents {keep[:8].tolist()}...")
    out = br.attn_routed(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, [0, 32], keep)
    torch.cuda.synchronize()
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, [0, 32], keep)
    offs = [int(x) for x in w.segment_offsets]
    rows = np.r_[np.arange(offs[-2], offs[-1]), np.nonzero(~dropped)[0][::37]]
    O_ref, _ = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, [0, 32], keep, rows)
    check_attn(out, O_ref, rows=rows, what="top-32 routed")


def test_routed_long_top256():
    """The bench's routed configuration at full size: the long prompt (500 documents, T = 100,096)
    with its top 256 documents kept.  Kept documents' rows are bit-identical to the unrouted
    kernel's (their plan items are the same); the query rows and sampled kept rows match the
    oracle."""
    w = workloads.make("long", 0)
    dev = upload(w)
    s_ref, keep = _oracle_top_b(w, 256)
    _check_gpu_top_b(w, dev, s_ref, keep, 256)
    log(f"[routed long] top-256 of {w.num_docs} documents")
    full = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
    out = br.attn_routed(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, [0, 256], keep)
    torch.cuda.synchronize()
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, [0, 256], keep)
    offs = [int(x) for x in w.segment_offsets]
    kept_doc_rows = np.nonzero(~dropped)[0]
    kept_doc_rows = kept_doc_rows[(kept_doc_rows >= offs[1]) & (kept_doc_rows < offs[-2])]
    kr = torch.as_tensor(kept_doc_rows, device="cuda")
    assert torch.equal(out[kr], full[kr]), "kept documents' rows differ from the unrouted kernel"
    rng = np.random.default_rng(3)
    # the oracle takes about two seconds per query row here: first, middle and last query rows
    rows = np.r_[[offs[-2], (offs[-2] + offs[-1]) // 2, offs[-1] - 1], rng.choice(kept_doc_rows, 24, replace=False)]
    O_ref, _ = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, [0, 256], keep, rows)
    check_attn(out, O_ref, rows=rows, what="top-256 routed, long prompt")
