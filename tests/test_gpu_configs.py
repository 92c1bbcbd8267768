"""GPU parity on the named workloads at their full sizes, in the launch configuration the bench
times (one br_rank_prompts call per step: on the caller's stream below 24,576 tokens, with the
readout on the side stream above): the worked shape (every row checked), the long list (sampled
rows, all scores), the ragged lists with a planted document, and the 16-prompt batch."""
import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import check_attn, check_order, check_scores, log, upload

pytestmark = pytest.mark.gpu


def _segment_rows(w, b, s):
    offs = w.segment_offsets[w.seg_ptr[b]:w.seg_ptr[b + 1]]
    return np.arange(int(offs[s]), int(offs[s + 1]))


def _sample_rows(w, b, docs):
    n = int(w.seg_ptr[b + 1] - w.seg_ptr[b])
    parts = [_segment_rows(w, b, 0)] + [_segment_rows(w, b, 1 + k) for k in docs] + [_segment_rows(w, b, n - 2)]
    return np.concatenate(parts)


def _rank_step(w, dev):
    """The bench's step: attention, readout and rank in one library call."""
    out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr,
                             w.doc_offsets, w.doc_ptr)
    torch.cuda.synchronize()
    return out, s, o


def _scores_and_order(w, s, o, what):
    s = s.cpu().numpy().astype(np.float64)
    ref, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    check_scores(s, ref, w.n_signal, what)
    check_order(o.cpu().numpy(), ref, w.doc_ptr, what)
    base = 0
    for b in range(w.num_prompts):
        N = int(w.doc_ptr[b + 1] - w.doc_ptr[b] - 1)
        assert abs(s[base:base + N].sum() - w.n_signal) <= 1e-3 * w.n_signal, f"{what}: sum of scores"
        base += N
    return s, ref, o.cpu().numpy()


def test_worked_all_rows():
    w = workloads.make("worked", 0)
    log("[gpu] worked seed 0: attention (all rows) + scores + order")
    dev = upload(w)
    out, s, o = _rank_step(w, dev)
    ref, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    err = check_attn(out, ref, what="worked")
    log(f"[gpu] worked max-abs error {err:.3e}")
    _scores_and_order(w, s, o, "worked")


def test_long_sampled_rows_and_scores():
    w = workloads.make("long", 0)
    log("[gpu] long seed 0: attention (sampled rows) + scores + order")
    dev = upload(w)
    out, s, o = _rank_step(w, dev)
    rows = _sample_rows(w, 0, [0, 1, 250, 498, 499])
    ref, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=rows)
    err = check_attn(out, ref, rows=rows, what="long")
    log(f"[gpu] long max-abs error {err:.3e} over {len(rows)} rows")
    _scores_and_order(w, s, o, "long")


@pytest.mark.parametrize("seed", range(5))
def test_ragged_planted_document(seed):
    w = workloads.make("ragged", seed)
    log(f"[gpu] ragged seed {seed}: T={w.total_tokens} planted={w.planted}")
    dev = upload(w)
    out, s, o = _rank_step(w, dev)
    k = w.planted[0]
    rows = _sample_rows(w, 0, sorted({0, k, 199}))
    ref, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=rows)
    check_attn(out, ref, rows=rows, what=f"ragged seed {seed}")
    s, ref_s, order = _scores_and_order(w, s, o, f"ragged seed {seed}")
    # the planted document is the oracle's clear winner for these seeds, and the GPU's argmax
    top = np.sort(ref_s)[::-1]
    assert int(np.argmax(ref_s)) == k and top[0] - top[1] > 1e-3
    assert int(order[0]) == k


def test_batched_prompts():
    w = workloads.make("batched", 0)
    log(f"[gpu] batched: B={w.num_prompts} T={w.total_tokens}")
    dev = upload(w)
    out, s, o = _rank_step(w, dev)
    rows = np.concatenate([_sample_rows(w, b, [0, 99]) for b in (0, 7, 15)])
    ref, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=rows)
    check_attn(out, ref, rows=rows, what="batched")
    _scores_and_order(w, s, o, "batched")
