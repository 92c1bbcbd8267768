"""GPU checks of SSMax scaling (BlockSearch, section 5.1): the per-call logit factor
s * ln N / sqrt(d) passed as softmax_scale to the attention and the readout, against the pages'
gold-weight closed form and the fp64 oracle, through the C ABI."""
import math
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import LSE_RTOL, check_attn, check_order, check_scores, dev_bf16, log, upload
from pins import random_prompts

pytestmark = pytest.mark.gpu


def test_ssmax_factor_matches_oracle():
    for s, n, d in [(0.43, 2, 64), (0.43, 500, 128), (0.2, 10000, 128), (1.0, 37, 64)]:
        got = br.ssmax_scale(s, n, d)
        want = orc.ssmax_scale(s, n, d)
        assert abs(got - want) <= 1e-6 * want, (s, n, d, got, want)


@pytest.mark.parametrize("n,s,delta", [(100, 0.43, 2.0), (1000, 0.43, 3.0), (5000, 0.43, 4.0), (500, 0.25, 5.0),
                                       (64, 1.0, 1.5)])
def test_ssmax_gold_weight_on_gpu(n, s, delta):
    """One query token over a corpus with one gold key Delta above N - 1 distractors (its own key
    is the N-th distractor): the output's marker channel is the gold weight 1 / (1 + N^(1 - s Delta))."""
    d = 64
    K = np.zeros((n + 1, 1, d), np.float32); V = np.zeros((n + 1, 1, d), np.float32)
    gold = (7 * n) // 13
    K[gold, 0, 0] = delta
    V[gold, 0, 0] = 1.0
    Q = np.zeros((1, 1, d), np.float32); Q[0, 0, 0] = 8.0          # q.k / sqrt(64) = k[0]
    bits = workloads.f32_to_bf16_bits
    log(f"[ssmax gold] N={n} s={s} delta={delta}")
    out = br.query_attn(dev_bf16(bits(Q)), dev_bf16(bits(K)), dev_bf16(bits(V)), n, [n, n + 1],
                        softmax_scale=br.ssmax_scale(s, n, d))
    torch.cuda.synchronize()
    got = float(out[0, 0, 0].float())
    want = 1.0 / (1.0 + n ** (1.0 - s * delta))
    # P is rounded to bf16 before P.V and the output is stored in bf16: two relative 2^-9 roundings
    assert abs(got - want) <= 8e-3 * want + 1e-6, (got, want)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ssmax_prompt_parity(seed):
    """Attention, readout and rank of one prompt with the SSMax factor for its N documents."""
    rng = random.Random(70 + seed)
    p = rng.randint(8, 64)
    n = rng.randint(20, 60)
    lens = [rng.randint(20, 160) for _ in range(n)]
    prompts = [(p, lens, rng.randint(8, 48))]
    hq, hkv, d = [(32, 8, 128), (8, 2, 64), (16, 16, 128)][seed]
    w = workloads.make_custom(prompts, hq, hkv, d, 4, 1700 + seed)
    log(f"[ssmax parity] seed={seed} N={n} T={w.total_tokens} Hq={hq} Hkv={hkv} d={d}")
    scale = br.ssmax_scale(0.43, n, d)
    dev = upload(w)
    out, lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True, softmax_scale=scale)
    scores = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, softmax_scale=scale)
    order = br.sort_docs(scores, w.doc_ptr)
    torch.cuda.synchronize()
    ref_scale = orc.ssmax_scale(0.43, n, d)
    O_ref, lse_ref = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=np.arange(w.total_tokens),
                                   scale=ref_scale)
    check_attn(out, O_ref, what="attention under SSMax")
    lg = lse.cpu().numpy().astype(np.float64)
    rel = np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    assert rel.max() <= LSE_RTOL, f"lse rel err {rel.max():.3e}"
    s_ref, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr, scale=ref_scale)
    check_scores(scores.cpu().numpy().astype(np.float64), s_ref, 4, what="scores under SSMax")
    check_order(order.cpu().numpy(), s_ref, w.doc_ptr, what="order under SSMax")
    assert math.isclose(scale, ref_scale, rel_tol=1e-6)
