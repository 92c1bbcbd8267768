"""GPU parity of the additive sink (br_attn_fwd_sink) against the fp64 oracle, through the C ABI.

The sink appends exp(b) to every row's softmax denominator (BlockSearch, section 5.1, and its
appendix note on the sink), i.e. scales each output row by sigma(lse - b) <= 1; the kernel adds
2^(b log2 e - m) to its fp32 row sum before the one reciprocal, so the error bound of the plain
attention (max-abs 2e-2 on outputs) holds unchanged."""
import math
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import check_attn, log, to_f64, upload, LSE_RTOL
from pins import random_prompts

pytestmark = pytest.mark.gpu


def test_sink_minus_inf_is_plain_attention_bit_for_bit():
    """b = -inf leaves the output and lse bit-identical to br_attn_fwd, on the worked shape (its
    query rows take the split-key merge)."""
    w = workloads.make("worked", 0)
    dev = upload(w)
    log(f"[sink] -inf vs plain: worked T={w.total_tokens}")
    a, al = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True)
    b, bl = br.attn_fwd_sink(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, -math.inf, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(al, bl)


@pytest.mark.parametrize("seed", range(4))
def test_sink_parity_small(seed):
    rng = random.Random(900 + seed)
    hq, hkv, d = [(4, 1, 64), (8, 2, 128), (8, 8, 128), (16, 4, 64)][seed]
    prompts = random_prompts(rng, batch=2, p_max=70, n_max=8, l_max=150, q_max=100, p_min=0 if seed % 2 else 1)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 3900 + seed)
    dev = upload(w)
    ref_plain, ref_lse = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    # thresholds around the rows' own log-sum-exp, so gates span (0, 1)
    for b in (float(np.median(ref_lse)), float(np.median(ref_lse)) + 3.0, -2.0):
        log(f"[sink] seed={seed} Hq={hq} Hkv={hkv} d={d} T={w.total_tokens} b={b:.3f}")
        out, lse = br.attn_fwd_sink(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, b, lse=True)
        torch.cuda.synchronize()
        ref, rl = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, sink=b)
        check_attn(out, ref, what=f"sink b={b:.3f}")
        got_l = to_f64(lse)
        assert np.abs(got_l - rl).max() <= LSE_RTOL * max(1.0, np.abs(rl).max())
        gate = 1.0 / (1.0 + np.exp(b - rl))
        assert gate.min() < 0.9 or b < 0  # the thresholds do gate some rows


def test_sink_long_prompt_sampled_rows():
    """The long ranking prompt at full size, sampled rows of every kind (the query rows go through
    the split-key merge, which adds the sink after combining the chunks)."""
    w = workloads.make("long", 0)
    dev = upload(w)
    so = np.asarray(w.segment_offsets)
    T = w.total_tokens
    rows = [0, 63] + [int(so[1 + k]) + j for k in (0, 250, 499) for j in (0, 199)] + list(range(T - 32, T))
    b = 4.0
    log(f"[sink] long prompt T={T}, b={b}, {len(rows)} sampled rows")
    out = br.attn_fwd_sink(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, b)
    torch.cuda.synchronize()
    ref, rl = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=rows, sink=b)
    check_attn(out, ref, rows=rows, what="long sink")
