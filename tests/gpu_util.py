"""Helpers shared by the GPU tests: device upload of seeded workloads, tolerances, checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_attention_segment_amd as br

# Tolerances (stated with the method's target: bf16 inputs, fp32 accumulation).
ATTN_ATOL = 2e-2          # max-abs on attention outputs
LSE_RTOL = 1e-3           # relative on log-sum-exp
SCORE_RTOL = 1e-3         # relative on s_k ...
SCORE_ATOL_PER_SIGNAL = 1e-30  # ... plus an absolute floor per signal token, felt only near fp32 underflow
ORDER_GAP = 1e-3          # order must agree wherever the oracle's neighbouring gap exceeds this


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def upload(w):
    return dict(Q=dev_bf16(w.Q), K=dev_bf16(w.K), V=dev_bf16(w.V), Q_S=dev_bf16(w.Q_S))


def run_attn(w, dev, lse=False, scale=0.0):
    r = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=lse, softmax_scale=scale)
    torch.cuda.synchronize()
    return r


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_attn(got_bf16: torch.Tensor, ref: np.ndarray, rows=None, what=""):
    g = to_f64(got_bf16 if rows is None else got_bf16[torch.as_tensor(rows, device=got_bf16.device)])
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref).max()
    assert err <= ATTN_ATOL, f"{what}: max-abs error {err:.3e} > {ATTN_ATOL}"
    return err


def check_scores(got: np.ndarray, ref: np.ndarray, n_signal: int, what=""):
    tol = SCORE_RTOL * np.abs(ref) + SCORE_ATOL_PER_SIGNAL * n_signal
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} scores out of tolerance, worst {np.abs(got - ref).max():.3e}"


def check_order(order_gpu: np.ndarray, ref_scores: np.ndarray, doc_ptr, what=""):
    """Argmax and every adjacent oracle pair separated by more than ORDER_GAP must agree."""
    dp = np.asarray(doc_ptr)
    base = 0
    for b in range(len(dp) - 1):
        N = int(dp[b + 1] - dp[b] - 1)
        s = ref_scores[base:base + N]
        og = order_gpu[base:base + N]
        assert sorted(og.tolist()) == list(range(N)), f"{what}: prompt {b} order is not a permutation"
        oref = sorted(range(N), key=lambda k: (-s[k], k))
        pos = np.empty(N, dtype=np.int64)
        pos[og] = np.arange(N)
        for a_, b_ in zip(oref[:-1], oref[1:]):
            if s[a_] - s[b_] > ORDER_GAP:
                assert pos[a_] < pos[b_], f"{what}: prompt {b}: docs {a_},{b_} (gap {s[a_] - s[b_]:.2e}) swapped"
        if N > 1 and s[oref[0]] - s[oref[1]] > ORDER_GAP:
            assert og[0] == oref[0], f"{what}: prompt {b}: argmax {og[0]} != {oref[0]}"
        base += N
