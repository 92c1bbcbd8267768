"""GPU parity of query-only attention over a cached corpus (br_query_attn_fwd) against the fp64
oracle, on seeded inputs, through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import ATTN_ATOL, LSE_RTOL, check_attn, dev_bf16, log

pytestmark = pytest.mark.gpu


def _case(seed, corpus, qlens, hq, hkv, d, q_scale=1.0):
    rng = np.random.default_rng(seed)
    T = corpus + sum(qlens)
    bf = lambda a: workloads.f32_to_bf16_bits(a.astype(np.float32))
    K = bf(rng.standard_normal((T, hkv, d))); V = bf(rng.standard_normal((T, hkv, d)))
    Q = bf(rng.standard_normal((T - corpus, hq, d)) * q_scale)
    qo = np.cumsum([corpus] + list(qlens)).astype(np.int32)
    return Q, K, V, qo


CASES = [
    # (seed, corpus, query lengths, Hq, Hkv, d)
    (0, 0, [5, 1, 40], 4, 4, 64),
    (1, 37, [1], 8, 2, 128),
    (2, 200, [33, 7, 129], 32, 8, 128),
    (3, 1000, [31, 32, 2], 8, 1, 64),
    (4, 4100, [40, 25, 3, 64], 8, 2, 128),  # many split chunks, merged
    (5, 333, [300], 16, 2, 128),            # several row tiles per query
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_c{c[1]}_G{c[3] // c[4]}_d{c[5]}" for c in CASES])
def test_query_attn_parity(case):
    seed, corpus, qlens, hq, hkv, d = case
    log(f"[query parity] seed={seed} corpus={corpus} queries={qlens} Hq={hq} Hkv={hkv} d={d}")
    Q, K, V, qo = _case(seed, corpus, qlens, hq, hkv, d)
    out, lse = br.query_attn(dev_bf16(Q), dev_bf16(K), dev_bf16(V), corpus, qo, lse=True)
    torch.cuda.synchronize()
    O_ref, lse_ref = orc.query_attn(Q, K, V, corpus, qo)
    check_attn(out, O_ref, what=f"query attn {case}")
    l = lse.cpu().numpy().astype(np.float64)
    rel = np.abs(l - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    assert rel.max() <= LSE_RTOL, f"lse rel error {rel.max():.3e}"


def test_query_attn_sharp_softmax():
    Q, K, V, qo = _case(9, 700, [20, 45], 8, 2, 128, q_scale=8.0)
    log("[query parity] sharp softmax (Q x 8)")
    out = br.query_attn(dev_bf16(Q), dev_bf16(K), dev_bf16(V), 700, qo)
    torch.cuda.synchronize()
    check_attn(out, orc.query_attn(Q, K, V, 700, qo)[0], what="sharp")


def test_query_attn_matches_prompt_query_rows():
    """Over the corpus of the worked prompt (instruction + 100 documents), query-only attention
    for its final query equals the prompt kernel's query rows."""
    w = workloads.make("worked", 0)
    offs = [int(x) for x in w.segment_offsets]
    qs, qe = offs[-2], offs[-1]
    log(f"[query parity] worked prompt corpus={qs} query={qe - qs}")
    Q, K, V = dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V)
    full = br.attn_fwd(Q, K, V, w.segment_offsets, w.seg_ptr)
    part = br.query_attn(Q[qs:qe].contiguous(), K, V, qs, np.array([qs, qe], dtype=np.int32))
    torch.cuda.synchronize()
    diff = (full[qs:qe].float() - part.float()).abs().max().item()
    assert diff <= ATTN_ATOL, diff
    # and both against the oracle on a sample of the rows
    rows = np.arange(qs, qe, 5)
    O_ref, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=rows)
    check_attn(part, O_ref, rows=rows - qs, what="query-only vs oracle")


def test_query_attn_other_queries_do_not_leak():
    """Changing one query's tokens leaves the other queries' outputs bit-identical."""
    Q, K, V, qo = _case(12, 500, [30, 17, 64], 8, 2, 128)
    log("[query parity] isolation between queries")
    a = br.query_attn(dev_bf16(Q), dev_bf16(K), dev_bf16(V), 500, qo)
    K2, V2 = K.copy(), V.copy()
    K2[qo[1]:qo[2]] ^= np.uint16(0x0040); V2[qo[1]:qo[2]] ^= np.uint16(0x0040)
    b = br.query_attn(dev_bf16(Q), dev_bf16(K2), dev_bf16(V2), 500, qo)
    torch.cuda.synchronize()
    for q in (0, 2):
        lo, hi = int(qo[q]) - 500, int(qo[q + 1]) - 500
        assert torch.equal(a[lo:hi], b[lo:hi]), q


def test_query_attn_long_corpus_bench_config():
    """The bench's query-only configuration at full size: 16 queries of 32 tokens over the long
    prompt's cached corpus (instruction + 500 documents, 100,064 tokens).  Queries are independent,
    so three of them are checked against the oracle run on the corpus plus that query alone."""
    w = workloads.make("long", 0)
    offs = [int(x) for x in w.segment_offsets]
    corpus = offs[-2]
    Hq, d, Hkv = w.Q.shape[1], w.Q.shape[2], w.K.shape[1]
    rng = np.random.default_rng(1000)
    nq, ql = 16, 32
    bf = lambda a: workloads.f32_to_bf16_bits(a.astype(np.float32))
    Kq, Vq = bf(rng.standard_normal((nq * ql, Hkv, d))), bf(rng.standard_normal((nq * ql, Hkv, d)))
    Qq = bf(rng.standard_normal((nq * ql, Hq, d)))
    K = np.concatenate([w.K[:corpus], Kq]); V = np.concatenate([w.V[:corpus], Vq])
    qo = (np.arange(nq + 1) * ql + corpus).astype(np.int32)
    log(f"[query long] {nq} x {ql} tokens over a {corpus}-token corpus")
    out, lse = br.query_attn(dev_bf16(Qq), dev_bf16(K), dev_bf16(V), corpus, qo, lse=True)
    torch.cuda.synchronize()
    for b in (0, 7, 15):
        a, e = b * ql, (b + 1) * ql
        Ks = np.concatenate([w.K[:corpus], Kq[a:e]]); Vs = np.concatenate([w.V[:corpus], Vq[a:e]])
        O_ref, lse_ref = orc.query_attn(Qq[a:e], Ks, Vs, corpus, [corpus, corpus + ql])
        check_attn(out[a:e], O_ref, what=f"query {b}")
        rel = np.abs(lse[a:e].cpu().numpy() - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
        assert rel.max() <= LSE_RTOL, f"query {b}: lse rel err {rel.max():.3e}"
