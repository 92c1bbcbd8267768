"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes the oracle module and raises AssertionError when the oracle disagrees
with a closed form, a printed number, an invariant, a library routine or a brute-force
evaluation.  The mutation tests run every pin against deliberately broken copies of the
oracle and require at least one pin to fail for each, so the pins are known to have teeth.
"""
from __future__ import annotations

import json
import math
import os
import random

import numpy as np
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------------------
# small random inputs
# --------------------------------------------------------------------------------------
def random_prompts(rng: random.Random, batch=1, p_max=40, n_max=6, l_max=70, q_max=40, p_min=0):
    prompts = []
    for _ in range(batch):
        p = rng.randint(p_min, p_max)
        n = rng.randint(1, n_max)
        lens = [rng.randint(1, l_max) for _ in range(n)]
        q = rng.randint(1, q_max)
        prompts.append((p, lens, q))
    return prompts


def small_case(seed, hq=2, hkv=1, d=8, batch=2, n_signal=1, **kw):
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=batch, **kw)
    prompts = [(p, l, max(q, n_signal)) for (p, l, q) in prompts]
    return workloads.make_custom(prompts, hq, hkv, d, n_signal, seed)


def _f64(x):
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# mask / pair counts
# --------------------------------------------------------------------------------------
def pin_closed_form_counts(orc):
    """Counting the explicit mask reproduces the blog's closed form (diagonal blocks whole),
    and the causal count is that minus n(n-1)/2 per segment."""
    rng = random.Random(1234)
    for t in range(25):
        prompts = random_prompts(rng, batch=rng.randint(1, 3), p_min=0)
        seg, sp, _, _ = workloads.segment_tables(prompts)
        blk = orc.count_pairs(seg, sp, full_diagonal=True)
        exact = orc.count_pairs(seg, sp, full_diagonal=False)
        want_blk = sum(orc.closed_form_pairs(p, l, q) for (p, l, q) in prompts)
        # closed form, typed independently here from the blog's complexity section
        ref_blk = sum(p * p + sum(x * x + p * x for x in l) + q * (p + q + sum(l)) for (p, l, q) in prompts)
        diag = sum(n * (n - 1) // 2 for (p, l, q) in prompts for n in [p, q] + list(l))
        assert want_blk == ref_blk, (prompts, want_blk, ref_blk)
        assert blk == ref_blk, (prompts, blk, ref_blk)
        assert exact == ref_blk - diag, (prompts, exact, ref_blk - diag)
        # the (causal, whole-diagonal) pair of counts, in that order
        assert orc.allowed_pair_counts(seg, sp) == (ref_blk - diag, ref_blk), prompts


def pin_worked_example(orc):
    """The blog's worked example: p=q=32, N=100, l=128 -> L=12,864, ~165.48M dense pairs,
    2.46M allowed pairs (printed rounded)."""
    with open(os.path.join(GOLDEN, "blog_worked_example.json")) as f:
        g = json.load(f)
    prompts = [(g["p"], [g["doc_len"]] * g["n_docs"], g["q"])]
    seg, sp, _, _ = workloads.segment_tables(prompts)
    L = int(seg[-1])
    assert L == g["dense_side_printed"]
    assert round(L * L / 1e6, 2) == g["dense_pairs_printed_millions"]
    blk = orc.count_pairs(seg, sp, full_diagonal=True)
    assert round(blk / 1e6, 2) == g["allowed_pairs_printed_millions"], blk
    assert blk == orc.closed_form_pairs(g["p"], [g["doc_len"]] * g["n_docs"], g["q"])


# --------------------------------------------------------------------------------------
# attention rows reduce to textbook causal attention
# --------------------------------------------------------------------------------------
def _sdpa_causal(q, k, v):
    """torch's scaled_dot_product_attention, causal, float64, GQA by its own rule.

    q [n, Hq, d], k/v [n, Hkv, d] -> [n, Hq, d]"""
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         enable_gqa=qt.shape[1] != kt.shape[1])
    return o[0].permute(1, 0, 2).numpy()


def _check_textbook(orc, w, O, tol=1e-10):
    Q, K, V = _f64(w.Q), _f64(w.K), _f64(w.V)
    so, sp = w.segment_offsets, w.seg_ptr
    for b in range(w.num_prompts):
        offs = [int(x) for x in so[sp[b]:sp[b + 1]]]
        a, p_end, q_start, e = offs[0], offs[1], offs[-2], offs[-1]
        full = _sdpa_causal(Q[a:e], K[a:e], V[a:e])
        # instruction rows and query rows = rows of plain causal attention over the prompt
        np.testing.assert_allclose(O[a:p_end], full[:p_end - a], rtol=0, atol=tol)
        np.testing.assert_allclose(O[q_start:e], full[q_start - a:], rtol=0, atol=tol)
        # document k rows = last l_k rows of causal attention over [instruction ; d_k]
        for s in range(1, len(offs) - 2):
            da, de = offs[s], offs[s + 1]
            idx = np.r_[a:p_end, da:de]
            sub = _sdpa_causal(Q[idx], K[idx], V[idx])
            np.testing.assert_allclose(O[da:de], sub[p_end - a:], rtol=0, atol=tol)


def pin_textbook_rows(orc):
    for seed, (hq, hkv, d) in enumerate([(2, 1, 8), (4, 2, 16), (3, 3, 8), (8, 2, 8)]):
        w = small_case(100 + seed, hq=hq, hkv=hkv, d=d, batch=2)
        O, _ = orc.attn_dense(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
        _check_textbook(orc, w, O)
        O2, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, row_block=7)
        _check_textbook(orc, w, O2)


def pin_textbook_rows_no_prefix(orc):
    """p = 0 (BlockSearch drops the instruction prefix)."""
    rng = random.Random(77)
    prompts = [(0, [rng.randint(1, 30) for _ in range(4)], 9), (0, [5, 1, 17], 3)]
    w = workloads.make_custom(prompts, 4, 2, 8, 1, 77)
    O, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    _check_textbook(orc, w, O)


def pin_sink_limits_and_gate(orc):
    """Additive sink ([BS] 5.1): b = -inf leaves the plain softmax output exactly; a huge b drives
    the output to zero; for every b the output is the plain output times sigma(lse - b), the gate
    form of the appendix note on the sink."""
    w = small_case(61, hq=4, hkv=2, d=8, batch=2)
    O, lse = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    O1, lse1 = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, sink=-math.inf)
    assert np.array_equal(O, O1) and np.array_equal(lse, lse1)
    O2, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, sink=600.0)
    assert np.abs(O2).max() < 1e-200
    for b in (-3.0, 0.0, 1.5, 4.0):
        Ob, lb = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, sink=b, row_block=5)
        assert np.allclose(lb, lse, rtol=1e-13, atol=1e-13)  # other row blocks: other summation order
        gate = 1.0 / (1.0 + np.exp(b - lse))
        assert np.allclose(Ob, O * gate[:, :, None], rtol=1e-12, atol=1e-15), b


def pin_sink_single_key(orc):
    """A row that reads one key (the prompt's first token) has the closed form
    v / (1 + exp(b - s)), s = q.k / sqrt(d): the sink is the only other slot of its softmax."""
    w = small_case(62, hq=2, hkv=1, d=8, batch=1)
    q, k, v = (workloads.bf16_bits_to_f32(x[0]).astype(np.float64) for x in (w.Q, w.K, w.V))
    for b in (-2.0, 0.3, 3.0):
        O, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=[0], sink=b)
        for h in range(2):
            s_ = float(q[h] @ k[0]) / math.sqrt(8)
            want = v[0] / (1.0 + math.exp(b - s_))
            assert np.allclose(O[0, h], want, rtol=1e-12, atol=1e-15), (b, h)


# --------------------------------------------------------------------------------------
# brute force from the chunked formulation (BlockRank summary, chunked implementation):
# documents attend to [K_Inst, K_k], the query to everything, the instruction causally.
# --------------------------------------------------------------------------------------
def _brute_chunked(w, scale=None):
    Q, K, V = _f64(w.Q), _f64(w.K), _f64(w.V)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    O = np.zeros_like(Q)
    so, sp = w.segment_offsets, w.seg_ptr
    for b in range(w.num_prompts):
        offs = [int(x) for x in so[sp[b]:sp[b + 1]]]
        inst = list(range(offs[0], offs[1]))
        for s in range(len(offs) - 1):
            seg = list(range(offs[s], offs[s + 1]))
            for i in seg:
                if s == 0:
                    keys = [j for j in inst if j <= i]
                elif s == len(offs) - 2:
                    keys = list(range(offs[0], i + 1))
                else:
                    keys = inst + [j for j in seg if j <= i]
                for h in range(Hq):
                    g = h * Hkv // Hq
                    z = [sum(Q[i, h, t] * K[j, g, t] for t in range(d)) * sc for j in keys]
                    mz = max(z)
                    e = [math.exp(x - mz) for x in z]
                    tot = sum(e)
                    for t in range(d):
                        O[i, h, t] = sum(e[n] * V[keys[n], g, t] for n in range(len(keys))) / tot
    return O


def pin_bruteforce_chunked(orc):
    for seed, (hq, hkv) in enumerate([(2, 1), (1, 1), (4, 2)]):
        rng = random.Random(500 + seed)
        prompts = random_prompts(rng, batch=2, p_max=5, n_max=3, l_max=6, q_max=5)
        w = workloads.make_custom(prompts, hq, hkv, 4, 1, 500 + seed)
        ref = _brute_chunked(w)
        O, _ = orc.attn_dense(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
        O2, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, row_block=3)
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(O2, ref, rtol=0, atol=1e-12)


def pin_special_rows(orc):
    """A row that may only read itself returns its own V; its LSE is its own logit."""
    w = small_case(9, hq=2, hkv=1, d=8, batch=1, p_min=1)
    O, lse = orc.attn_dense(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    Q, K, V = _f64(w.Q), _f64(w.K), _f64(w.V)
    for h in range(2):
        np.testing.assert_array_equal(O[0, h], V[0, 0])
        assert abs(lse[0, h] - Q[0, h] @ K[0, 0] / math.sqrt(8)) < 1e-12
    # without a prefix, the first token of every document reads only itself
    prompts = [(0, [3, 1, 4], 2)]
    w = workloads.make_custom(prompts, 2, 1, 8, 1, 10)
    O, lse = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    V = _f64(w.V)
    for t in (0, 3, 4):
        for h in range(2):
            np.testing.assert_array_equal(O[t, h], V[t, 0])


def pin_document_isolation(orc):
    """A document's outputs do not change when other documents (or the query) change, and
    move with the document when documents are permuted."""
    rng = random.Random(31)
    lens = [rng.randint(3, 20) for _ in range(5)]
    w = workloads.make_custom([(6, lens, 4)], 4, 2, 8, 1, 31)
    O, _ = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    so = [int(x) for x in w.segment_offsets]
    # alter every document except doc 2 and the query
    Q2, K2, V2 = w.Q.copy(), w.K.copy(), w.V.copy()
    keep = range(so[3], so[4])
    noise = np.random.default_rng(5)
    for t in range(so[1], so[-1]):
        if t not in keep:
            K2[t] = noise.integers(0x3000, 0x4000, size=K2[t].shape, dtype=np.uint16)
            V2[t] = noise.integers(0x3000, 0x4000, size=V2[t].shape, dtype=np.uint16)
            Q2[t] = noise.integers(0x3000, 0x4000, size=Q2[t].shape, dtype=np.uint16)
    O2, _ = orc.attn_rows(Q2, K2, V2, w.segment_offsets, w.seg_ptr)
    np.testing.assert_array_equal(O2[so[3]:so[4]], O[so[3]:so[4]])
    np.testing.assert_array_equal(O2[:so[1]], O[:so[1]])
    # permute the documents: each document's block moves unchanged
    perm = [3, 0, 4, 2, 1]
    spans = [(so[1 + k], so[2 + k]) for k in range(5)]
    idx = np.r_[0:so[1], np.concatenate([np.arange(*spans[k]) for k in perm]), so[-2]:so[-1]]
    wp_seg, wp_sp, _, _ = workloads.segment_tables([(6, [lens[k] for k in perm], 4)])
    Op, _ = orc.attn_rows(w.Q[idx], w.K[idx], w.V[idx], wp_seg, wp_sp)
    pos = so[1]
    for k in perm:
        a, e = spans[k]
        np.testing.assert_array_equal(Op[pos:pos + (e - a)], O[a:e])
        pos += e - a
    # query rows: unchanged up to summation order
    np.testing.assert_allclose(Op[-4:], O[-4:], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# readout (BlockRank summary, score computation steps 1-4; blog, attention supervision)
# --------------------------------------------------------------------------------------
def _brute_scores(w, scale=None):
    Qs, K = _f64(w.Q_S), _f64(w.K)
    B, S, Hq, d = Qs.shape
    Hkv = K.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = []
    for b in range(B):
        offs = [int(x) for x in w.doc_offsets[w.doc_ptr[b]:w.doc_ptr[b + 1]]]
        docs = list(range(offs[0], offs[-1]))
        s = [0.0] * (len(offs) - 1)
        for h in range(Hq):
            g = h * Hkv // Hq
            for i in range(S):
                z = {j: sum(Qs[b, i, h, t] * K[j, g, t] for t in range(d)) * sc for j in docs}
                mz = max(z.values())
                den = sum(math.exp(v - mz) for v in z.values())
                for k in range(len(offs) - 1):
                    s[k] += sum(math.exp(z[j] - mz) for j in range(offs[k], offs[k + 1])) / den / Hq
        out.extend(s)
    return np.asarray(out)


def pin_readout_bruteforce(orc):
    for seed, (hq, hkv) in enumerate([(2, 1), (4, 2), (1, 1)]):
        rng = random.Random(900 + seed)
        prompts = random_prompts(rng, batch=2, p_max=4, n_max=4, l_max=6, q_max=4)
        prompts = [(p, l, max(q, 2)) for (p, l, q) in prompts]
        w = workloads.make_custom(prompts, hq, hkv, 4, 2, 900 + seed)
        s, hs = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
        np.testing.assert_allclose(s, _brute_scores(w), rtol=1e-12, atol=1e-14)


def pin_readout_mass(orc):
    """sum_k s_k = |S| per prompt (blog, attention supervision); scores = mean of head_scores."""
    w = small_case(41, hq=4, hkv=2, d=16, batch=3, n_signal=3, n_max=8)
    s, hs = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    base = 0
    for b in range(w.num_prompts):
        N = int(w.doc_ptr[b + 1] - w.doc_ptr[b] - 1)
        assert abs(s[base:base + N].sum() - w.n_signal) < 1e-12
        np.testing.assert_allclose(hs[:, base:base + N].sum(axis=1), w.n_signal, rtol=0, atol=1e-12)
        base += N
    np.testing.assert_allclose(s, hs.mean(axis=0), rtol=0, atol=1e-15)


def pin_readout_uniform(orc):
    """All document keys equal (per KV head), or Q_S = 0 -> every document token gets the same
    weight, so s_k = |S| l_k / D.  One document -> s_1 = |S|."""
    rng = random.Random(8)
    prompts = random_prompts(rng, batch=2, p_max=5, n_max=6, l_max=12, q_max=6)
    prompts = [(p, l, max(q, 3)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, 4, 2, 8, 3, 8)
    K = w.K.copy()
    for b in range(w.num_prompts):
        a = int(w.doc_offsets[w.doc_ptr[b]]); e = int(w.doc_offsets[w.doc_ptr[b + 1] - 1])
        K[a:e] = K[a]
    zeroQ = np.zeros_like(w.Q_S)
    for (qs, kk) in ((w.Q_S, K), (zeroQ, w.K)):
        s, _ = orc.doc_scores(qs, kk, w.doc_offsets, w.doc_ptr)
        want = []
        for (p, l, q) in w.prompts:
            want.extend([3 * x / sum(l) for x in l])
        np.testing.assert_allclose(s, want, rtol=1e-12, atol=0)
    w1 = workloads.make_custom([(4, [7], 3), (0, [1], 5)], 2, 1, 8, 3, 3)
    s, _ = orc.doc_scores(w1.Q_S, w1.K, w1.doc_offsets, w1.doc_ptr)
    np.testing.assert_allclose(s, [3.0, 3.0], rtol=1e-14)


def pin_readout_permutation(orc):
    """Permuting the documents permutes the scores."""
    lens = [4, 9, 2, 7, 5]
    w = workloads.make_custom([(3, lens, 4)], 4, 2, 8, 2, 55)
    s, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    perm = [2, 4, 0, 1, 3]
    so = [int(x) for x in w.segment_offsets]
    idx = np.r_[0:so[1], np.concatenate([np.arange(so[1 + k], so[2 + k]) for k in perm]), so[-2]:so[-1]]
    _, _, dp_o, dp_p = workloads.segment_tables([(3, [lens[k] for k in perm], 4)])
    sp_, _ = orc.doc_scores(w.Q_S, w.K[idx], dp_o, dp_p)
    np.testing.assert_allclose(sp_, s[perm], rtol=1e-12, atol=0)


# --------------------------------------------------------------------------------------
# rank (BlockRank summary, attention-based inference step 3; blog, direct output)
# --------------------------------------------------------------------------------------
def pin_rank_bruteforce(orc):
    """Position of document k = number of documents with a larger score, plus the number of
    lower-indexed documents with an equal score."""
    r = np.random.default_rng(3)
    for n_list in ([1], [5, 1, 9], [64, 3], [200]):
        scores = np.concatenate([np.round(r.random(n) * 4) / 4 for n in n_list])  # many ties
        dp = np.cumsum([0] + [n + 1 for n in n_list])
        order = orc.rank(scores, dp)
        base = 0
        for n in n_list:
            s = scores[base:base + n]
            want = np.empty(n, dtype=np.int64)
            for k in range(n):
                pos = sum(1 for j in range(n) if s[j] > s[k] or (s[j] == s[k] and j < k))
                want[pos] = k
            np.testing.assert_array_equal(order[base:base + n], want)
            base += n


# --------------------------------------------------------------------------------------
# query-only attention over a cached corpus (BlockSearch section 3.2)
# --------------------------------------------------------------------------------------
def _query_case(seed, corpus, qlens, hq=4, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    T = corpus + sum(qlens)
    bf = lambda a: workloads.f32_to_bf16_bits(a.astype(np.float32))
    K = bf(rng.standard_normal((T, hkv, d))); V = bf(rng.standard_normal((T, hkv, d)))
    Q = bf(rng.standard_normal((T - corpus, hq, d)))
    qo = np.cumsum([corpus] + list(qlens))
    return Q, K, V, qo


def pin_query_attn_no_corpus(orc):
    """corpus_len = 0: every query is plain causal attention over its own tokens (torch SDPA)."""
    Q, K, V, qo = _query_case(5, 0, [7, 1, 12, 5])
    O, _ = orc.query_attn(Q, K, V, 0, qo)
    for b in range(len(qo) - 1):
        a, e = int(qo[b]), int(qo[b + 1])
        want = _sdpa_causal(_f64(Q)[a:e], _f64(K)[a:e], _f64(V)[a:e])
        np.testing.assert_allclose(O[a:e], want, rtol=0, atol=1e-10)


def pin_query_attn_is_prompt_query_rows(orc):
    """A BlockRank prompt's final-query rows are query-only attention over the corpus made of its
    instruction and documents: compare with the rows of causal attention over the whole prompt
    (torch SDPA) and with the prompt oracle's own query rows."""
    for seed in range(3):
        w = small_case(300 + seed, hq=4, hkv=2, d=8, batch=1)
        offs = [int(x) for x in w.segment_offsets]
        qs, qe = offs[-2], offs[-1]
        Qf, Kf, Vf = _f64(w.Q), _f64(w.K), _f64(w.V)
        O, lse = orc.query_attn(w.Q[qs:qe], w.K[:qe], w.V[:qe], qs, [qs, qe])
        full = _sdpa_causal(Qf[:qe], Kf[:qe], Vf[:qe])
        np.testing.assert_allclose(O, full[qs:qe], rtol=0, atol=1e-10)
        O2, lse2 = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, rows=np.arange(qs, qe))
        np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def pin_query_attn_isolation(orc):
    """A query reads the corpus and nothing of the other queries; brute force per row."""
    corpus, qlens = 9, [4, 6, 3]
    Q, K, V, qo = _query_case(11, corpus, qlens, hq=2, hkv=1, d=4)
    O, _ = orc.query_attn(Q, K, V, corpus, qo)
    Qf, Kf, Vf = _f64(Q), _f64(K), _f64(V)
    sc = 1.0 / math.sqrt(4)
    for b in range(len(qlens)):
        for i in range(int(qo[b]), int(qo[b + 1])):
            keys = list(range(corpus)) + list(range(int(qo[b]), i + 1))
            for h in range(2):
                z = [sum(Qf[i - corpus, h, t] * Kf[j, 0, t] for t in range(4)) * sc for j in keys]
                m = max(z); e = [math.exp(v - m) for v in z]; s_ = sum(e)
                want = [sum(e[n] * Vf[j, 0, t] for n, j in enumerate(keys)) / s_ for t in range(4)]
                np.testing.assert_allclose(O[i - corpus, h], want, rtol=0, atol=1e-12)
    # changing query 1's keys/values leaves queries 0 and 2 unchanged
    K2, V2 = K.copy(), V.copy()
    K2[qo[1]:qo[2]] ^= np.uint16(0x0040); V2[qo[1]:qo[2]] ^= np.uint16(0x0040)
    O2, _ = orc.query_attn(Q, K2, V2, corpus, qo)
    for b in (0, 2):
        a, e = int(qo[b]) - corpus, int(qo[b + 1]) - corpus
        np.testing.assert_array_equal(O[a:e], O2[a:e])
    assert not np.allclose(O[qo[1] - corpus:qo[2] - corpus], O2[qo[1] - corpus:qo[2] - corpus])


# --------------------------------------------------------------------------------------
# top-B routing (BlockSearch section 5.1)
# --------------------------------------------------------------------------------------
def _routing_case(seed):
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=2, p_max=12, n_max=6, l_max=20, q_max=9, p_min=1)
    w = workloads.make_custom(prompts, 4, 2, 8, 1, seed)
    keep_ptr, keep = [0], []
    for (_, lens, _) in prompts:
        ks = sorted(rng.sample(range(len(lens)), rng.randint(0, len(lens))))
        rng.shuffle(ks)
        keep += ks
        keep_ptr.append(len(keep))
    return w, prompts, np.array(keep_ptr), np.array(keep, dtype=np.int64)


def _computed_rows(w, keep_ptr, keep, orc):
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, keep_ptr, keep)
    return np.nonzero(~dropped)[0]


def pin_routing_keep_all(orc):
    """Keeping every document is the unrouted prompt."""
    w = small_case(401, hq=4, hkv=2, d=8, batch=2)
    n_docs = [int(w.seg_ptr[b + 1] - w.seg_ptr[b] - 3) for b in range(w.num_prompts)]
    keep_ptr = np.cumsum([0] + n_docs); keep = np.concatenate([np.arange(n)[::-1] for n in n_docs])
    rows = np.arange(int(w.segment_offsets[-1]))
    O, lse = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, keep_ptr, keep, rows)
    O2, lse2 = orc.attn_rows(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def pin_routing_is_compaction(orc):
    """Routing equals dropping the documents from the prompt: gather the instruction, the kept
    documents (in prompt order) and the query into a shorter prompt and run the prompt oracle."""
    for seed in range(3):
        w, prompts, keep_ptr, keep = _routing_case(500 + seed)
        so = [int(x) for x in w.segment_offsets]; sp = [int(x) for x in w.seg_ptr]
        gather, new_offs, new_ptr = [], [], [0]
        for b, (p, lens, q) in enumerate(prompts):
            offs = so[sp[b]:sp[b + 1]]
            kept = set(int(k) for k in keep[keep_ptr[b]:keep_ptr[b + 1]])
            docs = [k for k in range(len(lens)) if k in kept]
            if not docs:
                continue  # a prompt needs at least one document; check it below by rows only
            base = len(gather)
            seg = [(offs[0], offs[1])] + [(offs[k + 1], offs[k + 2]) for k in docs] + [(offs[-2], offs[-1])]
            cur = base
            new_offs.append(cur)
            for a, e in seg:
                gather.extend(range(a, e)); cur += e - a; new_offs.append(cur)
            new_ptr.append(len(new_offs))
        if not gather:
            continue
        g = np.array(gather)
        O_c, _ = orc.attn_rows(w.Q[g], w.K[g], w.V[g], np.array(new_offs), np.array(new_ptr))
        O_r, _ = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, keep_ptr, keep, g)
        np.testing.assert_allclose(O_r, O_c, rtol=0, atol=1e-12)


def pin_routing_ignores_dropped(orc):
    """Dropped documents' keys and values change no computed row."""
    w, prompts, keep_ptr, keep = _routing_case(600)
    rows = _computed_rows(w, keep_ptr, keep, orc)
    O, _ = orc.attn_routed(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, keep_ptr, keep, rows)
    dropped = orc.dropped_tokens(w.segment_offsets, w.seg_ptr, keep_ptr, keep)
    assert dropped.any()
    K2, V2 = w.K.copy(), w.V.copy()
    K2[dropped] ^= np.uint16(0x0100); V2[dropped] ^= np.uint16(0x0100)
    O2, _ = orc.attn_routed(w.Q, K2, V2, w.segment_offsets, w.seg_ptr, keep_ptr, keep, rows)
    np.testing.assert_array_equal(O, O2)


# --------------------------------------------------------------------------------------
# SSMax ([BS] section 5.1): scores times s * ln N
# --------------------------------------------------------------------------------------
def pin_ssmax_gold_weight(orc):
    """[BS] 5.2: under SSMax a gold key scoring Delta above N equal distractors gets weight
    1 / (1 + N^(1 - s Delta)).  Built as one query token over a corpus of one gold key and
    N - 1 distractors (its own key is the N-th distractor); V marks the gold key."""
    d = 4
    for n, s, delta in [(10, 0.43, 1.0), (100, 0.43, 2.5), (1000, 0.43, 4.0), (500, 0.2, 3.0), (2, 1.0, 0.5)]:
        K = np.zeros((n + 1, 1, d)); V = np.zeros((n + 1, 1, d))
        gold = n // 2
        K[gold, 0, 0] = delta
        V[gold, 0, 0] = 1.0
        Q = np.zeros((1, 1, d)); Q[0, 0, 0] = math.sqrt(d)          # q.k / sqrt(d) = k[0]
        O, _ = orc.query_attn(Q, K, V, n, [n, n + 1], scale=orc.ssmax_scale(s, n, d))
        want = 1.0 / (1.0 + n ** (1.0 - s * delta))
        assert abs(O[0, 0, 0] - want) < 1e-12, (n, s, delta, O[0, 0, 0], want)


def pin_ssmax_readout_gold_mass(orc):
    """The readout under SSMax: one signal row, N one-token documents, the gold one Delta above
    the rest, so its mass is 1 / (1 + (N - 1) N^(-s Delta)) ([BS] 5.1 scaling applied to the
    readout's softmax over document tokens)."""
    d = 4
    for n, s, delta in [(8, 0.43, 2.0), (300, 0.43, 3.0)]:
        K = np.zeros((n + 2, 1, d))            # instruction token, n documents, query token
        gold = 1 + n // 3
        K[gold, 0, 0] = delta
        Q_S = np.zeros((1, 1, 1, d)); Q_S[0, 0, 0, 0] = math.sqrt(d)
        doc_offsets = np.arange(1, n + 2)
        scores, _ = orc.doc_scores(Q_S, K, doc_offsets, [0, n + 1], scale=orc.ssmax_scale(s, n, d))
        want = 1.0 / (1.0 + (n - 1) * n ** (-s * delta))
        assert abs(scores[gold - 1] - want) < 1e-12, (n, scores[gold - 1], want)


# --------------------------------------------------------------------------------------
# permutation-invariant positions and RoPE ([BR] 3.4; [BS] 3.2; RoFormer)
# --------------------------------------------------------------------------------------
def pin_rope_positions_golden(orc):
    """Position ids against the hand-written fixture of the pages' two rules."""
    with open(os.path.join(GOLDEN, "rope_positions.json")) as f:
        g = json.load(f)
    for key in ("blockrank", "blocksearch"):
        r = g[key]
        got = orc.rope_positions(g["segment_offsets"], g["seg_ptr"], r["query_pos0"], r["docs_after_instruction"])
        assert got.tolist() == r["positions"], (key, got.tolist())


def pin_rope_rotation_values(orc):
    """Rotation by a known angle.  d = 2: the unit vector (1, 0) at position m becomes
    (cos m, sin m).  d = 4, base 10000: the second pair turns by m * 10000^(-1/2), so exactly
    one radian at m = 100, while the first pair turns by m radians."""
    for m in (0, 1, 3, 17):
        out = orc.rope_apply(np.array([[[1.0, 0.0]]]), [m], 10000.0)
        assert np.allclose(out[0, 0], [math.cos(m), math.sin(m)], atol=1e-14)
    for inter in (False, True):
        x = np.zeros((1, 1, 4))
        a0, b0 = (0, 1) if inter else (0, 2)
        a1, b1 = (2, 3) if inter else (1, 3)
        x[0, 0, a1] = 1.0
        out = orc.rope_apply(x, [100], 10000.0, interleaved=inter)[0, 0]
        assert abs(out[a1] - math.cos(1.0)) < 1e-14 and abs(out[b1] - math.sin(1.0)) < 1e-14, (inter, out)
        assert abs(out[a0]) < 1e-15 and abs(out[b0]) < 1e-15
        x = np.zeros((1, 1, 4)); x[0, 0, b0] = 1.0                   # (0, 1) on the first pair
        out = orc.rope_apply(x, [100], 10000.0, interleaved=inter)[0, 0]
        assert abs(out[a0] + math.sin(100.0)) < 1e-13 and abs(out[b0] - math.cos(100.0)) < 1e-13


def pin_rope_relative_position(orc):
    """RoFormer's defining property: <R(m) q, R(n) k> depends only on n - m, equals
    <q, R(n - m) k>, and the rotation keeps norms."""
    rng = np.random.default_rng(5)
    for d, inter in [(8, False), (8, True), (64, False)]:
        q = rng.standard_normal((1, 1, d)); k = rng.standard_normal((1, 1, d))
        for m, n, c in [(3, 7, 100), (8192, 5, -4000), (0, 250, 37)]:
            rq = lambda x, pos: orc.rope_apply(x, [pos], 10000.0, inter)[0, 0]
            a = rq(q, m) @ rq(k, n)
            b = rq(q, m + c) @ rq(k, n + c)
            e = q[0, 0] @ rq(k, n - m)
            assert abs(a - b) < 1e-9 and abs(a - e) < 1e-9, (d, inter, m, n, a, b, e)
            assert abs(np.linalg.norm(rq(q, m)) - np.linalg.norm(q)) < 1e-12


def pin_rope_permutation_invariance(orc):
    """[BR] 3.4: with the shared document position space, a document's representation does not
    depend on its place in the list.  Rotating Q and K with the prompt's positions and running
    the block-sparse attention, each document's output rows are the same after the documents
    are permuted."""
    rng = np.random.default_rng(9)
    p, lens, q = 5, [4, 7, 3, 6], 4
    hq, hkv, d = 2, 1, 8
    def build(order):
        offs = [0, p]
        for k in order:
            offs.append(offs[-1] + lens[k])
        offs.append(offs[-1] + q)
        return offs
    Xq = {k: rng.standard_normal((lens[k], hq, d)) for k in range(len(lens))}
    Xk = {k: rng.standard_normal((lens[k], hkv, d)) for k in range(len(lens))}
    Xv = {k: rng.standard_normal((lens[k], hkv, d)) for k in range(len(lens))}
    inst = [rng.standard_normal((p, h, d)) for h in (hq, hkv, hkv)]
    qry = [rng.standard_normal((q, h, d)) for h in (hq, hkv, hkv)]
    outs = []
    for order in ([0, 1, 2, 3], [2, 0, 3, 1]):
        offs = build(order)
        Q = np.concatenate([inst[0]] + [Xq[k] for k in order] + [qry[0]])
        K = np.concatenate([inst[1]] + [Xk[k] for k in order] + [qry[1]])
        V = np.concatenate([inst[2]] + [Xv[k] for k in order] + [qry[2]])
        pos = orc.rope_positions(offs, [0, len(offs)])
        O, _ = orc.attn_rows(orc.rope_apply(Q, pos, 10000.0), orc.rope_apply(K, pos, 10000.0), V, offs,
                             [0, len(offs)], rows=np.arange(offs[-1]))
        outs.append({k: O[offs[1 + i]:offs[2 + i]] for i, k in enumerate(order)})
    for k in range(len(lens)):
        assert np.abs(outs[0][k] - outs[1][k]).max() < 1e-12, k


def pin_signal_positions(orc):
    """The readout's signal rows are each prompt's last |S| query tokens, so their positions are
    the prompt positions of those tokens."""
    rng = random.Random(13)
    for seed in range(4):
        prompts = [(p, l, max(q, 5)) for (p, l, q) in random_prompts(rng, batch=3)]
        seg, sp, _, _ = workloads.segment_tables(prompts)
        for q0, after in [(8192, True), (300, False)]:
            pos = orc.rope_positions(seg, sp, q0, after)
            sig = orc.signal_positions(seg, sp, 5, q0)
            for b in range(len(prompts)):
                end = int(seg[sp[b + 1] - 1])
                assert sig[b].tolist() == pos[end - 5:end].tolist(), (seed, b)


# --------------------------------------------------------------------------------------
# backward pass: gradients against finite differences of the pinned forward, identities,
# and autograd through a library attention
# --------------------------------------------------------------------------------------
def _bwd_case(seed, hq=4, hkv=2, d=8):
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=2, p_max=6, n_max=3, l_max=7, q_max=5)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 4000 + seed)
    nrng = np.random.default_rng(seed)
    T = w.total_tokens
    # float64 inputs, not bf16 bit patterns: finite differences need a smooth function
    Q, K, V = (nrng.standard_normal((T, h, d)) for h in (hq, hkv, hkv))
    dO = nrng.standard_normal((T, hq, d))
    return w, Q, K, V, dO


def pin_attn_bwd_finite_differences(orc):
    """Central differences of sum(O * dO), with O from the pinned forward oracle."""
    for seed in (0, 1):
        w, Q, K, V, dO = _bwd_case(seed)
        so, sp = w.segment_offsets, w.seg_ptr
        dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, so, sp)
        f = lambda q, k, v: float((orc.attn_rows(q, k, v, so, sp)[0] * dO).sum())
        rng = np.random.default_rng(seed + 50)
        eps = 1e-6
        for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
            for _ in range(12):
                ix = tuple(int(rng.integers(0, n)) for n in X.shape)
                Xp, Xm = X.copy(), X.copy()
                Xp[ix] += eps
                Xm[ix] -= eps
                args_p = {"Q": (Xp, K, V), "K": (Q, Xp, V), "V": (Q, K, Xp)}[name]
                args_m = {"Q": (Xm, K, V), "K": (Q, Xm, V), "V": (Q, K, Xm)}[name]
                fd = (f(*args_p) - f(*args_m)) / (2 * eps)
                assert abs(fd - G[ix]) < 1e-6 * max(1.0, abs(fd)), (seed, name, ix, fd, G[ix])


def pin_attn_bwd_identities(orc):
    """Every P row sums to one and every dS row to zero, so per prompt and KV head the keys' dV
    sum to the rows' dO (over the group's heads) and the keys' dK sum to zero."""
    for seed in (2, 3):
        w, Q, K, V, dO = _bwd_case(seed, hq=4, hkv=1)
        dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, w.segment_offsets, w.seg_ptr)
        so, sp = np.asarray(w.segment_offsets), np.asarray(w.seg_ptr)
        for b in range(len(sp) - 1):
            a, e = int(so[sp[b]]), int(so[sp[b + 1] - 1])
            assert np.allclose(dV[a:e, 0].sum(axis=0), dO[a:e].sum(axis=(0, 1)), atol=1e-10)
            assert np.allclose(dK[a:e, 0].sum(axis=0), 0.0, atol=1e-10)


def pin_attn_bwd_autograd(orc):
    """Against torch's autograd through scaled_dot_product_attention (float64, CPU) with the
    prompt's boolean mask."""
    w, Q, K, V, dO = _bwd_case(4, hq=4, hkv=2, d=8)
    dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, w.segment_offsets, w.seg_ptr)
    tables = orc.token_tables(w.segment_offsets, w.seg_ptr)
    T = w.total_tokens
    idx = np.arange(T)
    mask = torch.from_numpy(orc.allowed(idx[:, None], idx[None, :], tables))
    q = torch.from_numpy(Q).permute(1, 0, 2).contiguous().requires_grad_(True)      # [Hq, T, d]
    k = torch.from_numpy(K).permute(1, 0, 2).contiguous().requires_grad_(True)      # [Hkv, T, d]
    v = torch.from_numpy(V).permute(1, 0, 2).contiguous().requires_grad_(True)
    kk, vv = k.repeat_interleave(2, dim=0), v.repeat_interleave(2, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask)
    out.backward(torch.from_numpy(dO).permute(1, 0, 2))
    assert np.allclose(q.grad.permute(1, 0, 2).numpy(), dQ, atol=1e-10)
    assert np.allclose(k.grad.permute(1, 0, 2).numpy(), dK, atol=1e-10)
    assert np.allclose(v.grad.permute(1, 0, 2).numpy(), dV, atol=1e-10)


def _autograd_grads(orc, w, Q, K, V, dO, G):
    """dQ, dK, dV from torch's autograd through scaled_dot_product_attention (float64, CPU) with
    the prompt's boolean mask, KV heads repeated G times."""
    tables = orc.token_tables(w.segment_offsets, w.seg_ptr)
    idx = np.arange(w.total_tokens)
    mask = torch.from_numpy(orc.allowed(idx[:, None], idx[None, :], tables))
    q = torch.from_numpy(Q).permute(1, 0, 2).contiguous().requires_grad_(True)
    k = torch.from_numpy(K).permute(1, 0, 2).contiguous().requires_grad_(True)
    v = torch.from_numpy(V).permute(1, 0, 2).contiguous().requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, dim=0), v.repeat_interleave(G, dim=0), attn_mask=mask)
    out.backward(torch.from_numpy(dO).permute(1, 0, 2))
    return (x.grad.permute(1, 0, 2).numpy() for x in (q, k, v))


def pin_attn_bwd_sampled(orc):
    """The sampled backward (selected rows' dQ, selected keys' dK and dV) against torch's autograd
    at those entries: rows and keys of every kind, repeats, several row blocks per segment, and
    a KV-head subset whose other heads stay zero."""
    rng = random.Random(77)
    prompts = random_prompts(rng, batch=2, p_max=9, n_max=4, l_max=11, q_max=7)
    w = workloads.make_custom(prompts, 4, 2, 8, 1, 4077)
    nrng = np.random.default_rng(77)
    T = w.total_tokens
    Q, K, V = (nrng.standard_normal((T, h, 8)) for h in (4, 2, 2))
    dO = nrng.standard_normal((T, 4, 8))
    gQ, gK, gV = _autograd_grads(orc, w, Q, K, V, dO, 2)
    rows = np.concatenate([nrng.integers(0, T, 12), [0, T - 1, 5, 5]])
    keys = np.concatenate([nrng.integers(0, T, 12), [0, T - 1, 3, 3]])
    for rb in (256, 3):
        dQ, dK, dV = orc.attn_bwd_sampled(Q, K, V, dO, w.segment_offsets, w.seg_ptr, rows, keys, row_block=rb)
        assert np.allclose(dQ, gQ[rows], atol=1e-10), rb
        assert np.allclose(dK, gK[keys], atol=1e-10), rb
        assert np.allclose(dV, gV[keys], atol=1e-10), rb
    dQ, dK, dV = orc.attn_bwd_sampled(Q, K, V, dO, w.segment_offsets, w.seg_ptr, rows, keys, kv_heads=[1])
    assert np.allclose(dQ[:, 2:], gQ[rows][:, 2:], atol=1e-10) and not dQ[:, :2].any()
    assert np.allclose(dK[:, 1], gK[keys][:, 1], atol=1e-10) and not dK[:, 0].any()
    assert np.allclose(dV[:, 1], gV[keys][:, 1], atol=1e-10) and not dV[:, 0].any()


def pin_infonce(orc):
    """Equal scores give loss ln N and gradient (1/N - onehot)/tau; the gradient sums to zero per
    prompt; it matches central differences of the loss; the loss is torch's cross entropy of the
    logits s/tau."""
    L, g = orc.infonce(np.full(5, 0.3), [0, 6], [2], tau=0.05)
    assert abs(L[0] - math.log(5)) < 1e-12
    want = np.full(5, 0.2 / 0.05); want[2] -= 1.0 / 0.05
    assert np.allclose(g, want, atol=1e-12)
    rng = np.random.default_rng(1)
    s = rng.uniform(0, 1, 9); dp = [0, 5, 11]; gold = [3, 1]
    L, g = orc.infonce(s, dp, gold, tau=0.05)
    assert abs(g[:4].sum()) < 1e-9 and abs(g[4:].sum()) < 1e-9
    for i in range(9):
        sp_, sm = s.copy(), s.copy()
        sp_[i] += 1e-6; sm[i] -= 1e-6
        fd = (orc.infonce(sp_, dp, gold)[0].sum() - orc.infonce(sm, dp, gold)[0].sum()) / 2e-6
        assert abs(fd - g[i]) < 1e-5 * max(1.0, abs(fd)), (i, fd, g[i])
    ce = torch.nn.functional.cross_entropy(torch.from_numpy(s[:4] / 0.05)[None], torch.tensor([3]))
    assert abs(float(ce) - L[0]) < 1e-12


def _readout_bwd_case(seed, hq=4, hkv=2, d=8, S=3):
    rng = random.Random(seed)
    prompts = [(p, l, max(q, S)) for (p, l, q) in random_prompts(rng, batch=2, p_max=5, n_max=4, l_max=6, q_max=5)]
    w = workloads.make_custom(prompts, hq, hkv, d, S, 4100 + seed)
    nrng = np.random.default_rng(seed)
    Q_S = nrng.standard_normal((w.num_prompts, S, hq, d))
    K = nrng.standard_normal((w.total_tokens, hkv, d))
    ds = nrng.standard_normal(w.num_docs)
    return w, Q_S, K, ds


def pin_readout_bwd_finite_differences(orc):
    """Central differences of sum_k dscores_k s_k, with s from the pinned readout oracle."""
    for seed in (0, 1):
        w, Q_S, K, ds = _readout_bwd_case(seed)
        dQs, dK = orc.doc_scores_bwd(Q_S, K, w.doc_offsets, w.doc_ptr, ds)
        f = lambda qs, k: float(orc.doc_scores(qs, k, w.doc_offsets, w.doc_ptr)[0] @ ds)
        rng = np.random.default_rng(seed + 60)
        eps = 1e-6
        for _ in range(12):
            ix = tuple(int(rng.integers(0, n)) for n in Q_S.shape)
            a, b = Q_S.copy(), Q_S.copy()
            a[ix] += eps; b[ix] -= eps
            fd = (f(a, K) - f(b, K)) / (2 * eps)
            assert abs(fd - dQs[ix]) < 1e-6 * max(1.0, abs(fd)), ("Q_S", ix, fd, dQs[ix])
            jx = tuple(int(rng.integers(0, n)) for n in K.shape)
            a, b = K.copy(), K.copy()
            a[jx] += eps; b[jx] -= eps
            fd = (f(Q_S, a) - f(Q_S, b)) / (2 * eps)
            assert abs(fd - dK[jx]) < 1e-6 * max(1.0, abs(fd)), ("K", jx, fd, dK[jx])


def pin_readout_bwd_identities(orc):
    """The scores of a prompt sum to |S| whatever Q_S and K are, so a dscores constant over a
    prompt's documents has zero gradient; dK is zero on instruction and query tokens."""
    w, Q_S, K, ds = _readout_bwd_case(3)
    const = np.repeat([0.7, -1.3], [int(w.doc_ptr[1] - 1), int(w.doc_ptr[2] - w.doc_ptr[1] - 1)])
    dQs, dK = orc.doc_scores_bwd(Q_S, K, w.doc_offsets, w.doc_ptr, const)
    assert np.abs(dQs).max() < 1e-12 and np.abs(dK).max() < 1e-12
    dQs, dK = orc.doc_scores_bwd(Q_S, K, w.doc_offsets, w.doc_ptr, ds)
    kind = orc.token_tables(w.segment_offsets, w.seg_ptr)[2]
    assert np.abs(dK[kind != orc.KIND_D]).max() == 0.0 and np.abs(dK[kind == orc.KIND_D]).max() > 0


ALL_PINS = [
    pin_closed_form_counts, pin_worked_example, pin_textbook_rows, pin_textbook_rows_no_prefix,
    pin_bruteforce_chunked, pin_special_rows, pin_document_isolation, pin_readout_bruteforce,
    pin_readout_mass, pin_readout_uniform, pin_readout_permutation, pin_rank_bruteforce,
    pin_query_attn_no_corpus, pin_query_attn_is_prompt_query_rows, pin_query_attn_isolation,
    pin_routing_keep_all, pin_routing_is_compaction, pin_routing_ignores_dropped,
    pin_ssmax_gold_weight, pin_ssmax_readout_gold_mass, pin_rope_positions_golden, pin_rope_rotation_values,
    pin_rope_relative_position, pin_rope_permutation_invariance, pin_signal_positions,
    pin_attn_bwd_finite_differences, pin_attn_bwd_identities, pin_attn_bwd_autograd, pin_attn_bwd_sampled,
    pin_infonce, pin_sink_limits_and_gate, pin_sink_single_key,
    pin_readout_bwd_finite_differences, pin_readout_bwd_identities,
]
