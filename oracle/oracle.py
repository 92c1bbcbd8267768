"""Plain fp64 CPU oracle for BlockRank's block-sparse prefill attention and score readout.

TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP path: it is written
from the pages' definitions, slowly and explicitly, in float64 over the same bf16 input
values the GPU reads.

Sources (page title, then section / equation):
  [BR]  "Scalable In-context Ranking with Generative Models" summary (BlockRank), section 3.4:
        "Blockwise Structured Attention" (token-type rules, chunked implementation),
        "Score computation procedure" (steps 1-4), "Efficient Attention-Based Inference".
  [BLOG] BlockRank blog post (hongjun7.github.io): sections on directed attention (mask
        matrix M with causal diagonal blocks C), complexity (allowed-pair closed form and
        the p=q=32, N=100, l=128 example), attention supervision (z, alpha', s_k and the
        identity sum_k s_k = |S|) and direct output (argmax / sorted list).
  [BS]  "Can Language Models Actually Retrieve In-Context?" (BlockSearch), section 3.2
        "Block-sparse attention": documents attend causally within their own block, the
        query block over everything and causally to itself, no instruction prefix.

Readings taken where the pages are silent or disagree (each also listed in the design notes):
  * Causality inside every segment, diagonal included ([BLOG] diagonal blocks C, [BS] 3.2);
    [BR] does not say "causal" for documents or the query.
  * Ragged segments, no padding tokens ([BLOG] ragged l_i) rather than [BR]'s padded chunks.
  * Query head h reads KV head floor(h / G), G = Hq / Hkv (grouped-query attention; the
    grouping is not on the pages).
  * Scale 1/sqrt(d) with d the head dimension, for attention and readout ([BR] step 2);
    callers may pass another scale.
  * Readout: per-head softmax over all document tokens of the prompt, summed over signal
    tokens, averaged over the Hq heads, so sum_k s_k = |S| ([BLOG]); head_scores keeps the
    per-head sums.  Sum, not mean, over signal tokens ([BR] "sum is used in practice").
  * Prompts in one call are independent: no attention across prompts, one sort per prompt.
  * Rank: descending score, ties to the lower document index.
  * Top-B routing ([BS] 5.1): dropped documents leave the attention altogether (their rows are
    not computed, no row reads their keys); the instruction and the query always stay.
  * Query-only attention over a cached corpus ([BS] 3.2, "prefill once, score many queries"):
    each query reads the whole corpus unmasked and its own tokens causally, never another
    query's tokens; the corpus is whatever precedes the queries (for BlockRank, the
    instruction and the documents).
  * SSMax ([BS] 5.1, length-aware softmax): the pre-softmax scores q.k/sqrt(d) are multiplied
    by s * ln N, N the number of documents of the prompt, natural logarithm; the same factor
    serves every attention row of the prompt and the readout, whose weights are the softmax
    of those scores.
  * Position ids ([BR] 3.4 "Permutation-invariant position embeddings"): instruction token i
    at i, token j of every document at p + j (p = instruction length), query token i at
    8192 + i.  [BS] 3.2 variant: document positions restart at 0 and the query starts at 300.
  * RoPE (RoFormer, cited by [BS] 3.2; Mistral uses it per the BlockRank analysis page): pair k
    of a head vector turns by pos * theta^(-2k/d).  Two pairings exist in practice, adjacent
    entries (2k, 2k+1) as in RoFormer's definition, or halves (k, k + d/2) as in the GPT-NeoX
    layout; both are provided.  The base theta is not on the pages: a parameter.
  * Additive sink ([BS] 5.1 and its appendix note on the sink): its equation is not on the page;
    from the text, exp(b) is appended to every row's softmax denominator (b one scalar per call,
    the layer's threshold b_L, a caller input), which equals the plain output times the gate
    sigma(lse - b) that the appendix describes, lse being the row's natural log-sum-exp of its
    scaled scores.
  * Backward ([BR] 3.4, auxiliary loss): gradients of the block-sparse attention with respect to
    Q, K and V for an upstream dO; the InfoNCE loss per prompt with temperature tau = 0.05 on the
    readout scores s_k (the sum over prompts is the total); and the readout's gradient with
    respect to Q_S and K.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

KIND_I, KIND_D, KIND_Q = 0, 1, 2


# --------------------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------------------
def to_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64; float arrays are just widened."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def token_tables(segment_offsets: np.ndarray, seg_ptr: np.ndarray):
    """Per token: prompt id, global segment id and kind (I / D / Q).

    Prompt b's segments are [o_0, o_1) = instruction, [o_k, o_{k+1}) = document k for
    k = 1..N, and the last span = final query, with o = segment_offsets[seg_ptr[b]:seg_ptr[b+1]].
    """
    so = np.asarray(segment_offsets, dtype=np.int64)
    sp = np.asarray(seg_ptr, dtype=np.int64)
    T = int(so[sp[-1] - 1])
    prompt = np.full(T, -1, dtype=np.int64)
    seg = np.full(T, -1, dtype=np.int64)
    kind = np.full(T, -1, dtype=np.int64)
    gseg = 0
    for b in range(len(sp) - 1):
        offs = so[sp[b]:sp[b + 1]]
        nseg = len(offs) - 1
        for s in range(nseg):
            a, e = int(offs[s]), int(offs[s + 1])
            prompt[a:e] = b
            seg[a:e] = gseg
            kind[a:e] = KIND_I if s == 0 else (KIND_Q if s == nseg - 1 else KIND_D)
            gseg += 1
    assert (prompt >= 0).all(), "segment table does not cover every token"
    return prompt, seg, kind


# --------------------------------------------------------------------------------------
# the mask ([BR] token-type rules; [BLOG] mask matrix M; [BS] 3.2)
# --------------------------------------------------------------------------------------
def allowed(i, j, tables) -> np.ndarray:
    """May row token i read key token j?  (broadcasting over index arrays)

    Same prompt, j <= i, and one of: j in i's own segment (causal diagonal block), j in the
    instruction (every row after it reads the whole prefix), or i in the final query (the
    query reads everything before it).
    """
    prompt, seg, kind = tables
    i = np.asarray(i); j = np.asarray(j)
    same_prompt = prompt[i] == prompt[j]
    causal = j <= i
    same_seg = seg[i] == seg[j]
    return same_prompt & causal & (same_seg | (kind[j] == KIND_I) | (kind[i] == KIND_Q))


def allowed_full_diagonal(i, j, tables) -> np.ndarray:
    """The same block pattern with each diagonal block C counted whole (no causal cut).

    This is the pattern whose size the blog's closed form counts: whole blocks C_I, C_{d_k},
    C_q plus the instruction column block for documents and the full query row block.
    """
    prompt, seg, kind = tables
    i = np.asarray(i); j = np.asarray(j)
    same_prompt = prompt[i] == prompt[j]
    same_seg = seg[i] == seg[j]
    doc_reads_prefix = (kind[i] == KIND_D) & (kind[j] == KIND_I)
    return same_prompt & (same_seg | doc_reads_prefix | (kind[i] == KIND_Q))


def count_pairs(segment_offsets, seg_ptr, full_diagonal: bool = False, row_block: int = 512) -> int:
    """Count allowed (row, key) pairs by evaluating the predicate on every pair of each prompt."""
    tables = token_tables(segment_offsets, seg_ptr)
    pred = allowed_full_diagonal if full_diagonal else allowed
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    total = 0
    for b in range(len(sp) - 1):
        a, e = int(so[sp[b]]), int(so[sp[b + 1] - 1])
        keys = np.arange(a, e)
        for r0 in range(a, e, row_block):
            rows = np.arange(r0, min(r0 + row_block, e))
            total += int(pred(rows[:, None], keys[None, :], tables).sum())
    return total


def closed_form_pairs(p: int, lengths: Sequence[int], q: int) -> int:
    """[BLOG] complexity section: p^2 + sum_i (l_i^2 + p l_i) + q (p + q + sum_i l_i)."""
    D = sum(int(l) for l in lengths)
    return p * p + sum(int(l) * int(l) + p * int(l) for l in lengths) + q * (p + q + D)


# --------------------------------------------------------------------------------------
# attention: softmax(Q K^T * scale + M) V  ([BLOG] directed attention)
# --------------------------------------------------------------------------------------
def kv_head(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query attention: query head h reads KV head floor(h / G), G = Hq / Hkv."""
    return h // (num_q_heads // num_kv_heads)


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def _masked_softmax_av(q, k, v, mask, scale):
    """q [R,d], k/v [C,d], mask [R,C] -> (out [R,d], lse [R]) in float64."""
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def _masked_softmax_sink_av(q, k, v, mask, scale, sink):
    """The same with an additive sink ([BS] 5.1, length-aware softmax): the constant exp(sink) is
    appended to every row's softmax denominator, so the weights of a row sum to less than one.
    q [R,d], k/v [C,d], mask [R,C] -> (out [R,d], lse [R]); lse is the plain log-sum-exp of the
    row's scores, without the sink."""
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v) / (l + np.exp(sink - m))
    lse = (m + np.log(l))[:, 0]
    return out, lse


def attn_dense(Q, K, V, segment_offsets, seg_ptr, scale: Optional[float] = None):
    """Materialise the whole T x T boolean mask and run masked softmax attention per head.

    For small inputs only.  Returns (O [T,Hq,d], lse [T,Hq]) in float64.
    """
    Qf, Kf, Vf = to_f64(Q), to_f64(K), to_f64(V)
    T, Hq, d = Qf.shape
    Hkv = Kf.shape[1]
    sc = _scale(d, scale)
    tables = token_tables(segment_offsets, seg_ptr)
    idx = np.arange(T)
    mask = allowed(idx[:, None], idx[None, :], tables)
    O = np.zeros((T, Hq, d)); lse = np.zeros((T, Hq))
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        O[:, h], lse[:, h] = _masked_softmax_av(Qf[:, h], Kf[:, g], Vf[:, g], mask, sc)
    return O, lse


def attn_rows(Q, K, V, segment_offsets, seg_ptr, rows=None, scale: Optional[float] = None,
              row_block: int = 256, sink: Optional[float] = None):
    """Attention for selected rows: per block of rows of one segment, evaluate the predicate
    against every key of the prompt, gather the keys any row may read, and run a dense
    float64 masked softmax over them.

    rows: absolute token indices (default: all).  sink: the additive sink's constant b ([BS] 5.1;
    None for the plain softmax), appended to every row's denominator as exp(b).  Returns
    (O [R,Hq,d], lse [R,Hq]) in the order of ``rows``; lse never includes the sink.
    """
    T = int(np.asarray(segment_offsets)[-1])
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    Kf, Vf = to_f64(K), to_f64(V)
    Hkv, d = Kf.shape[1], Kf.shape[2]
    Hq = np.asarray(Q).shape[1]
    sc = _scale(d, scale)
    tables = token_tables(segment_offsets, seg_ptr)
    prompt, seg, _ = tables
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    O = np.zeros((len(rows), Hq, d)); lse = np.zeros((len(rows), Hq))
    order = np.argsort(seg[rows], kind="stable")
    # blocks of rows that share a segment
    starts = [0] + [n for n in range(1, len(order)) if seg[rows[order[n]]] != seg[rows[order[n - 1]]]]
    starts.append(len(order))
    for a_, e_ in zip(starts[:-1], starts[1:]):
        for c0 in range(a_, e_, row_block):
            sel = order[c0:min(c0 + row_block, e_)]
            r = rows[sel]
            b = int(prompt[r[0]])
            pa, pe = int(so[sp[b]]), int(so[sp[b + 1] - 1])
            keys = np.arange(pa, pe)
            m = allowed(r[:, None], keys[None, :], tables)
            cols = keys[m.any(axis=0)]
            mc = m[:, m.any(axis=0)]
            qr = to_f64(np.asarray(Q)[r])
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                if sink is None:
                    O[sel, h], lse[sel, h] = _masked_softmax_av(qr[:, h], Kf[cols, g], Vf[cols, g], mc, sc)
                else:
                    O[sel, h], lse[sel, h] = _masked_softmax_sink_av(qr[:, h], Kf[cols, g], Vf[cols, g], mc, sc,
                                                                     float(sink))
    return O, lse


def query_attn(Q, K, V, corpus_len: int, query_offsets, scale: Optional[float] = None):
    """Query-only attention over a cached corpus ([BS] section 3.2: the query block attends over
    the whole corpus and causally to itself; the corpus keys/values are computed once and reused).

    K, V [T, Hkv, d]: the corpus [0, corpus_len) followed by the queries' own tokens; query b owns
    tokens [query_offsets[b], query_offsets[b+1]).  Q [T - corpus_len, Hq, d] holds the query rows
    only.  Row i of query b reads key j iff j < corpus_len or query_offsets[b] <= j <= i.
    Returns (O [T - corpus_len, Hq, d], lse [T - corpus_len, Hq]) in float64.
    """
    Qf, Kf, Vf = to_f64(Q), to_f64(K), to_f64(V)
    Hq, d = Qf.shape[1], Qf.shape[2]
    Hkv = Kf.shape[1]
    sc = _scale(d, scale)
    qo = [int(x) for x in query_offsets]
    O = np.zeros(Qf.shape); lse = np.zeros(Qf.shape[:2])
    for b in range(len(qo) - 1):
        qs, qe = qo[b], qo[b + 1]
        rows = np.arange(qs, qe)
        keys = np.concatenate([np.arange(0, corpus_len), np.arange(qs, qe)])
        mask = (keys[None, :] < corpus_len) | ((keys[None, :] >= qs) & (keys[None, :] <= rows[:, None]))
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            O[qs - corpus_len:qe - corpus_len, h], lse[qs - corpus_len:qe - corpus_len, h] = _masked_softmax_av(
                Qf[qs - corpus_len:qe - corpus_len, h], Kf[keys, g], Vf[keys, g], mask, sc)
    return O, lse


def dropped_tokens(segment_offsets, seg_ptr, keep_ptr, keep) -> np.ndarray:
    """Boolean per token: True for the tokens of documents that top-B routing drops."""
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    T = int(so[-1])
    out = np.zeros(T, dtype=bool)
    for b in range(len(sp) - 1):
        offs = so[sp[b]:sp[b + 1]]
        kept = set(int(k) for k in np.asarray(keep)[int(keep_ptr[b]):int(keep_ptr[b + 1])])
        for k in range(len(offs) - 3):
            if k not in kept:
                out[int(offs[k + 1]):int(offs[k + 2])] = True
    return out


def attn_routed(Q, K, V, segment_offsets, seg_ptr, keep_ptr, keep, rows, scale: Optional[float] = None):
    """Top-B routed attention ([BS] section 5.1, document-level sparse attention): only the kept
    documents take part.  Row i reads key j iff the prompt rule allows it and j is not a token of
    a dropped document (the instruction and the query are never dropped).  Dropped documents'
    own rows are not part of the output; asking for them raises.

    rows: absolute token indices.  Returns (O [R,Hq,d], lse [R,Hq]) in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    dropped = dropped_tokens(segment_offsets, seg_ptr, keep_ptr, keep)
    if dropped[rows].any():
        raise ValueError("rows of dropped documents are not computed")
    Kf, Vf = to_f64(K), to_f64(V)
    Hkv, d = Kf.shape[1], Kf.shape[2]
    Hq = np.asarray(Q).shape[1]
    sc = _scale(d, scale)
    tables = token_tables(segment_offsets, seg_ptr)
    prompt = tables[0]
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    O = np.zeros((len(rows), Hq, d)); lse = np.zeros((len(rows), Hq))
    for n, i in enumerate(rows):
        b = int(prompt[i])
        keys = np.arange(int(so[sp[b]]), int(so[sp[b + 1] - 1]))
        m = allowed(np.array([i])[:, None], keys[None, :], tables) & ~dropped[keys][None, :]
        cols = keys[m[0]]
        qi = to_f64(np.asarray(Q)[i:i + 1])
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            o, l = _masked_softmax_av(qi[:, h], Kf[cols, g], Vf[cols, g], np.ones((1, len(cols)), bool), sc)
            O[n, h], lse[n, h] = o[0], l[0]
    return O, lse


# --------------------------------------------------------------------------------------
# backward pass ([BR] 3.4 auxiliary loss: the gradient flows back through the attention)
# --------------------------------------------------------------------------------------
def attn_bwd(Q, K, V, dO, segment_offsets, seg_ptr, scale: Optional[float] = None, prompts=None):
    """Gradients of O = softmax(scale * Q K^T + M) V with respect to Q, K and V, given dO.

    Per prompt and query head h (KV head g = h // G), with the prompt's explicit mask:
        P   = softmax over the allowed keys of scale * Q K^T
        dV_g += P^T dO_h
        dP  = dO_h V_g^T
        dS  = P * (dP - rowsum(P * dP))          (the softmax Jacobian applied row by row)
        dQ_h = scale * dS K_g,   dK_g += scale * dS^T Q_h
    prompts: indices of the prompts to evaluate (default: all); other rows stay zero.
    Returns (dQ [T,Hq,d], dK [T,Hkv,d], dV [T,Hkv,d]) in float64."""
    Qf, Kf, Vf, dOf = to_f64(Q), to_f64(K), to_f64(V), to_f64(dO)
    T, Hq, d = Qf.shape
    Hkv = Kf.shape[1]
    sc = _scale(d, scale)
    tables = token_tables(segment_offsets, seg_ptr)
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    dQ, dK, dV = np.zeros_like(Qf), np.zeros_like(Kf), np.zeros_like(Vf)
    for b in (range(len(sp) - 1) if prompts is None else prompts):
        a, e = int(so[sp[b]]), int(so[sp[b + 1] - 1])
        idx = np.arange(a, e)
        mask = allowed(idx[:, None], idx[None, :], tables)
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s = np.where(mask, (Qf[a:e, h] @ Kf[a:e, g].T) * sc, -np.inf)
            P = np.exp(s - s.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dV[a:e, g] += P.T @ dOf[a:e, h]
            dP = dOf[a:e, h] @ Vf[a:e, g].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[a:e, h] = sc * (dS @ Kf[a:e, g])
            dK[a:e, g] += sc * (dS.T @ Qf[a:e, h])
    return dQ, dK, dV


def attn_bwd_sampled(Q, K, V, dO, segment_offsets, seg_ptr, rows=(), keys=(), scale: Optional[float] = None,
                     kv_heads=None, row_block: int = 256):
    """Selected entries of attn_bwd's gradients, for prompts too long for the dense per-prompt
    evaluation: dQ at the given rows, dK and dV at the given keys.

    The per-row formulas are attn_bwd's: for row i and query head h (KV head g),
        P_i  = softmax over the keys row i may read of scale * Q_i K^T
        dP_i = dO_i V^T,   dS_i = P_i * (dP_i - sum_j P_ij dP_ij)
        dQ_i = scale * dS_i K,   dK_j += scale * dS_ij Q_i,   dV_j += P_ij dO_i
    Only the rows that matter are evaluated: the selected rows, and every row that may read a
    selected key (each such row's softmax still runs over all of its keys).  Rows are taken in
    blocks of one segment, each block against the keys any of its rows may read.
    kv_heads: KV heads to evaluate (default all); the outputs of other heads stay zero.
    Returns (dQ [R,Hq,d], dK [Kn,Hkv,d], dV [Kn,Hkv,d]) in float64, in the order given."""
    Kf, Vf = to_f64(K), to_f64(V)
    Hkv, d = Kf.shape[1], Kf.shape[2]
    Hq = np.asarray(Q).shape[1]
    sc = _scale(d, scale)
    tables = token_tables(segment_offsets, seg_ptr)
    prompt, seg, _ = tables
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    keys = np.asarray(keys, dtype=np.int64).reshape(-1)
    heads = [h for h in range(Hq) if kv_heads is None or kv_head(h, Hq, Hkv) in set(kv_heads)]
    dQ = np.zeros((len(rows), Hq, d)); dK = np.zeros((len(keys), Hkv, d)); dV = np.zeros((len(keys), Hkv, d))
    # rows that may read a selected key
    readers = [rows]
    for b in np.unique(prompt[keys]):
        pa, pe = int(so[sp[b]]), int(so[sp[b + 1] - 1])
        idx = np.arange(pa, pe)
        kb = np.unique(keys[prompt[keys] == b])
        hit = np.zeros(len(idx), dtype=bool)
        for c0 in range(0, len(kb), 64):
            hit |= allowed(idx[:, None], kb[None, c0:c0 + 64], tables).any(axis=1)
        readers.append(idx[hit])
    ev = np.unique(np.concatenate(readers))
    order = np.argsort(seg[ev], kind="stable")
    starts = [0] + [n for n in range(1, len(order)) if seg[ev[order[n]]] != seg[ev[order[n - 1]]]]
    starts.append(len(order))
    for a_, e_ in zip(starts[:-1], starts[1:]):
        for c0 in range(a_, e_, row_block):
            r = ev[order[c0:min(c0 + row_block, e_)]]
            b = int(prompt[r[0]])
            pa, pe = int(so[sp[b]]), int(so[sp[b + 1] - 1])
            cand = np.arange(pa, pe)
            m = allowed(r[:, None], cand[None, :], tables)
            cols = cand[m.any(axis=0)]
            mc = m[:, m.any(axis=0)]
            qr, dor = to_f64(np.asarray(Q)[r]), to_f64(np.asarray(dO)[r])
            # output slots: selected rows in this block, selected keys among its columns
            in_block = set(r.tolist())
            q_out = [(n, int(np.searchsorted(r, rows[n]))) for n in range(len(rows)) if int(rows[n]) in in_block]
            colpos = {int(c): n for n, c in enumerate(cols)}
            k_out = [(n, colpos[int(keys[n])]) for n in range(len(keys)) if int(keys[n]) in colpos]
            for h in heads:
                g = kv_head(h, Hq, Hkv)
                s = np.where(mc, (qr[:, h] @ Kf[cols, g].T) * sc, -np.inf)
                P = np.exp(s - s.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                dP = dor[:, h] @ Vf[cols, g].T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                for n, i in q_out:
                    dQ[n, h] = sc * (dS[i] @ Kf[cols, g])
                for n, c in k_out:
                    dK[n, g] += sc * (dS[:, c] @ qr[:, h])
                    dV[n, g] += P[:, c] @ dor[:, h]
    return dQ, dK, dV


def infonce(scores, doc_ptr, gold, tau: float = 0.05):
    """[BR] auxiliary loss per prompt: L_b = -log(exp(s_gold / tau) / sum_k exp(s_k / tau)) over the
    prompt's documents; gold holds each prompt's local index of the relevant document.
    Returns (losses [B], dL/ds [sum N_b]) for the total sum_b L_b: (softmax(s / tau) - onehot) / tau."""
    s = np.asarray(scores, dtype=np.float64)
    dp = np.asarray(doc_ptr, dtype=np.int64)
    losses, grad = [], np.zeros_like(s)
    base = 0
    for b in range(len(dp) - 1):
        N = int(dp[b + 1] - dp[b] - 1)
        z = s[base:base + N] / tau
        m = z.max()
        lse = m + math.log(np.exp(z - m).sum())
        k = int(gold[b])
        losses.append(lse - z[k])
        p = np.exp(z - lse)
        p[k] -= 1.0
        grad[base:base + N] = p / tau
        base += N
    return np.asarray(losses), grad


def doc_scores_bwd(Q_S, K, doc_offsets, doc_ptr, dscores, scale: Optional[float] = None):
    """Gradient of sum_k dscores_k * s_k through the readout, with respect to Q_S and K.

    For signal row i, head h (KV head g) and document token j of document k(j):
        alpha = softmax over the prompt's document tokens of z = scale * Q_S[i,h] . K[j,g]
        dz_ij = (1/Hq) * alpha_ij * (dscores_k(j) - sum_j' alpha_ij' dscores_k(j'))
        dQ_S[i,h] = scale * sum_j dz_ij K[j,g],   dK[j,g] += scale * sum_(i, h in g) dz_ij Q_S[i,h]
    Returns (dQ_S [B,S,Hq,d], dK [T,Hkv,d]) in float64; dK is zero outside document tokens."""
    Qs, Kf = to_f64(Q_S), to_f64(K)
    B, S, Hq, d = Qs.shape
    Hkv = Kf.shape[1]
    sc = _scale(d, scale)
    do = np.asarray(doc_offsets, dtype=np.int64); dp = np.asarray(doc_ptr, dtype=np.int64)
    ds = np.asarray(dscores, dtype=np.float64)
    dQs, dK = np.zeros_like(Qs), np.zeros_like(Kf)
    base = 0
    for b in range(B):
        offs = do[dp[b]:dp[b + 1]]
        N = len(offs) - 1
        a, e = int(offs[0]), int(offs[-1])
        gj = np.repeat(ds[base:base + N], np.diff(offs))           # dscores of each token's document
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            z = (Qs[b, :, h, :] @ Kf[a:e, g, :].T) * sc
            alpha = np.exp(z - z.max(axis=1, keepdims=True))
            alpha /= alpha.sum(axis=1, keepdims=True)
            dz = alpha * (gj[None, :] - (alpha * gj[None, :]).sum(axis=1, keepdims=True)) / Hq
            dQs[b, :, h, :] = sc * (dz @ Kf[a:e, g, :])
            dK[a:e, g, :] += sc * (dz.T @ Qs[b, :, h, :])
        base += N
    return dQs, dK


# --------------------------------------------------------------------------------------
# length-aware softmax scaling ([BS] section 5.1, SSMax)
# --------------------------------------------------------------------------------------
def ssmax_scale(s: float, n_docs: int, head_dim: int) -> float:
    """Factor on q.k under SSMax: the pre-softmax score q.k / sqrt(d) times s * ln N.

    N = n_docs, the corpus size in documents ([BS] 5.1 multiplies by s log N so that a gold
    document scoring Delta above N distractors keeps weight 1 / (1 + N^(1 - s Delta)))."""
    if n_docs < 1 or head_dim < 1:
        raise ValueError("n_docs and head_dim must be positive")
    return float(s) * math.log(n_docs) / math.sqrt(head_dim)


# --------------------------------------------------------------------------------------
# permutation-invariant positions and rotary embedding ([BR] 3.4; [BS] 3.2)
# --------------------------------------------------------------------------------------
def rope_positions(segment_offsets, seg_ptr, query_pos0: int = 8192,
                   docs_after_instruction: bool = True) -> np.ndarray:
    """Position id of every token ([BR] 3.4 "Permutation-invariant position embeddings").

    Instruction token i -> i.  Token j of any document -> j + p when docs_after_instruction
    (p = the prompt's instruction length, so every document starts at p whatever its place in
    the list), else j ([BS] 3.2: positions reset at each document start).  Query token i ->
    query_pos0 + i (8192 in [BR]; 300 in [BS]).  Returns int64 [T]."""
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    pos = np.full(int(so[sp[-1] - 1]), -1, dtype=np.int64)
    for b in range(len(sp) - 1):
        offs = [int(x) for x in so[sp[b]:sp[b + 1]]]
        p = offs[1] - offs[0]
        for t in range(offs[0], offs[1]):                      # instruction
            pos[t] = t - offs[0]
        for k in range(1, len(offs) - 2):                      # documents d_1 .. d_N
            for t in range(offs[k], offs[k + 1]):
                pos[t] = (t - offs[k]) + (p if docs_after_instruction else 0)
        for t in range(offs[-2], offs[-1]):                    # final query
            pos[t] = query_pos0 + (t - offs[-2])
    assert (pos >= 0).all(), "segment table does not cover every token"
    return pos


def rope_pairs(d: int, interleaved: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Indices (a_k, b_k) of the k-th rotated pair, k = 0..d/2-1."""
    k = np.arange(d // 2)
    return (2 * k, 2 * k + 1) if interleaved else (k, k + d // 2)


def rope_apply(X, positions, theta: float, interleaved: bool = False) -> np.ndarray:
    """Rotary embedding of X [R, H, d] at positions [R] in float64.

    Pair k = (a_k, b_k) turns by the angle pos * theta^(-2k/d):
        a' = a cos - b sin,   b' = a sin + b cos."""
    Xf = to_f64(X)
    d = Xf.shape[-1]
    a_idx, b_idx = rope_pairs(d, interleaved)
    freq = float(theta) ** (-2.0 * np.arange(d // 2) / d)          # [d/2]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]  # [R, d/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = Xf[..., a_idx], Xf[..., b_idx]
    out = np.empty_like(Xf)
    out[..., a_idx] = a * c - b * s
    out[..., b_idx] = a * s + b * c
    return out


def signal_positions(segment_offsets, seg_ptr, n_signal: int, query_pos0: int = 8192) -> np.ndarray:
    """Positions of each prompt's last n_signal query tokens (the readout's signal rows), [B, S]."""
    so = np.asarray(segment_offsets, dtype=np.int64); sp = np.asarray(seg_ptr, dtype=np.int64)
    out = []
    for b in range(len(sp) - 1):
        qlen = int(so[sp[b + 1] - 1] - so[sp[b + 1] - 2])
        out.append(query_pos0 + np.arange(qlen - n_signal, qlen))
    return np.asarray(out, dtype=np.int64)


# --------------------------------------------------------------------------------------
# score readout ([BR] score computation steps 1-4; [BLOG] attention supervision)
# --------------------------------------------------------------------------------------
def doc_scores(Q_S, K, doc_offsets, doc_ptr, num_q_heads: Optional[int] = None,
               scale: Optional[float] = None):
    """s_k = (1/Hq) sum_h sum_{i in S} sum_{j in d_k} alpha'_{ihj}, alpha' = softmax over all
    document tokens of the prompt of z_{ihj} = Q_S[i,h] . K[j, h/G] * scale.

    Q_S [B, S, Hq, d]; K [T, Hkv, d]; doc_offsets / doc_ptr as in the segment-table format.
    Returns (scores [sum N_b], head_scores [Hq, sum N_b]) in float64, where head_scores[h, k]
    is the signal-token sum for head h alone (scores = head_scores.mean(axis=0)).
    """
    Qs, Kf = to_f64(Q_S), to_f64(K)
    B, S, Hq, d = Qs.shape
    Hkv = Kf.shape[1]
    sc = _scale(d, scale)
    do = np.asarray(doc_offsets, dtype=np.int64); dp = np.asarray(doc_ptr, dtype=np.int64)
    n_total = int(len(do) - B)
    head_scores = np.zeros((Hq, n_total))
    base = 0
    for b in range(B):
        offs = do[dp[b]:dp[b + 1]]
        N = len(offs) - 1
        a, e = int(offs[0]), int(offs[-1])
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            z = (Qs[b, :, h, :] @ Kf[a:e, g, :].T) * sc          # [S, D]
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)
            alpha = w / w.sum(axis=1, keepdims=True)              # softmax over T_docs
            per_doc = np.add.reduceat(alpha, offs[:-1] - a, axis=1)  # [S, N]
            head_scores[h, base:base + N] = per_doc.sum(axis=0)    # sum over signal tokens
        base += N
    return head_scores.mean(axis=0), head_scores


def rank(scores, doc_ptr) -> np.ndarray:
    """Per prompt, local document indices in descending score order, ties to the lower index
    ([BR] argmax / arg-top-K; [BLOG] direct output: a sorted list)."""
    s = np.asarray(scores)
    dp = np.asarray(doc_ptr, dtype=np.int64)
    out: List[int] = []
    base = 0
    for b in range(len(dp) - 1):
        N = int(dp[b + 1] - dp[b] - 1)
        local = [float(x) for x in s[base:base + N]]
        out.extend(sorted(range(N), key=lambda k: (-local[k], k)))
        base += N
    return np.asarray(out, dtype=np.int32)


def allowed_pair_counts(segment_offsets, seg_ptr) -> Tuple[int, int]:
    """(exact causal count, count with diagonal blocks whole), both by brute-force counting."""
    return (count_pairs(segment_offsets, seg_ptr, False), count_pairs(segment_offsets, seg_ptr, True))
