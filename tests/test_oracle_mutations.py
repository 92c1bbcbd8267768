"""Plant plausible mistakes in the oracle (CPU only) and require some pin to catch each.

Every mutation swaps one oracle function for a broken copy; the pins then run against the
patched module.  A mutation that no pin detects would mean the pins leave that part of the
oracle unchecked.
"""
import math

import numpy as np
import pytest

import oracle.oracle as orc
from pins import ALL_PINS

I, D, Q = orc.KIND_I, orc.KIND_D, orc.KIND_Q


def _no_causal(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (prompt[i] == prompt[j]) & ((seg[i] == seg[j]) | ((kind[j] == I) & (j <= i)) | (kind[i] == Q))


def _docs_skip_prefix(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (prompt[i] == prompt[j]) & (j <= i) & ((seg[i] == seg[j]) | (kind[i] == Q))


def _query_skips_docs(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (prompt[i] == prompt[j]) & (j <= i) & ((seg[i] == seg[j]) | (kind[j] == I))


def _cross_prompt(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (j <= i) & ((seg[i] == seg[j]) | (kind[j] == I) | (kind[i] == Q))


def _docs_read_query(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (prompt[i] == prompt[j]) & (j <= i) & ((seg[i] == seg[j]) | (kind[j] == I) | (kind[i] == Q)) \
        | ((prompt[i] == prompt[j]) & (kind[i] == D) & (kind[j] == Q))


def _closed_form_no_prefix_term(p, lengths, q):
    D_ = sum(lengths)
    return p * p + sum(l * l for l in lengths) + q * (p + q + D_)


def _full_diag_no_query(i, j, t):
    prompt, seg, kind = t
    i = np.asarray(i); j = np.asarray(j)
    return (prompt[i] == prompt[j]) & ((seg[i] == seg[j]) | ((kind[i] == D) & (kind[j] == I)))


def _gqa_modulo(h, hq, hkv):
    return h % hkv


def _softmax_no_scale(q, k, v, mask, scale):
    return _ORIG_SOFTMAX(q, k, v, mask, 1.0)


def _softmax_sum_not_normalised(q, k, v, mask, scale):
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p @ v, m[:, 0]


def _scores_mean_over_signal(Q_S, K, doc_offsets, doc_ptr, num_q_heads=None, scale=None):
    s, hs = _ORIG_SCORES(Q_S, K, doc_offsets, doc_ptr, num_q_heads, scale)
    S = np.asarray(Q_S).shape[1]
    return s / S, hs / S


def _scores_sum_over_heads(Q_S, K, doc_offsets, doc_ptr, num_q_heads=None, scale=None):
    s, hs = _ORIG_SCORES(Q_S, K, doc_offsets, doc_ptr, num_q_heads, scale)
    return hs.sum(axis=0), hs


def _scores_softmax_over_prompt(Q_S, K, doc_offsets, doc_ptr, num_q_heads=None, scale=None):
    # normalise over the documents plus the token before them (an instruction/query leak)
    Qs, Kf = orc.to_f64(Q_S), orc.to_f64(K)
    B, S, Hq, d = Qs.shape
    Hkv = Kf.shape[1]
    sc = 1 / math.sqrt(d)
    do = np.asarray(doc_offsets, dtype=np.int64); dp = np.asarray(doc_ptr, dtype=np.int64)
    hs = np.zeros((Hq, len(do) - B)); base = 0
    for b in range(B):
        offs = do[dp[b]:dp[b + 1]]; N = len(offs) - 1
        a, e = int(offs[0]), int(offs[-1])
        lo = max(a - 1, 0)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            z = (Qs[b, :, h] @ Kf[lo:e, g].T) * sc
            w = np.exp(z - z.max(1, keepdims=True)); w /= w.sum(1, keepdims=True)
            hs[h, base:base + N] = np.add.reduceat(w[:, a - lo:], offs[:-1] - a, axis=1).sum(0)
        base += N
    return hs.mean(0), hs


def _scores_shifted_boundaries(Q_S, K, doc_offsets, doc_ptr, num_q_heads=None, scale=None):
    do = np.asarray(doc_offsets).copy()
    B = len(doc_ptr) - 1
    for b in range(B):
        a, e = doc_ptr[b], doc_ptr[b + 1]
        inner = do[a + 1:e - 1]
        do[a + 1:e - 1] = np.minimum(inner + 1, do[e - 1] - 1)
    return _ORIG_SCORES(Q_S, K, do, doc_ptr, num_q_heads, scale)


def _rank_ties_high(scores, doc_ptr):
    s = np.asarray(scores); dp = np.asarray(doc_ptr); out = []; base = 0
    for b in range(len(dp) - 1):
        N = int(dp[b + 1] - dp[b] - 1)
        loc = list(s[base:base + N])
        out.extend(sorted(range(N), key=lambda k: (-loc[k], -k)))
        base += N
    return np.asarray(out, dtype=np.int32)


def _rank_ascending(scores, doc_ptr):
    s = np.asarray(scores); dp = np.asarray(doc_ptr); out = []; base = 0
    for b in range(len(dp) - 1):
        N = int(dp[b + 1] - dp[b] - 1)
        loc = list(s[base:base + N])
        out.extend(sorted(range(N), key=lambda k: (loc[k], k)))
        base += N
    return np.asarray(out, dtype=np.int32)


_ORIG_SOFTMAX = orc._masked_softmax_av
_ORIG_SCORES = orc.doc_scores

def _query_no_causal(Q, K, V, corpus_len, query_offsets, scale=None):
    """query rows read all of their own query's tokens"""
    Qf, Kf, Vf = orc.to_f64(Q), orc.to_f64(K), orc.to_f64(V)
    Hq, d = Qf.shape[1], Qf.shape[2]
    sc = orc._scale(d, scale)
    O = np.zeros(Qf.shape); lse = np.zeros(Qf.shape[:2])
    qo = [int(x) for x in query_offsets]
    for b in range(len(qo) - 1):
        qs, qe = qo[b], qo[b + 1]
        keys = np.r_[0:corpus_len, qs:qe]
        mask = np.ones((qe - qs, len(keys)), dtype=bool)
        for h in range(Hq):
            g = orc.kv_head(h, Hq, Kf.shape[1])
            O[qs - corpus_len:qe - corpus_len, h], lse[qs - corpus_len:qe - corpus_len, h] = orc._masked_softmax_av(
                Qf[qs - corpus_len:qe - corpus_len, h], Kf[keys, g], Vf[keys, g], mask, sc)
    return O, lse


def _query_reads_previous_queries(Q, K, V, corpus_len, query_offsets, scale=None):
    """query rows also read earlier queries' tokens (the corpus grows with each query)"""
    qo = [int(x) for x in query_offsets]
    O = np.zeros(np.asarray(Q).shape, dtype=np.float64); lse = np.zeros(np.asarray(Q).shape[:2])
    for b in range(len(qo) - 1):
        a, e = qo[b], qo[b + 1]
        o, l = _real_query_attn(np.asarray(Q)[a - corpus_len:e - corpus_len], np.asarray(K)[:e], np.asarray(V)[:e],
                                a, [a, e], scale)
        O[a - corpus_len:e - corpus_len] = o
        lse[a - corpus_len:e - corpus_len] = l
    return O, lse


def _query_skips_corpus(Q, K, V, corpus_len, query_offsets, scale=None):
    """query rows read only their own tokens"""
    qo = [int(x) for x in query_offsets]
    O = np.zeros(np.asarray(Q).shape, dtype=np.float64); lse = np.zeros(np.asarray(Q).shape[:2])
    for b in range(len(qo) - 1):
        a, e = qo[b], qo[b + 1]
        o, l = _real_query_attn(np.asarray(Q)[a - corpus_len:e - corpus_len], np.asarray(K)[a:e], np.asarray(V)[a:e],
                                0, [0, e - a], scale)
        O[a - corpus_len:e - corpus_len] = o
        lse[a - corpus_len:e - corpus_len] = l
    return O, lse


_real_query_attn = orc.query_attn


def _routing_reads_dropped(Q, K, V, so, sp, keep_ptr, keep, rows, scale=None):
    """query rows still read the dropped documents (routing ignored)"""
    return orc.attn_rows(Q, K, V, so, sp, rows=rows, scale=scale)


def _routing_drops_everything(Q, K, V, so, sp, keep_ptr, keep, rows, scale=None):
    """the query reads no document at all (the kept list ignored for its keys)"""
    rows = np.asarray(rows, dtype=np.int64)
    kind = orc.token_tables(so, sp)[2]
    O, lse = _real_attn_routed(Q, K, V, so, sp, keep_ptr, keep, rows, scale)
    qrows = rows[kind[rows] == orc.KIND_Q]
    if len(qrows):
        n = len(np.asarray(sp)) - 1
        # a keep list that keeps nothing, applied to the query rows only
        o2, l2 = _real_attn_routed(Q, K, V, so, sp, np.zeros(n + 1, dtype=np.int64), np.zeros(0, dtype=np.int64),
                                   qrows, scale)
        sel = kind[rows] == orc.KIND_Q
        O[sel], lse[sel] = o2, l2
    return O, lse


_real_attn_routed = orc.attn_routed
_real_bwd_sampled = orc.attn_bwd_sampled



_real_ssmax = orc.ssmax_scale
_real_positions = orc.rope_positions


def _ssmax_log2(s, n_docs, head_dim):
    """log base 2 instead of the natural log"""
    return float(s) * math.log2(n_docs) / math.sqrt(head_dim)


def _ssmax_drops_sqrt_d(s, n_docs, head_dim):
    """s * ln N used as the whole factor on q.k (the 1/sqrt(d) of the scores forgotten)"""
    return float(s) * math.log(n_docs)


def _positions_sequential(segment_offsets, seg_ptr, query_pos0=8192, docs_after_instruction=True):
    """ordinary sequential positions across each prompt"""
    so = np.asarray(segment_offsets); sp = np.asarray(seg_ptr)
    pos = np.zeros(int(so[sp[-1] - 1]), dtype=np.int64)
    for b in range(len(sp) - 1):
        a, e = int(so[sp[b]]), int(so[sp[b + 1] - 1])
        pos[a:e] = np.arange(e - a)
    return pos


def _positions_docs_from_zero(segment_offsets, seg_ptr, query_pos0=8192, docs_after_instruction=True):
    """documents restart at 0 even under the instruction-offset rule"""
    return _real_positions(segment_offsets, seg_ptr, query_pos0, False)


def _positions_query_off_by_one(segment_offsets, seg_ptr, query_pos0=8192, docs_after_instruction=True):
    """the query starts one position late"""
    return _real_positions(segment_offsets, seg_ptr, query_pos0 + 1, docs_after_instruction)


def _rope_generic(X, positions, theta, interleaved=False, sign=1.0, expo=2.0, force_half=False):
    Xf = orc.to_f64(X)
    d = Xf.shape[-1]
    k = np.arange(d // 2)
    a_idx, b_idx = (k, k + d // 2) if (force_half or not interleaved) else (2 * k, 2 * k + 1)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * (float(theta) ** (-expo * k / d))[None, :]
    c, sn = np.cos(ang)[:, None, :], sign * np.sin(ang)[:, None, :]
    a, b = Xf[..., a_idx], Xf[..., b_idx]
    out = np.empty_like(Xf)
    out[..., a_idx] = a * c - b * sn
    out[..., b_idx] = a * sn + b * c
    return out


def _rope_sin_sign(X, positions, theta, interleaved=False):
    """rotation by the negative angle"""
    return _rope_generic(X, positions, theta, interleaved, sign=-1.0)


def _rope_freq_exponent(X, positions, theta, interleaved=False):
    """frequencies theta^(-k/d) instead of theta^(-2k/d)"""
    return _rope_generic(X, positions, theta, interleaved, expo=1.0)


def _rope_ignores_pairing(X, positions, theta, interleaved=False):
    """half-split pairs whatever the pairing asked for"""
    return _rope_generic(X, positions, theta, interleaved, force_half=True)


_real_attn_bwd = orc.attn_bwd
_real_infonce = orc.infonce
_real_readout_bwd = orc.doc_scores_bwd


def _attn_bwd_generic(Q, K, V, dO, so, sp, scale=None, prompts=None, center=True, group=True, dk_scale=True):
    Qf, Kf, Vf, dOf = orc.to_f64(Q), orc.to_f64(K), orc.to_f64(V), orc.to_f64(dO)
    T, Hq, d = Qf.shape
    Hkv = Kf.shape[1]
    sc = orc._scale(d, scale)
    tables = orc.token_tables(so, sp)
    so_, sp_ = np.asarray(so), np.asarray(sp)
    dQ, dK, dV = np.zeros_like(Qf), np.zeros_like(Kf), np.zeros_like(Vf)
    for b in range(len(sp_) - 1):
        a, e = int(so_[sp_[b]]), int(so_[sp_[b + 1] - 1])
        idx = np.arange(a, e)
        mask = orc.allowed(idx[:, None], idx[None, :], tables)
        for h in range(Hq):
            g = orc.kv_head(h, Hq, Hkv)
            sco = np.where(mask, (Qf[a:e, h] @ Kf[a:e, g].T) * sc, -np.inf)
            P = np.exp(sco - sco.max(axis=1, keepdims=True)); P /= P.sum(axis=1, keepdims=True)
            dP = dOf[a:e, h] @ Vf[a:e, g].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True)) if center else P * dP
            dQ[a:e, h] = sc * (dS @ Kf[a:e, g])
            if group or h % (Hq // Hkv) == 0:
                dV[a:e, g] += P.T @ dOf[a:e, h]
                dK[a:e, g] += (sc if dk_scale else 1.0) * (dS.T @ Qf[a:e, h])
    return dQ, dK, dV


def _attn_bwd_no_centering(*a, **k):
    """dS = P * dP (the softmax Jacobian's row-sum term dropped)"""
    return _attn_bwd_generic(*a, center=False, **k)


def _attn_bwd_first_head_only(*a, **k):
    """dK and dV take only the first query head of each KV group"""
    return _attn_bwd_generic(*a, group=False, **k)


def _attn_bwd_dk_unscaled(*a, **k):
    """dK without the softmax scale"""
    return _attn_bwd_generic(*a, dk_scale=False, **k)


def _infonce_sign(scores, doc_ptr, gold, tau=0.05):
    """gradient with the wrong sign"""
    L, g = _real_infonce(scores, doc_ptr, gold, tau)
    return L, -g


def _infonce_no_tau(scores, doc_ptr, gold, tau=0.05):
    """gradient missing the 1/tau of the logits"""
    L, g = _real_infonce(scores, doc_ptr, gold, tau)
    return L, g * tau


def _readout_bwd_no_centering(Q_S, K, doc_offsets, doc_ptr, dscores, scale=None):
    """dz = alpha * dscores (the softmax Jacobian's centering dropped)"""
    Qs, Kf = orc.to_f64(Q_S), orc.to_f64(K)
    B, S, Hq, d = Qs.shape
    sc = orc._scale(d, scale)
    do, dp = np.asarray(doc_offsets), np.asarray(doc_ptr)
    ds = np.asarray(dscores, dtype=np.float64)
    dQs, dK = np.zeros_like(Qs), np.zeros_like(Kf)
    base = 0
    for b in range(B):
        offs = do[dp[b]:dp[b + 1]]; N = len(offs) - 1; a, e = int(offs[0]), int(offs[-1])
        gj = np.repeat(ds[base:base + N], np.diff(offs))
        for h in range(Hq):
            g = orc.kv_head(h, Hq, Kf.shape[1])
            z = (Qs[b, :, h, :] @ Kf[a:e, g, :].T) * sc
            al = np.exp(z - z.max(axis=1, keepdims=True)); al /= al.sum(axis=1, keepdims=True)
            dz = al * gj[None, :] / Hq
            dQs[b, :, h, :] = sc * (dz @ Kf[a:e, g, :])
            dK[a:e, g, :] += sc * (dz.T @ Qs[b, :, h, :])
        base += N
    return dQs, dK


def _readout_bwd_sum_heads(Q_S, K, doc_offsets, doc_ptr, dscores, scale=None):
    """gradient of the head sum instead of the head mean (1/Hq dropped)"""
    dQs, dK = _real_readout_bwd(Q_S, K, doc_offsets, doc_ptr, dscores, scale)
    Hq = np.asarray(Q_S).shape[2]
    return dQs * Hq, dK * Hq


def _bwd_sampled_own_segment_readers(Q, K, V, dO, so, sp, rows=(), keys=(), scale=None, kv_heads=None,
                                     row_block=256):
    """dK and dV of a key summed over the rows of its own segment only (the query rows, and for an
    instruction key the document rows, forgotten)"""
    tables = orc.token_tables(so, sp)
    seg = tables[1]
    keys = np.asarray(keys, dtype=np.int64).reshape(-1)
    dQ = _real_bwd_sampled(Q, K, V, dO, so, sp, rows, (), scale, kv_heads, row_block)[0]
    Kf, Vf = orc.to_f64(K), orc.to_f64(V)
    dK, dV = np.zeros((len(keys),) + Kf.shape[1:]), np.zeros((len(keys),) + Vf.shape[1:])
    for n, j in enumerate(keys):
        own = np.flatnonzero(seg == seg[j])
        _, full_k, full_v = orc.attn_bwd(Q, K, V, np.where(np.isin(np.arange(len(seg)), own)[:, None, None], dO, 0.0),
                                         so, sp, scale)
        dK[n], dV[n] = full_k[j], full_v[j]
    return dQ, dK, dV


def _sink_wrong_sign(q, k, v, mask, scale, sink):
    """exp(-b) appended to the denominator instead of exp(b)"""
    return _ORIG_SINK(q, k, v, mask, scale, -sink)


def _sink_outside_shift(q, k, v, mask, scale, sink):
    """exp(b) added to the max-shifted sum without the same shift"""
    s_ = (q @ k.T) * scale
    s_ = np.where(mask, s_, -np.inf)
    m = s_.max(axis=1, keepdims=True)
    p = np.exp(s_ - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / (l + np.exp(sink)), (m + np.log(l))[:, 0]


_ORIG_SINK = orc._masked_softmax_sink_av


MUTATIONS = {
    "mask_no_causal": ("allowed", _no_causal),
    "mask_docs_skip_prefix": ("allowed", _docs_skip_prefix),
    "mask_query_skips_docs": ("allowed", _query_skips_docs),
    "mask_cross_prompt": ("allowed", _cross_prompt),
    "mask_docs_read_query": ("allowed", _docs_read_query),
    "closed_form_drops_pl": ("closed_form_pairs", _closed_form_no_prefix_term),
    "full_diag_drops_query_rows": ("allowed_full_diagonal", _full_diag_no_query),
    "gqa_modulo": ("kv_head", _gqa_modulo),
    "softmax_no_scale": ("_masked_softmax_av", _softmax_no_scale),
    "softmax_not_normalised": ("_masked_softmax_av", _softmax_sum_not_normalised),
    "scores_mean_over_signal": ("doc_scores", _scores_mean_over_signal),
    "scores_sum_over_heads": ("doc_scores", _scores_sum_over_heads),
    "scores_softmax_leaks_outside_docs": ("doc_scores", _scores_softmax_over_prompt),
    "scores_shifted_boundaries": ("doc_scores", _scores_shifted_boundaries),
    "rank_ties_high": ("rank", _rank_ties_high),
    "rank_ascending": ("rank", _rank_ascending),
    "query_no_causal": ("query_attn", _query_no_causal),
    "query_reads_previous_queries": ("query_attn", _query_reads_previous_queries),
    "query_skips_corpus": ("query_attn", _query_skips_corpus),
    "routing_reads_dropped": ("attn_routed", _routing_reads_dropped),
    "routing_drops_everything": ("attn_routed", _routing_drops_everything),
    "ssmax_log2": ("ssmax_scale", _ssmax_log2),
    "ssmax_drops_sqrt_d": ("ssmax_scale", _ssmax_drops_sqrt_d),
    "positions_sequential": ("rope_positions", _positions_sequential),
    "positions_docs_from_zero": ("rope_positions", _positions_docs_from_zero),
    "positions_query_off_by_one": ("rope_positions", _positions_query_off_by_one),
    "rope_sin_sign": ("rope_apply", _rope_sin_sign),
    "rope_freq_exponent": ("rope_apply", _rope_freq_exponent),
    "rope_ignores_pairing": ("rope_apply", _rope_ignores_pairing),
    "attn_bwd_no_centering": ("attn_bwd", _attn_bwd_no_centering),
    "attn_bwd_first_head_only": ("attn_bwd", _attn_bwd_first_head_only),
    "attn_bwd_dk_unscaled": ("attn_bwd", _attn_bwd_dk_unscaled),
    "bwd_sampled_own_segment_readers": ("attn_bwd_sampled", _bwd_sampled_own_segment_readers),
    "infonce_sign": ("infonce", _infonce_sign),
    "sink_wrong_sign": ("_masked_softmax_sink_av", _sink_wrong_sign),
    "sink_outside_shift": ("_masked_softmax_sink_av", _sink_outside_shift),
    "infonce_no_tau": ("infonce", _infonce_no_tau),
    "readout_bwd_no_centering": ("doc_scores_bwd", _readout_bwd_no_centering),
    "readout_bwd_sum_heads": ("doc_scores_bwd", _readout_bwd_sum_heads),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutation {name}"
