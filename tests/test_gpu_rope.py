"""GPU parity of the rotary embedding with permutation-invariant positions (br_rope_fwd,
br_rope_signal_fwd) against the fp64 oracle, through the C ABI, and of the whole path with it:
rotation, block-sparse attention, readout and rank."""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import check_attn, check_order, check_scores, dev_bf16, log, upload
from pins import random_prompts

pytestmark = pytest.mark.gpu

BLOCKRANK = dict(query_pos0=8192, docs_after_instruction=True)
BLOCKSEARCH = dict(query_pos0=300, docs_after_instruction=False)


def bits_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of an fp64 array (through fp32), as bf16 bit patterns."""
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def pair_magnitude(X, interleaved: bool) -> np.ndarray:
    """|a| + |b| of the rotated pair each entry belongs to."""
    x = np.abs(orc.to_f64(X))
    a_idx, b_idx = orc.rope_pairs(x.shape[-1], interleaved)
    m = np.empty_like(x)
    m[..., a_idx] = x[..., a_idx] + x[..., b_idx]
    m[..., b_idx] = m[..., a_idx]
    return m


def check_rotation(got: torch.Tensor, ref: np.ndarray, X, interleaved: bool, what: str):
    """The kernel evaluates a cos - b sin (and a sin + b cos) in fp32 and rounds to bf16.  Bound:
    one bf16 ulp of the exact value plus the fp32 evaluation error, at most (|a| + |b|) * 2^-20
    (products, sum and sin/cos each within a few fp32 ulps), which matters only where the
    rotation cancels to near zero.  The result must also equal the nearest-even bf16 of the
    exact value almost everywhere (a mismatch needs the exact value within fp32 error of a
    rounding midpoint)."""
    g = bits_f64(got)
    a = np.abs(ref)
    ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.maximum(a, 1e-300))) - 7), 0.0)
    bound = ulp + pair_magnitude(X, interleaved) * 2.0 ** -20
    err = np.abs(g - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries beyond the bound, e.g. got {g[bad][:4]} "
                           f"want {ref[bad][:4]} bound {bound[bad][:4]}")
    want = round_bf16(ref).view(np.int16)
    have = got.contiguous().view(torch.int16).cpu().numpy()
    frac = float((want != have).mean())
    assert frac < 1e-3, f"{what}: {frac:.2e} of entries differ from the nearest-even bf16 of the exact rotation"
    return frac


CASES = [  # seed, Hq, Hkv, d, rule, interleaved, theta
    (0, 4, 1, 64, BLOCKRANK, False, 10000.0),
    (1, 32, 8, 128, BLOCKRANK, False, 1e6),
    (2, 8, 8, 128, BLOCKSEARCH, True, 10000.0),
    (3, 16, 2, 64, BLOCKSEARCH, False, 500000.0),
    (4, 8, 1, 128, BLOCKRANK, True, 10000.0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_q{c[4]['query_pos0']}"
                                             f"_{'adj' if c[5] else 'split'}" for c in CASES])
def test_rope_parity(case):
    seed, hq, hkv, d, rule, inter, theta = case
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=3, p_max=70, n_max=9, l_max=250, q_max=140)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 1300 + seed)
    log(f"[rope parity] seed={seed} Hq={hq} Hkv={hkv} d={d} T={w.total_tokens} rule={rule} adjacent={inter}")
    dev = upload(w)
    Qr, Kr = br.rope(dev["Q"], dev["K"], w.segment_offsets, w.seg_ptr, theta, interleaved=inter, **rule)
    torch.cuda.synchronize()
    pos = orc.rope_positions(w.segment_offsets, w.seg_ptr, **rule)
    check_rotation(Qr, orc.rope_apply(w.Q, pos, theta, inter), w.Q, inter, "Q")
    check_rotation(Kr, orc.rope_apply(w.K, pos, theta, inter), w.K, inter, "K")
    # inputs untouched out of place; in place gives the same bits
    assert torch.equal(dev["Q"], dev_bf16(w.Q)) and torch.equal(dev["K"], dev_bf16(w.K))
    q2, k2 = dev["Q"].clone(), dev["K"].clone()
    br.rope(q2, k2, w.segment_offsets, w.seg_ptr, theta, interleaved=inter, inplace=True, **rule)
    torch.cuda.synchronize()
    assert torch.equal(q2, Qr) and torch.equal(k2, Kr)


def test_rope_q_only_k_only_and_large_positions():
    rng = random.Random(11)
    prompts = random_prompts(rng, batch=2, p_max=40, n_max=5, l_max=120, q_max=60)
    w = workloads.make_custom(prompts, 8, 2, 128, 1, 1311)
    dev = upload(w)
    rule = dict(query_pos0=1_000_000, docs_after_instruction=True)
    log(f"[rope q-only / k-only] T={w.total_tokens} query_pos0=1e6")
    Qr, none_k = br.rope(dev["Q"], None, w.segment_offsets, w.seg_ptr, 10000.0, **rule)
    none_q, Kr = br.rope(None, dev["K"], w.segment_offsets, w.seg_ptr, 10000.0, **rule)
    torch.cuda.synchronize()
    assert none_k is None and none_q is None
    pos = orc.rope_positions(w.segment_offsets, w.seg_ptr, **rule)
    check_rotation(Qr, orc.rope_apply(w.Q, pos, 10000.0), w.Q, False, "Q alone")
    check_rotation(Kr, orc.rope_apply(w.K, pos, 10000.0), w.K, False, "K alone")
    Qb, Kb = br.rope(dev["Q"], dev["K"], w.segment_offsets, w.seg_ptr, 10000.0, **rule)
    torch.cuda.synchronize()
    assert torch.equal(Qb, Qr) and torch.equal(Kb, Kr)


@pytest.mark.parametrize("inter", [False, True])
def test_rope_signal_rows_match_query_rows(inter):
    rng = random.Random(21)
    prompts = random_prompts(rng, batch=3, p_max=40, n_max=6, l_max=100, q_max=50)
    prompts = [(p, l, max(q, 8)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, 32, 8, 128, 8, 1321)
    dev = upload(w)
    log(f"[rope signal] T={w.total_tokens} S=8 adjacent={inter}")
    Qr, _ = br.rope(dev["Q"], None, w.segment_offsets, w.seg_ptr, 10000.0, interleaved=inter)
    QSr = br.rope_signal(dev["Q_S"], w.segment_offsets, w.seg_ptr, 10000.0, interleaved=inter)
    torch.cuda.synchronize()
    rows = torch.as_tensor(w.signal_rows().reshape(-1), device="cuda")
    assert torch.equal(QSr.reshape(-1, 32, 128), Qr[rows]), "signal rows differ from the rotated query rows"
    spos = orc.signal_positions(w.segment_offsets, w.seg_ptr, 8)
    qs = w.Q_S.reshape(-1, 32, 128)
    check_rotation(QSr.reshape(-1, 32, 128), orc.rope_apply(qs, spos.reshape(-1), 10000.0, inter), qs, inter, "Q_S")


E2E = [(0, 32, 8, 128, BLOCKRANK, False), (1, 8, 2, 64, BLOCKSEARCH, True), (2, 16, 16, 128, BLOCKRANK, True)]


@pytest.mark.parametrize("case", E2E, ids=[f"s{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}" for c in E2E])
def test_rope_then_rank(case):
    """Rotation, attention, readout and rank on the GPU against the oracle's rotation (rounded to
    bf16, the precision the kernel stores it in) followed by the oracle's attention and readout."""
    seed, hq, hkv, d, rule, inter = case
    rng = random.Random(40 + seed)
    prompts = random_prompts(rng, batch=2, p_max=60, n_max=12, l_max=200, q_max=60)
    prompts = [(p, l, max(q, 4)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, hq, hkv, d, 4, 1340 + seed)
    log(f"[rope e2e] seed={seed} Hq={hq} Hkv={hkv} d={d} T={w.total_tokens}")
    dev = upload(w)
    so, sp = w.segment_offsets, w.seg_ptr
    Qr, Kr = br.rope(dev["Q"], dev["K"], so, sp, 10000.0, interleaved=inter, **rule)
    QSr = br.rope_signal(dev["Q_S"], so, sp, 10000.0, query_pos0=rule["query_pos0"], interleaved=inter)
    out = br.attn_fwd(Qr, Kr, dev["V"], so, sp)
    scores = br.doc_scores(QSr, Kr, w.doc_offsets, w.doc_ptr)
    order = br.sort_docs(scores, w.doc_ptr)
    torch.cuda.synchronize()
    pos = orc.rope_positions(so, sp, **rule)
    Qo = round_bf16(orc.rope_apply(w.Q, pos, 10000.0, inter))
    Ko = round_bf16(orc.rope_apply(w.K, pos, 10000.0, inter))
    spos = orc.signal_positions(so, sp, 4, rule["query_pos0"]).reshape(-1)
    QSo = round_bf16(orc.rope_apply(w.Q_S.reshape(-1, hq, d), spos, 10000.0, inter)).reshape(w.Q_S.shape)
    O_ref, _ = orc.attn_rows(Qo, Ko, w.V, so, sp, rows=np.arange(w.total_tokens))
    check_attn(out, O_ref, what="attention after rope")
    s_ref, _ = orc.doc_scores(QSo, Ko, w.doc_offsets, w.doc_ptr)
    s_gpu = scores.cpu().numpy().astype(np.float64)
    check_scores(s_gpu, s_ref, 4, what="scores after rope")
    check_order(order.cpu().numpy(), s_ref, w.doc_ptr, what="order after rope")


def test_rope_document_rows_permutation_invariant():
    """With the shared document position space, a document's attention rows come out bit-identical
    wherever the document sits in the list (positions and arithmetic do not depend on its place)."""
    rng = np.random.default_rng(3)
    p, lens, q = 48, [130, 77, 200, 64, 151], 40
    hq, hkv, d = 32, 8, 128
    f = lambda n, h: workloads.f32_to_bf16_bits(rng.standard_normal((n, h, d)).astype(np.float32))
    docs = [(f(l, hq), f(l, hkv), f(l, hkv)) for l in lens]
    inst = (f(p, hq), f(p, hkv), f(p, hkv))
    qry = (f(q, hq), f(q, hkv), f(q, hkv))
    res = []
    for order in ([0, 1, 2, 3, 4], [3, 0, 4, 2, 1]):
        offs = [0, p]
        for k in order:
            offs.append(offs[-1] + lens[k])
        offs.append(offs[-1] + q)
        cat = lambda i: np.concatenate([inst[i]] + [docs[k][i] for k in order] + [qry[i]])
        Q, K, V = dev_bf16(cat(0)), dev_bf16(cat(1)), dev_bf16(cat(2))
        so, sp = np.array(offs), np.array([0, len(offs)])
        log(f"[rope permutation] order={order}")
        Qr, Kr = br.rope(Q, K, so, sp, 10000.0)
        out = br.attn_fwd(Qr, Kr, V, so, sp)
        torch.cuda.synchronize()
        res.append({k: out[offs[1 + i]:offs[2 + i]].clone() for i, k in enumerate(order)})
    for k in range(len(lens)):
        assert torch.equal(res[0][k], res[1][k]), f"document {k} rows changed with its place in the list"


def test_rope_long_prompt_sampled_rows():
    """The long ranking prompt (T = 100,096) at full size: sampled rows against the oracle."""
    w = workloads.make("long", 0)
    dev = upload(w)
    log(f"[rope long] T={w.total_tokens}")
    Qr, Kr = br.rope(dev["Q"], dev["K"], w.segment_offsets, w.seg_ptr, 10000.0)
    torch.cuda.synchronize()
    pos = orc.rope_positions(w.segment_offsets, w.seg_ptr)
    rng = np.random.default_rng(0)
    offs = np.asarray(w.segment_offsets)
    rows = np.unique(np.concatenate([rng.integers(0, w.total_tokens, 600), offs[:-1], offs[1:] - 1,
                                     np.arange(offs[-2], offs[-1])]))
    rt = torch.as_tensor(rows, device="cuda")
    check_rotation(Qr[rt], orc.rope_apply(w.Q[rows], pos[rows], 10000.0), w.Q[rows], False, "long Q")
    check_rotation(Kr[rt], orc.rope_apply(w.K[rows], pos[rows], 10000.0), w.K[rows], False, "long K")


FUSED = [  # seed, Hq, Hkv, d, rule, interleaved
    (0, 32, 8, 128, BLOCKRANK, False), (1, 8, 2, 64, BLOCKSEARCH, True), (2, 16, 16, 128, BLOCKRANK, True),
    (3, 8, 1, 64, BLOCKRANK, False), (4, 32, 4, 128, BLOCKSEARCH, False),
]


@pytest.mark.parametrize("case", FUSED, ids=[f"s{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_q{c[4]['query_pos0']}_i{int(c[5])}"
                                             for c in FUSED])
def test_q_rotated_inside_attention_is_bit_identical(case):
    """br_attn_fwd_rope (K rotated beforehand, Q rotated by the attention kernel from a cos/sin
    table of the distinct positions) equals br_rope_fwd on Q and K followed by br_attn_fwd, bit
    for bit, output and lse; and it matches the oracle's rotate-then-attend rows."""
    seed, hq, hkv, d, rule, inter = case
    rng = random.Random(1700 + seed)
    prompts = random_prompts(rng, batch=3, p_max=60, n_max=7, l_max=140, q_max=70, p_min=0 if seed % 2 else 1)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 1800 + seed)
    dev = upload(w)
    log(f"[rope fused] seed={seed} Hq={hq} Hkv={hkv} d={d} {rule} interleaved={inter} T={w.total_tokens}")
    Qr, Kr = br.rope(dev["Q"], dev["K"], w.segment_offsets, w.seg_ptr, 10000.0, interleaved=inter, **rule)
    ref_out, ref_lse = br.attn_fwd(Qr, Kr, dev["V"], w.segment_offsets, w.seg_ptr, lse=True)
    _, Kr2 = br.rope(None, dev["K"], w.segment_offsets, w.seg_ptr, 10000.0, interleaved=inter, **rule)
    out, lse = br.attn_fwd_rope(dev["Q"], Kr2, dev["V"], w.segment_offsets, w.seg_ptr, 10000.0, interleaved=inter,
                                lse=True, **rule)
    torch.cuda.synchronize()
    assert torch.equal(Kr2, Kr)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    # and against the oracle: rotate in fp64, round to bf16 as the kernel does, attend
    pos = orc.rope_positions(w.segment_offsets, w.seg_ptr, rule["query_pos0"], rule["docs_after_instruction"])
    Qo = round_bf16(orc.rope_apply(w.Q, pos, 10000.0, inter))
    Ko = round_bf16(orc.rope_apply(w.K, pos, 10000.0, inter))
    ref, _ = orc.attn_rows(Qo, Ko, w.V, w.segment_offsets, w.seg_ptr)
    check_attn(out, ref, what="fused rope attention")


def test_q_rotated_inside_attention_long_prompt():
    """The long ranking prompt (split-key query rows, 100,096 tokens): bit-identical to the separate
    rotation followed by attention."""
    w = workloads.make("long", 0)
    dev = upload(w)
    log(f"[rope fused] long prompt T={w.total_tokens}")
    Qr, Kr = br.rope(dev["Q"], dev["K"], w.segment_offsets, w.seg_ptr, 10000.0)
    ref = br.attn_fwd(Qr, Kr, dev["V"], w.segment_offsets, w.seg_ptr)
    del Qr
    out = br.attn_fwd_rope(dev["Q"], Kr, dev["V"], w.segment_offsets, w.seg_ptr, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
