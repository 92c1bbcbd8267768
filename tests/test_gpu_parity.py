"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on seeded inputs.

Tolerances: attention max-abs <= 2e-2, LSE relative 1e-3, scores relative 1e-3 (+1e-6*|S|),
argmax / order agreement wherever the oracle's gap exceeds 1e-3, document rows bit-exact under
changes to other documents, and bitwise run-to-run determinism.
"""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import (ATTN_ATOL, LSE_RTOL, check_attn, check_order, check_scores, log, run_attn, to_f64,
                      upload)
from pins import random_prompts

pytestmark = pytest.mark.gpu


def _full_check(w, what, scale=0.0):
    log(f"[gpu] {what}: T={w.total_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim}")
    dev = upload(w)
    out, lse = run_attn(w, dev, lse=True, scale=scale)
    sc = None if scale <= 0 else scale
    ref, ref_lse = orc.attn_dense(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr, scale=sc)
    err = check_attn(out, ref, what=what)
    lg = to_f64(lse)
    rel = np.abs(lg - ref_lse) / np.maximum(np.abs(ref_lse), 1.0)
    assert rel.max() <= LSE_RTOL, f"{what}: lse rel err {rel.max():.3e}"
    scores, hs = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, head_scores=True,
                               softmax_scale=scale)
    order = br.sort_docs(scores, w.doc_ptr)
    torch.cuda.synchronize()
    ref_s, ref_hs = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr, scale=sc)
    check_scores(scores.cpu().numpy().astype(np.float64), ref_s, w.n_signal, what)
    check_scores(hs.cpu().numpy().astype(np.float64).ravel(), ref_hs.ravel(), w.n_signal, what + " head_scores")
    check_order(order.cpu().numpy(), ref_s, w.doc_ptr, what)
    return err


@pytest.mark.parametrize("seed", range(10))
def test_tiny_config(seed):
    w = workloads.make("tiny", seed)
    _full_check(w, f"tiny seed={seed}")


SHAPES = [(1, 1, 64), (2, 1, 64), (4, 1, 128), (8, 1, 64), (8, 2, 128), (32, 8, 128), (4, 4, 128), (16, 2, 64),
          (8, 4, 128)]


@pytest.mark.parametrize("case", range(18))
def test_random_small_tables(case):
    rng = random.Random(1000 + case)
    hq, hkv, d = SHAPES[case % len(SHAPES)]
    prompts = random_prompts(rng, batch=rng.randint(1, 3), p_max=40, n_max=6, l_max=70, q_max=40,
                             p_min=0 if case % 4 == 0 else 1)
    prompts = [(p, l, max(q, 2)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, hq, hkv, d, 2, 1000 + case)
    _full_check(w, f"random case={case} prompts={prompts}")


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (32, 8, 128)])
def test_degenerate_segments(hq, hkv, d):
    """The smallest segments: a one-token query carrying the one signal row, one- and two-token
    documents, an empty and a one-token instruction, a prompt with a single document."""
    prompts = [(0, [1, 2, 1], 1), (1, [1], 1), (0, [2], 1), (1, [1, 1, 2, 1], 1)]
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 77)
    _full_check(w, f"degenerate segments hq={hq} hkv={hkv} d={d}")


@pytest.mark.parametrize("case", range(4))
def test_ragged_tails_and_long_segments(case):
    """Segments longer than several tiles with ragged tails; a long prefix that forces the split-key
    query path with several chunks."""
    rng = random.Random(2000 + case)
    prompts = [(rng.randint(60, 200), [rng.randint(1, 300) for _ in range(rng.randint(3, 9))],
                rng.randint(30, 150)) for _ in range(rng.randint(1, 2))]
    hq, hkv, d = [(8, 2, 128), (4, 1, 64), (32, 8, 128), (2, 2, 128)][case]
    w = workloads.make_custom(prompts, hq, hkv, d, 4, 2000 + case)
    _full_check(w, f"ragged-tail case={case}")


def test_sharp_softmax_stress():
    rng = random.Random(77)
    prompts = random_prompts(rng, batch=2, p_max=40, n_max=6, l_max=90, q_max=40, p_min=1)
    prompts = [(p, l, max(q, 4)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, 8, 2, 128, 4, 77, q_scale=8.0)
    _full_check(w, "sharp softmax (Q x 8)")


def test_custom_scale():
    rng = random.Random(78)
    prompts = random_prompts(rng, batch=1, p_max=30, n_max=4, l_max=60, q_max=30, p_min=1)
    prompts = [(p, l, max(q, 2)) for (p, l, q) in prompts]
    w = workloads.make_custom(prompts, 4, 2, 64, 2, 78)
    _full_check(w, "custom scale 0.05", scale=0.05)


def test_document_isolation_bit_exact():
    """Document rows do not change, bit for bit, when other documents are permuted or altered."""
    lens = [37, 64, 129, 5, 90, 64]
    w = workloads.make_custom([(40, lens, 30)], 8, 2, 128, 2, 91)
    log("[gpu] isolation: base run")
    dev = upload(w)
    base = run_attn(w, dev).cpu()
    so = [int(x) for x in w.segment_offsets]
    spans = [(so[1 + k], so[2 + k]) for k in range(len(lens))]
    perm = [4, 2, 0, 5, 3, 1]
    idx = np.r_[0:so[1], np.concatenate([np.arange(*spans[k]) for k in perm]), so[-2]:so[-1]]
    seg_p, sp_p, _, _ = workloads.segment_tables([(40, [lens[k] for k in perm], 30)])
    wp = workloads.make_custom([(40, [lens[k] for k in perm], 30)], 8, 2, 128, 2, 91)
    wp.Q, wp.K, wp.V = w.Q[idx].copy(), w.K[idx].copy(), w.V[idx].copy()
    # alter document 3 (in the permuted prompt) completely
    a3, e3 = [int(x) for x in wp.segment_offsets[4:6]]
    noise = np.random.default_rng(3)
    wp.K[a3:e3] = noise.integers(0x3c00, 0x4000, size=wp.K[a3:e3].shape, dtype=np.uint16)
    wp.V[a3:e3] = noise.integers(0x3c00, 0x4000, size=wp.V[a3:e3].shape, dtype=np.uint16)
    log("[gpu] isolation: permuted + altered run")
    perm_out = run_attn(wp, upload(wp)).cpu()
    pos = so[1]
    b16 = lambda t: t.view(torch.int16).numpy()
    for slot, k in enumerate(perm):
        a, e = spans[k]
        if slot != 3:
            np.testing.assert_array_equal(b16(perm_out[pos:pos + (e - a)]), b16(base[a:e]), err_msg=f"doc {k}")
        pos += e - a
    np.testing.assert_array_equal(b16(perm_out[:so[1]]), b16(base[:so[1]]))


def test_sort_matches_oracle_rank_bit_exact():
    r = np.random.default_rng(11)
    n_list = [1, 7, 100, 500, 33, 8192, 10000, 16384]  # more than 8,192: several LDS chunks
    scores = np.concatenate([(np.round(r.random(n) * 64) / 64).astype(np.float32) for n in n_list])
    scores[5] = -0.0
    scores[6] = 0.0
    scores[20] = np.nan
    dp = np.cumsum([0] + [n + 1 for n in n_list]).astype(np.int32)
    log("[gpu] sort: ties, signed zeros, NaN, N up to 16,384")
    got = br.sort_docs(torch.from_numpy(scores).cuda(), dp).cpu().numpy()
    ref_in = np.where(np.isnan(scores), -np.inf, scores)
    np.testing.assert_array_equal(got, orc.rank(ref_in, dp))


def test_bitwise_determinism():
    w = workloads.make("worked", 1)
    dev = upload(w)
    log("[gpu] determinism: worked seed 1, two runs")
    r = []
    for _ in range(2):
        out, lse = run_attn(w, dev, lse=True)
        s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
        o = br.sort_docs(s, w.doc_ptr)
        torch.cuda.synchronize()
        r.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy(), s.cpu().numpy(), o.cpu().numpy()))
    for a, b in zip(r[0], r[1]):
        np.testing.assert_array_equal(a, b)


# Many short documents per prompt (two prompts of unequal size), many query heads per KV head, and
# a prompt of more than a thousand documents.
RANK_CUSTOM = {
    "many_docs": ([(16, [8] * 600, 16), (8, [3] * 40, 8)], dict(hq=8, hkv=2, d=64, n_signal=4)),
    "wide_heads": ([(8, [4] * 300, 8)], dict(hq=64, hkv=8, d=64, n_signal=2)),
    "over_1024_docs": ([(4, [2] * 1100, 4), (4, [5] * 7, 4)], dict(hq=4, hkv=2, d=64, n_signal=2)),
    "over_8192_docs": ([(4, [2] * 10000, 4)], dict(hq=4, hkv=2, d=64, n_signal=2)),
}


@pytest.mark.parametrize("config", ["worked", "batched", "ragged", "many_docs", "wide_heads", "over_1024_docs",
                                    "over_8192_docs"])
def test_rank_step_matches_separate_calls(config):
    """br_rank_prompts (one call, one plan upload) gives bit-identical attention output, lse, scores,
    head scores and order to br_attn_fwd + br_doc_scores + br_sort_docs, and the order is the
    oracle's rank of the scores, bit for bit (up to 10,000 documents in one prompt)."""
    if config in RANK_CUSTOM:
        prompts, kw = RANK_CUSTOM[config]
        w = workloads.make_custom(prompts, seed=3, **kw)
    else:
        w = workloads.make(config, 0)
    dev = upload(w)
    log(f"[gpu] fused rank step vs separate calls: {config}")
    a_out, a_lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True)
    a_s, a_hs = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, head_scores=True)
    a_o = br.sort_docs(a_s, w.doc_ptr)
    hs = torch.empty_like(a_hs)
    lse = torch.empty_like(a_lse)
    out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr, w.doc_offsets,
                             w.doc_ptr, lse=lse, head_scores=hs)
    torch.cuda.synchronize()
    assert torch.equal(out, a_out) and torch.equal(lse, a_lse)
    assert torch.equal(s, a_s) and torch.equal(hs, a_hs) and torch.equal(o, a_o)
    sc = s.cpu().numpy()
    np.testing.assert_array_equal(o.cpu().numpy(), orc.rank(np.where(np.isnan(sc), -np.inf, sc), w.doc_ptr))


def test_rank_step_side_stream_from_two_host_threads():
    """Batches of 24,576 tokens or more run the readout on the library's side stream.  Two host
    threads, each with its own stream, workspace and outputs, call the step at once, five times
    each: every result equals the separate calls' bit for bit (the side stream's fork and join
    events are shared, and a lock keeps the two threads' enqueues apart)."""
    import threading
    w = workloads.make_custom([(32, [150] * 110, 32), (32, [150] * 110, 32)], hq=8, hkv=2, d=64, n_signal=4,
                              seed=5)
    assert w.total_tokens >= 24576
    dev = upload(w)
    log(f"[gpu] side-stream rank step from two threads: T={w.total_tokens}")
    a_out = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
    a_s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    a_o = br.sort_docs(a_s, w.doc_ptr)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                got = []
                for _ in range(5):
                    out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets,
                                             w.seg_ptr, w.doc_offsets, w.doc_ptr, stream=stream)
                    got.append((out, s, o))
                stream.synchronize()
            results[tid] = got
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for tid in range(2):
        for out, s, o in results[tid]:
            assert torch.equal(out, a_out) and torch.equal(s, a_s) and torch.equal(o, a_o)


def test_calls_on_a_stream_that_is_not_current():
    """Calls given a stream that is not torch's current one, with outputs and workspace left to
    the binding, equal the calls on the current stream bit for bit, also when the default-stream
    memory they would otherwise reuse is being rewritten meanwhile."""
    w = workloads.make("worked", 0)
    dev = upload(w)
    log(f"[gpu] non-current stream: T={w.total_tokens}")
    a_out, a_lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True)
    a_s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    a_o = br.sort_docs(a_s, w.doc_ptr)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got = []
    for _ in range(3):
        out, lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True, stream=side)
        s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, stream=side)
        o = br.sort_docs(s, w.doc_ptr, stream=side)
        got.append((out, lse, s, o))
        # default-stream work that allocates and writes while the side stream may still run
        junk = torch.full((4 << 20,), 7.0, device="cuda")
        del junk
    side.synchronize()
    for out, lse, s, o in got:
        assert torch.equal(out, a_out) and torch.equal(lse, a_lse)
        assert torch.equal(s, a_s) and torch.equal(o, a_o)


def test_rank_step_plan_cache_tells_tables_apart():
    """The ranking step keeps its last few plans and reuses one when a call's dimensions and host
    tables are equal element by element.  Tables of the same size that differ only in document
    lengths, and the same tables with more signal rows, alternate: every call still equals the
    separate calls bit for bit."""
    kw = dict(hq=4, hkv=2, d=64, seed=9)
    variants = [workloads.make_custom([(16, [30, 50, 20], 16)], n_signal=4, **kw),
                workloads.make_custom([(16, [50, 30, 20], 16)], n_signal=4, **kw),
                workloads.make_custom([(16, [30, 50, 20], 16)], n_signal=8, **kw)]
    assert len({w.total_tokens for w in variants}) == 1
    refs = []
    for w in variants:
        dev = upload(w)
        out = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
        s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
        refs.append((dev, out, s, br.sort_docs(s, w.doc_ptr)))
    log("[gpu] rank step plan cache: three tables of one size, alternating")
    for rep in range(3):
        for w, (dev, a_out, a_s, a_o) in zip(variants, refs):
            out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr,
                                     w.doc_offsets, w.doc_ptr)
            torch.cuda.synchronize()
            assert torch.equal(out, a_out) and torch.equal(s, a_s) and torch.equal(o, a_o), (rep, w.prompts)


def test_rank_step_plan_device_copies_made_and_dropped():
    """From a plan's first reuse the step reads the plan from a device copy; six table sets used
    twice each in turn overflow the four kept plans, so copies are made and freed over and over
    (the first call of a set after its eviction uploads into the workspace again).  Every call
    equals the separate calls bit for bit."""
    kw = dict(hq=4, hkv=2, d=64, seed=11)
    lens = [[30, 50, 20], [50, 30, 20], [20, 30, 50], [40, 40, 20], [10, 60, 30], [25, 25, 50]]
    variants = [workloads.make_custom([(16, l, 16)], n_signal=4, **kw) for l in lens]
    refs = []
    for w in variants:
        dev = upload(w)
        out = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
        s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
        refs.append((dev, out, s, br.sort_docs(s, w.doc_ptr)))
    log("[gpu] rank step plan device copies: six table sets, two calls each, three rounds")
    for rep in range(3):
        for w, (dev, a_out, a_s, a_o) in zip(variants, refs):
            for call in range(2):
                out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr,
                                         w.doc_offsets, w.doc_ptr)
                torch.cuda.synchronize()
                assert torch.equal(out, a_out) and torch.equal(s, a_s) and torch.equal(o, a_o), (rep, call, w.prompts)


def test_rank_step_plan_device_copies_on_the_side_stream():
    """The same at 25,000+ tokens, where the readout and rank run on the library's side stream:
    five table sets of one size (document lengths permuted), two calls each, twice over, so
    plans are reused from their device copies, evicted and made again; every call equals the
    separate calls bit for bit."""
    kw = dict(hq=4, hkv=2, d=64, seed=13)
    base = [200 + 10 * i for i in range(60)]  # 60 documents, 29,700 document tokens
    variants = []
    for v in range(5):
        lens = base[v:] + base[:v]
        variants.append(workloads.make_custom([(64, lens, 32)], n_signal=4, **kw))
    assert all(w.total_tokens >= 24576 for w in variants)
    refs = []
    for w in variants:
        dev = upload(w)
        out = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr)
        s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
        refs.append((dev, out, s, br.sort_docs(s, w.doc_ptr)))
    log(f"[gpu] rank step plan device copies, side stream: five table sets of {variants[0].total_tokens} tokens")
    for rep in range(2):
        for w, (dev, a_out, a_s, a_o) in zip(variants, refs):
            for call in range(2):
                out, s, o = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr,
                                         w.doc_offsets, w.doc_ptr)
                torch.cuda.synchronize()
                assert torch.equal(out, a_out) and torch.equal(s, a_s) and torch.equal(o, a_o), (rep, call)


def test_many_prompts_rank_and_attention():
    """300 small prompts in one call (more than one sort launch's 256 prompts): attention against
    the dense oracle, scores and per-prompt order against the oracle's, and the one-call step equal
    to the separate calls."""
    r = np.random.default_rng(21)
    prompts = [(int(r.integers(0, 4)), [int(x) for x in r.integers(1, 6, size=int(r.integers(1, 4)))], 2)
               for _ in range(300)]
    w = workloads.make_custom(prompts, hq=2, hkv=1, d=64, n_signal=2, seed=21)
    dev = upload(w)
    log(f"[gpu] many prompts: B={w.num_prompts} T={w.total_tokens}")
    out = run_attn(w, dev)
    ref, _ = orc.attn_dense(w.Q, w.K, w.V, w.segment_offsets, w.seg_ptr)
    check_attn(out, ref, what="300 prompts")
    s = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    o = br.sort_docs(s, w.doc_ptr)
    torch.cuda.synchronize()
    ref_s, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    check_scores(s.cpu().numpy().astype(np.float64), ref_s, w.n_signal, "300 prompts")
    check_order(o.cpu().numpy(), ref_s, w.doc_ptr, "300 prompts")
    out2, s2, o2 = br.rank_step(dev["Q"], dev["K"], dev["V"], dev["Q_S"], w.segment_offsets, w.seg_ptr,
                                w.doc_offsets, w.doc_ptr)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(s2, s) and torch.equal(o2, o)
