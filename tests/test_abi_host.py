"""The C-ABI library on the host (no GPU): it loads, exports every declared symbol, rejects bad
arguments before any HIP call, and its attention plan covers exactly the allowed pairs."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from pins import random_prompts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_header_symbol():
    lib = br.load_library()
    with open(os.path.join(ROOT, "include", "blockrank.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(br_[a-z_]+)\s*\(", header))
    assert declared == set(br.EXPORTED), declared ^ set(br.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert br.version().startswith("blockrank-gfx950")


def _covered_pairs(items, tm, T):
    """(row, key) pairs the plan visits after its own masking."""
    pairs = set()
    for (row0, lim, a0, a1, b0, b1, slot, nt) in items:
        rows = range(row0, min(row0 + tm, lim))
        for i in rows:
            for j in range(a0, a1):
                pairs.add((i, j))
            for j in range(b0, min(b1, i + 1)):
                pairs.add((i, j))
    return pairs


@pytest.mark.parametrize("seed", range(12))
def test_plan_covers_exactly_the_mask(seed):
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=rng.randint(1, 3), p_max=70, n_max=5, l_max=150, q_max=140)
    hq, hkv = rng.choice([(1, 1), (2, 1), (4, 1), (8, 1), (32, 8)])
    seg, sp, _, _ = workloads.segment_tables(prompts)
    T = int(seg[-1])
    dims = br.make_dims(len(prompts), hq, hkv, 64, T)
    items, tm = br.attn_plan_items(dims, seg, sp)
    assert tm == 128 // (hq // hkv)
    got = _covered_pairs(items, tm, T)
    tables = orc.token_tables(seg, sp)
    idx = np.arange(T)
    mask = orc.allowed(idx[:, None], idx[None, :], tables)
    want = set(zip(*np.nonzero(mask)))
    assert got == {(int(a), int(b)) for a, b in want}
    # every row is owned by exactly one direct item or one split query tile
    owners = np.zeros(T, dtype=np.int64)
    split_tiles = set()
    for (row0, lim, a0, a1, b0, b1, slot, nt) in items:
        assert 0 <= row0 < lim <= T and 0 <= a0 <= a1 <= T and 0 <= b0 <= b1 <= T
        if slot < 0:
            owners[row0:min(row0 + tm, lim)] += 1
        elif (row0, lim) not in split_tiles:
            split_tiles.add((row0, lim))
            owners[row0:min(row0 + tm, lim)] += 1
    assert (owners == 1).all()


def test_plan_visits_no_forbidden_tile_at_worked_shape():
    w_seg, w_sp, _, _ = workloads.segment_tables([(32, [128] * 100, 32)])
    dims = br.make_dims(1, 32, 8, 128, int(w_seg[-1]))
    items, tm = br.attn_plan_items(dims, w_seg, w_sp)
    assert tm == 32
    # documents read only [0, 32) and their own span; the query reads [0, L)
    offs = list(map(int, w_seg))
    for (row0, lim, a0, a1, b0, b1, slot, nt) in items:
        if row0 >= offs[-2]:
            continue
        k = np.searchsorted(offs, row0, side="right") - 1
        if k == 0:
            assert (a0, a1) == (0, 0) and (b0, b1) == (0, min(row0 + tm, 32))
        else:
            assert (a0, a1) == (0, 32) and b0 == offs[k] and b1 <= offs[k + 1]


def _sched_cost(item):
    """Schedule cost of one item in quarter key tiles (direct row tile / split query chunk)."""
    row0, lim, a0, a1, b0, b1, slot, nt = map(int, item)
    return 4 * nt + 16 if slot < 0 else 5 * nt + 24


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("workgroups", [1, 7, 64, 512])
def test_schedule_is_a_balanced_permutation(seed, workgroups):
    rng = random.Random(100 + seed)
    prompts = random_prompts(rng, batch=rng.randint(1, 3), p_max=70, n_max=12, l_max=300, q_max=140)
    hq, hkv = rng.choice([(4, 1), (8, 2), (32, 8)])
    seg, sp, _, _ = workloads.segment_tables(prompts)
    dims = br.make_dims(len(prompts), hq, hkv, 128, int(seg[-1]))
    items, _ = br.attn_plan_items(dims, seg, sp)
    sched, ranges = br.attn_plan_schedule(dims, seg, sp, workgroups)
    W = len(ranges) - 1
    assert W == max(1, min(len(items), workgroups // hkv))
    assert ranges[0] == 0 and ranges[-1] == len(items) and (np.diff(ranges) >= 0).all()
    # a permutation of the plan's items
    assert sorted(map(tuple, sched.tolist())) == sorted(map(tuple, items.tolist()))
    # greedy list schedule: two workgroups' loads differ by at most one item's cost
    loads = [sum(_sched_cost(x) for x in sched[ranges[w]:ranges[w + 1]]) for w in range(W)]
    assert max(loads) - min(loads) <= max(_sched_cost(x) for x in items)


def test_schedule_rejects_bad_workgroups():
    seg, sp, _, _ = workloads.segment_tables([(8, [16, 16], 8)])
    dims = br.make_dims(1, 4, 1, 64, int(seg[-1]))
    with pytest.raises(br.BlockRankError) as ei:
        br.attn_plan_schedule(dims, seg, sp, 0)
    assert ei.value.status == br._lib.BR_ERR_INVALID_ARG


def test_schedule_spreads_a_document_over_workgroups():
    # the row tiles of one document are adjacent in time order, so they start on different
    # workgroups at about the same time (their keys are then shared in L2)
    seg, sp, _, _ = workloads.segment_tables([(64, [200] * 500, 32)])
    dims = br.make_dims(1, 32, 8, 128, int(seg[-1]))
    sched, ranges = br.attn_plan_schedule(dims, seg, sp, 512)
    owner = np.repeat(np.arange(len(ranges) - 1), np.diff(ranges))
    doc = 250
    lo, hi = int(seg[1 + doc]), int(seg[2 + doc])
    mine = np.nonzero((sched[:, 0] >= lo) & (sched[:, 0] < hi))[0]
    assert len(mine) == 7 and len(set(owner[mine].tolist())) == 7


def _fake(n=1):
    return ctypes.c_void_p(0x10000)  # non-NULL, 16-byte aligned; never dereferenced on error paths


BAD_TABLES = [
    ("seg_ptr0", [0, 4, 6, 8, 10], [1, 5], br._lib.BR_ERR_INVALID_ARG),
    ("too_few_offsets", [0, 4, 8], [0, 3], br._lib.BR_ERR_INVALID_ARG),
    ("empty_doc", [0, 4, 4, 8, 10], [0, 5], br._lib.BR_ERR_INVALID_ARG),
    ("empty_query", [0, 4, 6, 10, 10], [0, 5], br._lib.BR_ERR_INVALID_ARG),
    ("reversed", [0, 4, 3, 8, 10], [0, 5], br._lib.BR_ERR_INVALID_ARG),
    ("not_starting_at_0", [2, 4, 6, 8, 10], [0, 5], br._lib.BR_ERR_INVALID_ARG),
    ("total_mismatch", [0, 4, 6, 8, 9], [0, 5], br._lib.BR_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,seg,sp,status", BAD_TABLES, ids=[t[0] for t in BAD_TABLES])
def test_bad_segment_tables_rejected(name, seg, sp, status):
    dims = br.make_dims(1, 4, 2, 64, 10)
    with pytest.raises(br.BlockRankError) as ei:
        br.attn_workspace_bytes(dims, seg, sp)
    assert ei.value.status == status


def test_noncontiguous_prompts_rejected():
    dims = br.make_dims(2, 4, 2, 64, 20)
    with pytest.raises(br.BlockRankError) as ei:
        br.attn_workspace_bytes(dims, [0, 2, 5, 10, 11, 13, 16, 20], [0, 4, 8])
    assert "previous prompt" in ei.value.message


@pytest.mark.parametrize("hq,hkv,d,status", [(4, 3, 64, 1), (16, 1, 64, 2), (4, 2, 96, 2), (4, 2, 0, 1),
                                             (0, 1, 64, 1), (1024, 128, 128, 2), (2048, 256, 64, 2)])
def test_bad_dims_rejected(hq, hkv, d, status):
    dims = br.make_dims(1, hq, hkv, d, 10)
    with pytest.raises(br.BlockRankError) as ei:
        br.attn_workspace_bytes(dims, [0, 4, 6, 8, 10], [0, 5])
    assert ei.value.status == status


def test_attn_fwd_rejects_before_any_hip_call():
    lib = br.load_library()
    seg = np.array([0, 4, 6, 8, 10], dtype=np.int32)
    sp = np.array([0, 5], dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    dims = br.make_dims(1, 4, 2, 64, 10)
    need = br.attn_workspace_bytes(dims, seg, sp)
    f = _fake()
    # workspace too small
    st = lib.br_attn_fwd(ctypes.byref(dims), f, f, f, p(seg), p(sp), f, None, 0.0, f, need - 1, None)
    assert st == br._lib.BR_ERR_WORKSPACE
    # NULL input
    st = lib.br_attn_fwd(ctypes.byref(dims), None, f, f, p(seg), p(sp), f, None, 0.0, f, need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG
    # misaligned output
    st = lib.br_attn_fwd(ctypes.byref(dims), f, f, f, p(seg), p(sp), ctypes.c_void_p(0x10002), None, 0.0, f,
                         need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG
    # non-finite scale
    st = lib.br_attn_fwd(ctypes.byref(dims), f, f, f, p(seg), p(sp), f, None, float("nan"), f, need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG
    assert b"finite" in lib.br_last_error()


def test_doc_scores_and_sort_reject_bad_arguments():
    lib = br.load_library()
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    dims = br.make_dims(1, 4, 2, 64, 10)
    f = _fake()
    do = np.array([4, 6, 8], dtype=np.int32)
    dp = np.array([0, 3], dtype=np.int32)
    need = br.doc_scores_workspace_bytes(dims, 2, do, dp)
    assert lib.br_doc_scores(ctypes.byref(dims), f, 2, f, p(do), p(dp), f, None, 0.0, f, need - 1,
                             None) == br._lib.BR_ERR_WORKSPACE
    assert lib.br_doc_scores(ctypes.byref(dims), f, 0, f, p(do), p(dp), f, None, 0.0, f, need,
                             None) == br._lib.BR_ERR_INVALID_ARG
    assert lib.br_doc_scores(ctypes.byref(dims), f, 65, f, p(do), p(dp), f, None, 0.0, f, need,
                             None) == br._lib.BR_ERR_UNSUPPORTED
    bad = np.array([4, 4, 8], dtype=np.int32)
    assert lib.br_doc_scores(ctypes.byref(dims), f, 2, f, p(bad), p(dp), f, None, 0.0, f, need,
                             None) == br._lib.BR_ERR_INVALID_ARG
    beyond = np.array([4, 6, 11], dtype=np.int32)
    assert lib.br_doc_scores(ctypes.byref(dims), f, 2, f, p(beyond), p(dp), f, None, 0.0, f, need,
                             None) == br._lib.BR_ERR_INVALID_ARG
    big = np.array([0, 65538], dtype=np.int32)  # 65,537 documents: one more than the sort takes
    assert lib.br_sort_docs(f, p(big), 1, f, None) == br._lib.BR_ERR_UNSUPPORTED
    assert lib.br_sort_docs(f, p(np.array([0, 1], dtype=np.int32)), 1, f, None) == br._lib.BR_ERR_INVALID_ARG
    assert lib.br_sort_docs(None, p(dp), 1, f, None) == br._lib.BR_ERR_INVALID_ARG


# ---- query-only attention over a cached corpus (host side only) ----
def test_query_attn_workspace_and_bad_offsets():
    dims = br.make_dims(3, 8, 2, 128, 100 + 7 + 1 + 40)
    qo = np.array([100, 107, 108, 148], dtype=np.int32)
    assert br.query_attn_workspace_bytes(dims, 100, qo) > 0
    # corpus of 0 tokens: plain causal attention per query
    dims0 = br.make_dims(2, 8, 2, 128, 10)
    assert br.query_attn_workspace_bytes(dims0, 0, np.array([0, 3, 10], dtype=np.int32)) > 0
    bad = [
        (100, [99, 107, 108, 148]),   # first offset != corpus_len
        (100, [100, 107, 107, 148]),  # empty query
        (100, [100, 107, 108, 147]),  # last != total_tokens
        (-1, [-1, 107, 108, 148]),    # negative corpus
    ]
    for corpus, offs in bad:
        with pytest.raises(br.BlockRankError) as ei:
            br.query_attn_workspace_bytes(dims, corpus, np.array(offs, dtype=np.int32))
        assert ei.value.status == br._lib.BR_ERR_INVALID_ARG, (corpus, offs)


def test_query_attn_rejects_before_any_hip_call():
    lib = br.load_library()
    qo = np.array([64, 96], dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    dims = br.make_dims(1, 8, 2, 128, 96)
    need = br.query_attn_workspace_bytes(dims, 64, qo)
    f = _fake()
    st = lib.br_query_attn_fwd(ctypes.byref(dims), f, f, f, 64, p(qo), f, None, 0.0, f, need - 1, None)
    assert st == br._lib.BR_ERR_WORKSPACE
    st = lib.br_query_attn_fwd(ctypes.byref(dims), f, None, f, 64, p(qo), f, None, 0.0, f, need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG
    st = lib.br_query_attn_fwd(ctypes.byref(dims), f, f, f, 64, None, f, None, 0.0, f, need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG
    st = lib.br_query_attn_fwd(ctypes.byref(dims), f, f, f, 64, p(qo), f, None, float("inf"), f, need, None)
    assert st == br._lib.BR_ERR_INVALID_ARG


# ---- top-B routed attention (host side only) ----
def test_routed_workspace_and_bad_keep():
    seg, sp, _, _ = workloads.segment_tables([(8, [16, 12, 20], 8), (4, [10, 10], 6)])
    dims = br.make_dims(2, 8, 2, 64, int(seg[-1]))
    ok = br.attn_routed_workspace_bytes(dims, seg, sp, [0, 2, 3], [2, 0, 1])
    assert ok > 0
    # keeping every document sizes like the unrouted plan
    assert br.attn_routed_workspace_bytes(dims, seg, sp, [0, 3, 5], [0, 1, 2, 0, 1]) == \
        br.attn_workspace_bytes(dims, seg, sp)
    # no document kept anywhere is valid
    assert br.attn_routed_workspace_bytes(dims, seg, sp, [0, 0, 0], [0]) > 0
    bad = [
        ([0, 2, 3], [2, 3, 1]),   # document index out of range
        ([0, 2, 3], [1, 1, 0]),   # kept twice
        ([1, 2, 3], [0, 1, 0]),   # keep_ptr[0] != 0
        ([0, 2, 1], [0, 1, 0]),   # keep_ptr decreases
    ]
    for kp, kk in bad:
        with pytest.raises(br.BlockRankError) as ei:
            br.attn_routed_workspace_bytes(dims, seg, sp, kp, kk)
        assert ei.value.status == br._lib.BR_ERR_INVALID_ARG, (kp, kk)


# ---- SSMax factor and rotary embedding (host side only) ----
def test_ssmax_factor_and_bad_arguments():
    for s, n, d in [(0.43, 2, 64), (0.43, 500, 128), (0.2, 10000, 128)]:
        assert abs(br.ssmax_scale(s, n, d) - orc.ssmax_scale(s, n, d)) <= 1e-6 * orc.ssmax_scale(s, n, d)
    for s, n, d in [(0.43, 1, 64), (0.43, 0, 64), (0.0, 10, 64), (-1.0, 10, 64), (float("inf"), 10, 64),
                    (0.43, 10, 0)]:
        with pytest.raises(br.BlockRankError) as ei:
            br.ssmax_scale(s, n, d)
        assert ei.value.status == br._lib.BR_ERR_INVALID_ARG, (s, n, d)


@pytest.mark.parametrize("seed", range(6))
def test_rope_positions_match_oracle(seed):
    rng = random.Random(seed)
    prompts = random_prompts(rng, batch=rng.randint(1, 4), p_max=50, n_max=8, l_max=60, q_max=30)
    seg, sp, _, _ = workloads.segment_tables(prompts)
    dims = br.make_dims(len(prompts), 8, 2, 64, int(seg[-1]))
    for q0, after in [(8192, True), (300, False), (0, True), (123456, False)]:
        got = br.rope_positions(dims, seg, sp, q0, after)
        want = orc.rope_positions(seg, sp, q0, after)
        assert np.array_equal(got, want), (seed, q0, after)


def test_rope_rejects_before_any_hip_call():
    lib = br.load_library()
    seg, sp, _, _ = workloads.segment_tables([(8, [16, 12, 20], 8), (0, [10, 10], 6)])
    dims = br.make_dims(2, 8, 2, 64, int(seg[-1]))
    need = br.rope_workspace_bytes(dims, sp)
    assert need > 0
    p = lambda a: np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    segp, spp = p(seg), p(sp)
    f = _fake()
    INV, WS = br._lib.BR_ERR_INVALID_ARG, br._lib.BR_ERR_WORKSPACE
    call = lambda *a: lib.br_rope_fwd(ctypes.byref(dims), *a)
    assert call(f, f, f, f, segp, spp, 10000.0, 8192, 1, 0, f, need - 1, None) == WS
    assert call(f, f, f, f, segp, spp, 10000.0, 8192, 1, 0, None, need, None) == WS
    assert call(f, f, f, f, segp, spp, 0.0, 8192, 1, 0, f, need, None) == INV            # theta
    assert call(f, f, f, f, segp, spp, float("nan"), 8192, 1, 0, f, need, None) == INV
    assert call(f, f, f, f, segp, spp, 10000.0, -1, 1, 0, f, need, None) == INV          # query_pos0
    assert call(f, f, f, f, segp, spp, 10000.0, 2**31 - 3, 1, 0, f, need, None) == INV  # int32 overflow
    assert call(f, f, f, f, segp, spp, 10000.0, 8192, 2, 0, f, need, None) == INV        # rule flag
    assert call(f, f, f, f, segp, spp, 10000.0, 8192, 1, 2, f, need, None) == INV        # layout flag
    assert call(None, None, None, None, segp, spp, 10000.0, 8192, 1, 0, f, need, None) == INV
    assert call(f, f, None, f, segp, spp, 10000.0, 8192, 1, 0, f, need, None) == INV    # Q without Q_out
    assert call(f, f, f, f, None, spp, 10000.0, 8192, 1, 0, f, need, None) == INV
    sig = lambda *a: lib.br_rope_signal_fwd(ctypes.byref(dims), *a)
    assert sig(f, f, 7, segp, spp, 10000.0, 8192, 0, f, need, None) == INV   # second query has 6 tokens
    assert sig(f, f, 0, segp, spp, 10000.0, 8192, 0, f, need, None) == INV
    assert sig(f, f, 4, segp, spp, 10000.0, 8192, 0, f, 0, None) == WS
    pos = np.zeros(int(seg[-1]) - 1, dtype=np.int32)
    assert lib.br_rope_positions(ctypes.byref(dims), segp, spp, 8192, 1, p(pos), pos.size) == INV  # too small


# ---- attention backward plan (host side only) ----
@pytest.mark.parametrize("seed", range(6))
def test_bwd_plan_covers_exactly_the_mask(seed):
    """Every allowed (row, key) pair is visited by exactly one key-major item, no forbidden pair is,
    and every key lies in exactly one key tile (split tiles: the same keys in every chunk).  The
    last case has more than 4096 rows after the instruction, so its instruction keys are split."""
    rng = random.Random(100 + seed)
    if seed == 5:
        prompts = [(70, [180] * 25, 20)]
    else:
        prompts = random_prompts(rng, batch=rng.randint(1, 3), p_max=40, n_max=6, l_max=90, q_max=40)
    seg, sp, _, _ = workloads.segment_tables(prompts)
    T = int(seg[-1])
    dims = br.make_dims(len(prompts), 8, 2, 64, T)
    items, slots = br._lib.attn_bwd_plan_items(dims, seg, sp)
    cover = np.zeros((T, T), dtype=np.int32)
    key_owner = {}
    for k0, kl, c0, c1, u0, u1, slot, _ in items:
        assert 0 <= k0 < kl <= T and kl - k0 <= 64
        key_owner.setdefault((k0, kl), set()).add(slot)
        for r in range(c0, c1):
            cover[r, k0:min(kl, r + 1)] += 1
        if u1 > u0:
            cover[u0:u1, k0:kl] += 1
    tables = orc.token_tables(seg, sp)
    idx = np.arange(T)
    allowed = orc.allowed(idx[:, None], idx[None, :], tables)
    assert (cover[allowed] == 1).all(), "an allowed pair is missed or visited twice"
    assert (cover[~allowed] == 0).all(), "a forbidden pair is visited"
    keys = sorted(key_owner)
    assert keys[0][0] == 0 and keys[-1][1] == T
    assert all(a[1] == b[0] for a, b in zip(keys[:-1], keys[1:])), "key tiles do not tile the keys"
    used = sorted(s_ for v in key_owner.values() for s_ in v if s_ >= 0)
    assert used == list(range(slots))
    assert seed != 5 or slots > 0


# ---- InfoNCE and readout backward (host side only) ----
def test_infonce_and_readout_bwd_reject_before_any_hip_call():
    lib = br.load_library()
    p = lambda a: np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = _fake()
    dp = np.array([0, 4, 7], dtype=np.int32)   # 3 and 2 documents
    need = ctypes.c_size_t(0)
    assert lib.br_infonce_workspace_bytes(2, ctypes.byref(need)) == 0 and need.value > 0
    INV, WS, UNS = br._lib.BR_ERR_INVALID_ARG, br._lib.BR_ERR_WORKSPACE, br._lib.BR_ERR_UNSUPPORTED
    call = lambda gold, tau, ws=f, nb=need.value: lib.br_infonce(f, p(dp), 2, p(gold), tau, f, f, ws, nb, None)
    assert call([0, 2], 0.05) == INV            # gold 2 outside the second prompt's 2 documents
    assert call([-1, 0], 0.05) == INV
    assert call([0, 1], 0.0) == INV
    assert call([0, 1], float("inf")) == INV
    assert call([0, 1], 0.05, nb=need.value - 1) == WS
    assert lib.br_infonce(f, p([0, 1, 2]), 2, p([0, 0]), 0.05, f, f, f, need.value, None) == INV  # empty prompt
    n1 = ctypes.c_size_t(0)
    assert lib.br_infonce_workspace_bytes(1, ctypes.byref(n1)) == 0
    assert lib.br_infonce(f, p([0, 65538]), 1, p([0]), 0.05, f, f, f, n1.value, None) == UNS  # 65,537 documents
    # readout backward: too many signal rows per KV head, bad flags, workspace
    seg, sp, dof, dptr = workloads.segment_tables([(8, [16, 12, 20], 8), (4, [10, 10], 9)])
    dims = br.make_dims(2, 8, 1, 64, int(seg[-1]))   # G = 8
    with pytest.raises(br.BlockRankError) as ei:
        br.doc_scores_bwd_workspace_bytes(dims, 9, dof, dptr)     # 9 * 8 = 72 rows > 64
    assert ei.value.status == UNS
    nb = br.doc_scores_bwd_workspace_bytes(dims, 8, dof, dptr)
    bwd = lambda acc, scale, ws, n: lib.br_doc_scores_bwd(ctypes.byref(dims), f, 8, f, p(dof), p(dptr), f, f, f, acc,
                                                          scale, ws, n, None)
    assert bwd(2, 0.0, f, nb) == INV
    assert bwd(0, float("nan"), f, nb) == INV
    assert bwd(0, 0.0, f, nb - 1) == WS
    assert bwd(0, 0.0, None, nb) == WS


def test_attn_bwd_rejects_before_any_hip_call():
    lib = br.load_library()
    seg, sp, _, _ = workloads.segment_tables([(8, [16, 12, 20], 8), (4, [10, 10], 6)])
    dims = br.make_dims(2, 8, 2, 64, int(seg[-1]))
    need = br._lib.attn_bwd_workspace_bytes(dims, seg, sp)
    assert need > 0
    p = lambda a: np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = _fake()
    INV, WS = br._lib.BR_ERR_INVALID_ARG, br._lib.BR_ERR_WORKSPACE
    call = lambda *a: lib.br_attn_bwd(ctypes.byref(dims), *a)
    args = lambda **kw: [kw.get(k, v) for k, v in (("Q", f), ("K", f), ("V", f), ("O", f), ("dO", f), ("lse", f),
                                                 ("so", p(seg)), ("sp", p(sp)), ("dQ", f), ("dK", f), ("dV", f),
                                                 ("scale", 0.0), ("ws", f), ("n", need), ("st", None))]
    assert call(*args(n=need - 1)) == WS
    assert call(*args(ws=None)) == WS
    assert call(*args(dO=None)) == INV
    assert call(*args(lse=None)) == INV
    assert call(*args(dK=ctypes.c_void_p(0x10004))) == INV          # misaligned
    assert call(*args(scale=float("inf"))) == INV
    assert call(*args(sp=p([0, 5, 3]))) == INV                        # bad segment table
    bad = br.make_dims(2, 8, 3, 64, int(seg[-1]))                     # Hq not a multiple of Hkv
    assert lib.br_attn_bwd(ctypes.byref(bad), *args()) == INV


def test_rank_workspace_and_rejects_before_any_hip_call():
    lib = br.load_library()
    seg, sp, dof, dptr = workloads.segment_tables([(8, [16, 12, 20], 8), (4, [10, 10], 6)])
    dims = br.make_dims(2, 8, 2, 64, int(seg[-1]))
    need = br.rank_workspace_bytes(dims, seg, sp, 4, dof, dptr)
    assert need >= br.attn_workspace_bytes(dims, seg, sp) + br.doc_scores_workspace_bytes(dims, 4, dof, dptr) - 4096
    p = lambda a: np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = _fake()
    INV, WS, UNS = br._lib.BR_ERR_INVALID_ARG, br._lib.BR_ERR_WORKSPACE, br._lib.BR_ERR_UNSUPPORTED
    def call(**kw):
        a = dict(Q=f, K=f, V=f, QS=f, S=4, so=p(seg), sp=p(sp), do=p(dof), dp=p(dptr), out=f, lse=None, sc=f, hs=None,
                 order=f, scale=0.0, ws=f, n=need)
        a.update(kw)
        return lib.br_rank_prompts(ctypes.byref(dims), a["Q"], a["K"], a["V"], a["QS"], a["S"], a["so"], a["sp"],
                                   a["do"], a["dp"], a["out"], a["lse"], a["sc"], a["hs"], a["order"], a["scale"],
                                   a["ws"], a["n"], None)
    assert call(n=need - 1) == WS
    assert call(QS=None) == INV
    assert call(order=None) == INV
    assert call(S=0) == INV                    # no signal rows
    assert call(scale=float("nan")) == INV
    big = workloads.segment_tables([(2, [1] * 65537, 2)])
    dims2 = br.make_dims(1, 8, 2, 64, int(big[0][-1]))
    nb = ctypes.c_size_t(0)
    assert lib.br_rank_workspace_bytes(ctypes.byref(dims2), p(big[0]), p(big[1]), 1, p(big[2]), p(big[3]),
                                       ctypes.byref(nb)) == 0
    rc = lib.br_rank_prompts(ctypes.byref(dims2), f, f, f, f, 1, p(big[0]), p(big[1]), p(big[2]), p(big[3]), f, None,
                             f, None, f, 0.0, f, nb.value, None)
    assert rc == UNS                           # more documents than the sort takes


def test_noalloc_scratch_size_matches_header():
    """The binding's BR_NOALLOC_SCRATCH_BYTES copy equals the header's definition."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "blockrank.h")).read()
    m = re.search(r"#define BR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m, "BR_NOALLOC_SCRATCH_BYTES not found"
    assert br.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_binding_functions_run_on_their_stream(monkeypatch):
    """Every binding call that takes a ``stream`` makes it torch's current stream before it
    allocates outputs or workspace, so the caching allocator orders them on the kernels' stream."""
    import contextlib
    import inspect
    import torch
    from block_sparse_attention_segment_amd import _lib
    takes_stream = [n for n, f in inspect.getmembers(_lib, inspect.isfunction)
                    if not n.startswith("_") and "stream" in inspect.signature(f).parameters]
    assert len(takes_stream) >= 10, takes_stream
    for n in takes_stream:
        assert getattr(getattr(_lib, n), "runs_on_its_stream", False), n
    entered = []

    @contextlib.contextmanager
    def fake_stream(s):
        entered.append(s)
        yield

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)
    marker = object()
    x = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host tensors are refused inside, with the stream current
        br.attn_fwd(x, x, x, [0, 4], [0, 1], stream=marker)
    assert entered == [marker]
    with pytest.raises(ValueError):
        br.attn_fwd(x, x, x, [0, 4], [0, 1])
    assert entered == [marker]


def test_sink_rejects_nan_before_any_hip_call():
    lib = br.load_library()
    p = lambda a: np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = _fake()
    seg, sp, _, _ = workloads.segment_tables([(4, [5, 6], 3)])
    dims = br.make_dims(1, 4, 2, 64, int(seg[-1]))
    need = br.attn_workspace_bytes(dims, seg, sp)
    rc = lib.br_attn_fwd_sink(ctypes.byref(dims), f, f, f, p(seg), p(sp), f, None, 0.0, float("nan"), f, need, None)
    assert rc == br._lib.BR_ERR_INVALID_ARG
    rc = lib.br_attn_fwd_sink(ctypes.byref(dims), f, f, f, p(seg), p(sp), f, None, 0.0, 1.0, f, need - 1, None)
    assert rc == br._lib.BR_ERR_WORKSPACE


def test_attention_plan_item_limit():
    """A plan of 2^21 or more work items is refused as unsupported (the kernel packs an item index
    into 21 bits of a tile code); one just below the limit is accepted.  One-token documents take
    one item each; the query adds one item per 4,096-key chunk of the prefix."""
    n_ok = (1 << 21) - 600
    seg, sp, _, _ = workloads.segment_tables([(1, [1] * n_ok, 1)])
    dims = br.make_dims(1, 8, 1, 64, int(seg[-1]))
    items, _ = br.attn_plan_items(dims, seg, sp)
    assert (1 << 21) - 600 < len(items) < (1 << 21)
    seg, sp, _, _ = workloads.segment_tables([(1, [1] * (1 << 21), 1)])
    dims = br.make_dims(1, 8, 1, 64, int(seg[-1]))
    with pytest.raises(br.BlockRankError) as e:
        br.attn_plan_items(dims, seg, sp)
    assert e.value.status == br._lib.BR_ERR_UNSUPPORTED
