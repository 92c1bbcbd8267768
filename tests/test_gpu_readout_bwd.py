"""GPU parity of the InfoNCE auxiliary loss (br_infonce) and the readout backward
(br_doc_scores_bwd) against the fp64 oracle, through the C ABI.

Tolerances: InfoNCE runs in fp32 on the same fp32 scores: loss and gradient within 1e-5 relative
(gradient: of 1/tau).  The readout backward rounds dz to bf16 for both MFMA products: relative
Frobenius error <= 1e-2 and max-abs <= 3e-2 of the largest reference magnitude, as for the
attention backward."""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import log, upload
from pins import random_prompts

pytestmark = pytest.mark.gpu

FRO_RTOL = 1e-2
MAX_RTOL = 3e-2


def check_grad(got: np.ndarray, ref: np.ndarray, what: str, fro_tol=FRO_RTOL, max_tol=MAX_RTOL):
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = got - ref
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(err).max() / max(np.abs(ref).max(), 1e-30)
    log(f"  {what}: rel Frobenius {fro:.2e}, max-abs / max|ref| {mx:.2e}")
    assert fro <= fro_tol and mx <= max_tol, f"{what}: rel Frobenius {fro:.2e}, rel max {mx:.2e}"


def test_infonce_parity():
    rng = np.random.default_rng(0)
    counts = [1, 5, 100, 500, 3000, 10000, 16384]
    dp = np.concatenate([[0], np.cumsum(np.array(counts) + 1)]).astype(np.int32)
    s = np.concatenate([rng.uniform(0, 2, n) for n in counts]).astype(np.float32)
    gold = np.array([0, 4, 17, 250, 2999, 9000, 16383], dtype=np.int32)
    log(f"[infonce] documents per prompt {counts}")
    loss, ds = br.infonce(torch.from_numpy(s).cuda(), dp, gold, tau=0.05)
    torch.cuda.synchronize()
    L_ref, g_ref = orc.infonce(s.astype(np.float64), dp, gold, tau=0.05)
    L = loss.cpu().numpy().astype(np.float64)
    g = ds.cpu().numpy().astype(np.float64)
    assert np.abs(L - L_ref).max() <= 1e-5 * max(1.0, np.abs(L_ref).max()), (L, L_ref)
    assert np.abs(g - g_ref).max() <= 1e-5 / 0.05, np.abs(g - g_ref).max()
    assert L[0] == 0.0 and g[0] == 0.0          # one document: the loss is zero


CASES = [  # seed, Hq, Hkv, d, n_signal  (signal rows per KV head = n_signal * G)
    (0, 32, 8, 128, 8),   # 32 rows
    (1, 16, 2, 64, 8),    # 64 rows: two row blocks
    (2, 8, 8, 128, 4),    # G = 1
    (3, 8, 1, 128, 3),    # 24 rows
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_S{c[4]}" for c in CASES])
def test_readout_bwd_parity(case):
    seed, hq, hkv, d, S = case
    rng = random.Random(800 + seed)
    prompts = [(p, l, max(q, S)) for (p, l, q) in random_prompts(rng, batch=3, p_max=40, n_max=30, l_max=120, q_max=40)]
    w = workloads.make_custom(prompts, hq, hkv, d, S, 3300 + seed)
    log(f"[readout bwd] seed={seed} Hq={hq} Hkv={hkv} d={d} S={S} T={w.total_tokens} docs={w.num_docs}")
    dev = upload(w)
    nrng = np.random.default_rng(seed)
    dscores = nrng.standard_normal(w.num_docs).astype(np.float32)
    ds_t = torch.from_numpy(dscores).cuda()
    sentinel = 7.0
    dK0 = torch.full((w.total_tokens, hkv, d), sentinel, dtype=torch.float32, device="cuda")
    dQs, dK = br.doc_scores_bwd(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, ds_t, dK=dK0.clone())
    dQs2, dKacc = br.doc_scores_bwd(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, ds_t, dK=dK0.clone(),
                                    accumulate=True)
    torch.cuda.synchronize()
    rQs, rK = orc.doc_scores_bwd(w.Q_S, w.K, w.doc_offsets, w.doc_ptr, dscores.astype(np.float64))
    kind = orc.token_tables(w.segment_offsets, w.seg_ptr)[2]
    docs = kind == orc.KIND_D
    gK = dK.cpu().numpy().astype(np.float64)
    check_grad(dQs.cpu().numpy().astype(np.float64), rQs, "dQ_S")
    check_grad(gK[docs], rK[docs], "dK (document rows)")
    assert (gK[~docs] == sentinel).all(), "rows outside documents were written"
    assert torch.equal(dQs, dQs2)
    acc = dKacc.cpu().numpy().astype(np.float64)
    assert np.array_equal(acc[docs], (torch.from_numpy(gK[docs]).float() + sentinel).double().numpy()), \
        "accumulate did not add onto the existing rows"
    assert (acc[~docs] == sentinel).all()


def test_rank_loss_gradient_chain():
    """Readout, InfoNCE and the readout backward on the GPU, each on the previous step's GPU output,
    against the oracle's chain.  The scores' fp32 rounding passes through the 1/tau = 20 logits, so
    the chain's bound is three times the single step's."""
    rng = random.Random(5)
    prompts = [(32, [rng.randint(20, 150) for _ in range(25)], 16), (10, [rng.randint(20, 150) for _ in range(12)], 12)]
    w = workloads.make_custom(prompts, 32, 8, 128, 8, 3400, plant_docs=[1, 2])
    log(f"[loss chain] T={w.total_tokens} docs={w.num_docs}")
    dev = upload(w)
    gold = np.array([1, 2], dtype=np.int32)
    scores = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    loss, ds = br.infonce(scores, w.doc_ptr, gold)
    dQs, dK = br.doc_scores_bwd(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, ds)
    torch.cuda.synchronize()
    s_ref, _ = orc.doc_scores(w.Q_S, w.K, w.doc_offsets, w.doc_ptr)
    L_ref, g_ref = orc.infonce(s_ref, w.doc_ptr, gold)
    rQs, rK = orc.doc_scores_bwd(w.Q_S, w.K, w.doc_offsets, w.doc_ptr, g_ref)
    L = loss.cpu().numpy().astype(np.float64)
    log(f"  loss {L} vs {L_ref}")
    assert np.abs(L - L_ref).max() <= 1e-2 * max(1.0, np.abs(L_ref).max())
    check_grad(dQs.cpu().numpy().astype(np.float64), rQs, "dQ_S", 3 * FRO_RTOL, 3 * MAX_RTOL)
    docs = orc.token_tables(w.segment_offsets, w.seg_ptr)[2] == orc.KIND_D
    check_grad(dK.cpu().numpy().astype(np.float64)[docs], rK[docs], "dK", 3 * FRO_RTOL, 3 * MAX_RTOL)


def test_readout_bwd_long_prompt_full():
    """The long ranking prompt (T = 100,096, 500 documents, |S| = 8) at full size, every output
    against the oracle."""
    w = workloads.make("long", 0)
    log(f"[readout bwd long] T={w.total_tokens}")
    dev = upload(w)
    dscores = np.random.default_rng(1).standard_normal(w.num_docs).astype(np.float32)
    dQs, dK = br.doc_scores_bwd(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, torch.from_numpy(dscores).cuda())
    torch.cuda.synchronize()
    rQs, rK = orc.doc_scores_bwd(w.Q_S, w.K, w.doc_offsets, w.doc_ptr, dscores.astype(np.float64))
    check_grad(dQs.cpu().numpy().astype(np.float64), rQs, "dQ_S")
    offs = np.asarray(w.segment_offsets)
    a, e = int(offs[1]), int(offs[-2])
    check_grad(dK[a:e].cpu().numpy().astype(np.float64), rK[a:e], "dK (document rows)")
