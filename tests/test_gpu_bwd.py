"""GPU parity of the attention backward (br_attn_bwd) against the fp64 oracle, through the C ABI.

Tolerance (from the arithmetic): P and dS are formed in fp32 and rounded to bf16 before the
P^T dO, dS K and dS^T Q products, and O (an input, from the forward) is bf16, so each term
carries relative errors of a few 2^-9; summed over many keys with mixed signs the gradient's
error stays near 2^-9 of its norm.  Bound: relative Frobenius error <= 1e-2 and max-abs error
<= 3e-2 of the largest reference magnitude, per tensor."""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_segment_amd as br
import oracle.oracle as orc
import workloads
from gpu_util import dev_bf16, log, upload
from pins import random_prompts

pytestmark = pytest.mark.gpu

FRO_RTOL = 1e-2
MAX_RTOL = 3e-2


def check_grad(got: torch.Tensor, ref: np.ndarray, what: str):
    g = got.cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    err = g - ref
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(err).max() / max(np.abs(ref).max(), 1e-30)
    log(f"  {what}: rel Frobenius {fro:.2e}, max-abs / max|ref| {mx:.2e}")
    assert fro <= FRO_RTOL and mx <= MAX_RTOL, f"{what}: rel Frobenius {fro:.2e}, rel max {mx:.2e}"


def run_case(w, seed, scale=0.0):
    dev = upload(w)
    rng = np.random.default_rng(seed)
    dO_bits = workloads.f32_to_bf16_bits(rng.standard_normal(w.Q.shape).astype(np.float32))
    dO = dev_bf16(dO_bits)
    O, lse = br.attn_fwd(dev["Q"], dev["K"], dev["V"], w.segment_offsets, w.seg_ptr, lse=True, softmax_scale=scale)
    dQ, dK, dV = br.attn_bwd(dev["Q"], dev["K"], dev["V"], O, dO, lse, w.segment_offsets, w.seg_ptr,
                             softmax_scale=scale)
    torch.cuda.synchronize()
    return dQ, dK, dV, dO_bits


CASES = [(0, 4, 1, 64), (1, 32, 8, 128), (2, 8, 8, 128), (3, 16, 2, 64), (4, 8, 1, 128), (5, 16, 8, 64),
         (6, 8, 4, 128)]  # query heads per KV head 4, 4, 1, 8, 8, 2, 2


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}" for c in CASES])
def test_attn_bwd_parity(case):
    seed, hq, hkv, d = case
    rng = random.Random(500 + seed)
    prompts = random_prompts(rng, batch=2, p_max=70, n_max=8, l_max=150, q_max=100, p_min=0 if seed % 2 else 1)
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 2500 + seed)
    log(f"[attn bwd] seed={seed} Hq={hq} Hkv={hkv} d={d} T={w.total_tokens} prompts={[(p, len(l), q) for p, l, q in prompts]}")
    dQ, dK, dV, dO_bits = run_case(w, seed)
    rQ, rK, rV = orc.attn_bwd(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr)
    check_grad(dQ, rQ, "dQ")
    check_grad(dK, rK, "dK")
    check_grad(dV, rV, "dV")


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (8, 2, 128)])
def test_attn_bwd_degenerate_segments(hq, hkv, d):
    """The smallest segments: one-token queries and documents, empty and one-token instructions,
    rows that see a single key (their P is 1, so their dQ and the dK they send are zero)."""
    prompts = [(0, [1, 2, 1], 1), (1, [1], 1), (0, [2], 1), (1, [1, 1, 2, 1], 1), (3, [5, 1], 2)]
    w = workloads.make_custom(prompts, hq, hkv, d, 1, 2700)
    log(f"[attn bwd degenerate] Hq={hq} Hkv={hkv} d={d} T={w.total_tokens}")
    dQ, dK, dV, dO_bits = run_case(w, 11)
    rQ, rK, rV = orc.attn_bwd(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr)
    check_grad(dQ, rQ, "dQ")
    check_grad(dK, rK, "dK")
    check_grad(dV, rV, "dV")


def test_attn_bwd_split_rows_and_scale():
    """A prompt with more than 4096 rows after its instruction (the instruction keys' row range is
    split and summed) and a non-default softmax scale."""
    prompts = [(70, [180] * 25, 40)]
    w = workloads.make_custom(prompts, 4, 1, 64, 1, 2600)
    log(f"[attn bwd split] T={w.total_tokens}")
    dQ, dK, dV, dO_bits = run_case(w, 7, scale=0.2)
    rQ, rK, rV = orc.attn_bwd(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr, scale=0.2)
    check_grad(dQ, rQ, "dQ")
    check_grad(dK, rK, "dK")
    check_grad(dV, rV, "dV")


def test_attn_bwd_deterministic():
    rng = random.Random(9)
    prompts = random_prompts(rng, batch=2, p_max=60, n_max=6, l_max=120, q_max=60)
    w = workloads.make_custom(prompts, 8, 2, 128, 1, 2700)
    log(f"[attn bwd determinism] T={w.total_tokens}")
    a = run_case(w, 3)
    b = run_case(w, 3)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_attn_bwd_long_prompt_identities():
    """The long ranking prompt (T = 100,096) at full size, checked through identities that hold at
    any size: per KV head, the keys' dV sum to the group's dO summed over rows (every P row sums to
    one), and the keys' dK sum to zero (every dS row sums to zero)."""
    w = workloads.make("long", 0)
    log(f"[attn bwd long] T={w.total_tokens}")
    dQ, dK, dV, dO_bits = run_case(w, 11)
    G = w.Q.shape[1] // w.K.shape[1]
    dO = workloads.bf16_bits_to_f32(dO_bits).astype(np.float64)
    want_v = dO.reshape(dO.shape[0], -1, G, dO.shape[2]).sum(axis=(0, 2))       # [Hkv, d]
    got_v = dV.double().sum(dim=0).cpu().numpy()
    err_v = np.abs(got_v - want_v).max() / np.abs(want_v).max()
    # the dK sum is a cancellation: compare with the sum of magnitudes
    got_k = dK.double().sum(dim=0).cpu().numpy()
    mag_k = dK.double().abs().sum(dim=0).cpu().numpy()
    err_k = (np.abs(got_k) / mag_k).max()
    log(f"  sum dV vs sum dO: {err_v:.2e};  |sum dK| / sum |dK|: {err_k:.2e}")
    assert err_v <= 1e-2 and err_k <= 1e-2
    assert torch.isfinite(dQ).all() and torch.isfinite(dK).all() and torch.isfinite(dV).all()


def _long_samples(w):
    """Rows and keys of every kind in the long prompt: instruction, documents 0, 250 and 499 (first,
    second, middle and last token), and query tokens."""
    so = np.asarray(w.segment_offsets)
    T = w.total_tokens
    instr = [0, 1, int(so[1]) // 2, int(so[1]) - 1]
    docs = []
    for k in (0, 250, 499):
        a, e = int(so[1 + k]), int(so[2 + k])
        docs += [a, a + 1, (a + e) // 2, e - 1]
    query = [int(so[-2]), int(so[-2]) + 1, T - 9, T - 1]
    return instr, docs, query


@pytest.fixture(scope="module")
def long_bwd():
    w = workloads.make("long", 0)
    log(f"[attn bwd long samples] T={w.total_tokens}: GPU forward + backward")
    dQ, dK, dV, dO_bits = run_case(w, 11)
    return w, dQ.cpu(), dK.cpu(), dV.cpu(), dO_bits


def test_attn_bwd_long_prompt_sampled_rows_and_document_keys(long_bwd):
    """The long ranking prompt at full size: dQ at instruction, document and query rows and dK, dV
    at document and query keys, element by element against the oracle's sampled backward (each
    key's gradient summed over every row that reads it, the query rows included)."""
    w, dQ, dK, dV, dO_bits = long_bwd
    instr, docs, query = _long_samples(w)
    rows = instr + docs + query
    keys = docs + query
    log(f"  oracle: {len(rows)} rows, {len(keys)} keys, all heads")
    rQ, rK, rV = orc.attn_bwd_sampled(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr, rows, keys)
    check_grad(dQ[rows], rQ, "dQ rows")
    check_grad(dK[keys], rK, "dK document/query keys")
    check_grad(dV[keys], rV, "dV document/query keys")


def test_attn_bwd_long_prompt_instruction_keys(long_bwd):
    """dK and dV of instruction keys, which every one of the ~100k rows reads (the GPU sums them over
    split row ranges), for two KV heads against the oracle's sampled backward."""
    w, dQ, dK, dV, dO_bits = long_bwd
    instr, _, _ = _long_samples(w)
    heads = [0, 5]
    log(f"  oracle: instruction keys {instr}, KV heads {heads}, every reading row")
    _, rK, rV = orc.attn_bwd_sampled(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr, [], instr,
                                     kv_heads=heads)
    check_grad(dK[instr][:, heads], rK[:, heads], "dK instruction keys")
    check_grad(dV[instr][:, heads], rV[:, heads], "dV instruction keys")


def test_attn_bwd_edge_shapes():
    """Degenerate tables: no instruction, one-token documents and queries, a single document, and
    the largest group size."""
    prompts = [(0, [1, 1, 5], 1), (3, [1], 1), (0, [7], 2), (1, [2, 1, 1, 1], 3)]
    for hq, hkv, d in ((8, 1, 64), (4, 4, 128)):
        w = workloads.make_custom(prompts, hq, hkv, d, 1, 2800 + hq)
        log(f"[attn bwd edge] Hq={hq} Hkv={hkv} d={d} T={w.total_tokens}")
        dQ, dK, dV, dO_bits = run_case(w, 13)
        rQ, rK, rV = orc.attn_bwd(w.Q, w.K, w.V, dO_bits, w.segment_offsets, w.seg_ptr)
        check_grad(dQ, rQ, "dQ")
        check_grad(dK, rK, "dK")
        check_grad(dV, rV, "dV")


def test_readout_bwd_single_document_is_zero():
    """With one document per prompt every score is |S| whatever Q_S and K are: the readout's
    gradient is exactly zero (and InfoNCE's loss is zero)."""
    prompts = [(4, [9], 3), (0, [5], 2)]
    w = workloads.make_custom(prompts, 8, 2, 64, 2, 2900)
    dev = upload(w)
    log("[readout bwd] one document per prompt")
    scores = br.doc_scores(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr)
    loss, ds = br.infonce(scores, w.doc_ptr, np.zeros(2, dtype=np.int32))
    dQs, dK = br.doc_scores_bwd(dev["Q_S"], dev["K"], w.doc_offsets, w.doc_ptr, ds)
    torch.cuda.synchronize()
    assert torch.count_nonzero(loss) == 0 and torch.count_nonzero(ds) == 0
    assert torch.count_nonzero(dQs) == 0 and torch.count_nonzero(dK) == 0
