"""Seeded synthetic ranking prompts shared by the GPU path's tests, the bench and the oracle.

This module only *draws* inputs: segment tables, bf16 Q/K/V tensors and the signal-token
queries.  It holds none of the method's arithmetic (no mask, no softmax, no score); both
the CPU oracle and the HIP path consume what it returns.

Prompt layout (BlockRank blog, section on candidate arrangement): a ranking prompt is
``P = I || d_1 || ... || d_N || q`` -- an instruction prefix of ``p`` tokens, ``N``
documents of ragged lengths ``l_k`` and a final query of ``q`` tokens.  Several prompts
are packed back to back on one token axis ("THD" layout).

Shapes follow a Mistral-7B attention layer (32 query heads, 8 KV heads, head dim 128);
the BlockRank summary only says the model is Mistral-7B with grouped-query attention.
Values are N(0, 1) draws rounded to bf16 (round to nearest even); there are no trained
activations or datasets here, so these stand in for the MSMarco/BEIR-shaped prompts of
the BlockRank summary (~20K tokens at N=100, chunks of ~160 tokens, top-100 lists).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = ["Workload", "CONFIGS", "make", "make_custom", "segment_tables", "f32_to_bf16_bits",
           "bf16_bits_to_f32"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite by construction (normal draws), so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    n_signal: int
    # per prompt: (p, [l_1..l_N], q)
    prompts: List[tuple]
    # HOST int32 segment table: prompt b owns segment_offsets[seg_ptr[b] : seg_ptr[b+1]]
    # = {start, start+p, start+p+l_1, ..., start+p+D, start+L}  (N_b + 3 entries)
    segment_offsets: np.ndarray
    seg_ptr: np.ndarray
    # HOST int32 document spans: prompt b owns doc_offsets[doc_ptr[b] : doc_ptr[b+1]] (N_b + 1 entries)
    doc_offsets: np.ndarray
    doc_ptr: np.ndarray
    # bf16 bits (uint16), token-major packed
    Q: np.ndarray  # [T, Hq, d]
    K: np.ndarray  # [T, Hkv, d]
    V: np.ndarray  # [T, Hkv, d]
    Q_S: np.ndarray  # [B, n_signal, Hq, d]  (copies of the last n_signal query rows of each prompt)
    planted: Optional[List[int]] = None  # per prompt, local index of the planted document
    meta: Dict = field(default_factory=dict)

    @property
    def num_prompts(self) -> int:
        return len(self.prompts)

    @property
    def total_tokens(self) -> int:
        return int(self.segment_offsets[-1])

    @property
    def num_docs(self) -> int:
        return int(self.doc_offsets.shape[0] - self.num_prompts)

    def signal_rows(self) -> np.ndarray:
        """Absolute token index of each signal row, [B, n_signal]."""
        rows = []
        for b in range(self.num_prompts):
            end = int(self.segment_offsets[self.seg_ptr[b + 1] - 1])
            rows.append(np.arange(end - self.n_signal, end))
        return np.asarray(rows, dtype=np.int64)


# Named configurations.  Each entry: heads, dims, signal count, batch, and a length recipe.
CONFIGS: Dict[str, dict] = {
    # 1 head, d=64, p=32, N=4 docs of 64 tokens, q=32 (L=320), |S|=4
    "tiny": dict(hq=1, hkv=1, d=64, n_signal=4, batch=1, p=32, q=32, n_docs=4, lens=("fixed", 64)),
    # the blog's worked shape: p=q=32, N=100, l=128 (L=12,864), Mistral-7B layer 32/8 heads, d=128
    "worked": dict(hq=32, hkv=8, d=128, n_signal=8, batch=1, p=32, q=32, n_docs=100, lens=("fixed", 128)),
    # long list: p=64, q=32, N=500, l=200 (L=100,096)
    "long": dict(hq=32, hkv=8, d=128, n_signal=8, batch=1, p=64, q=32, n_docs=500, lens=("fixed", 200)),
    # ragged: p=48, q=24, N=200, l ~ U{32..256}; one planted document (length 256, K shifted)
    "ragged": dict(hq=32, hkv=8, d=128, n_signal=8, batch=1, p=48, q=24, n_docs=200,
                   lens=("uniform", 32, 256), plant=True),
    # batched re-rank: 16 prompts, p=q=32, N=100, l ~ U{64..192}
    "batched": dict(hq=32, hkv=8, d=128, n_signal=8, batch=16, p=32, q=32, n_docs=100,
                    lens=("uniform", 64, 192)),
}

PLANT_SHIFT = 0.5     # K rows of the planted document move by PLANT_SHIFT * mean(Q_S of the group)
PLANT_LENGTH = 256    # planted document length (top of the ragged range)


def segment_tables(prompts):
    """(segment_offsets, seg_ptr, doc_offsets, doc_ptr) int32 arrays for packed prompts."""
    seg, seg_ptr, doc, doc_ptr = [], [0], [], [0]
    start = 0
    for (p, lens, q) in prompts:
        offs = [start, start + p]
        for l in lens:
            offs.append(offs[-1] + int(l))
        offs.append(offs[-1] + q)
        seg.extend(offs)
        seg_ptr.append(len(seg))
        doc.extend(offs[1:-1])
        doc_ptr.append(len(doc))
        start = offs[-1]
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return i32(seg), i32(seg_ptr), i32(doc), i32(doc_ptr)


def make_custom(prompts, hq, hkv, d, n_signal, seed, name="custom", plant_docs=None,
                q_scale: float = 1.0) -> Workload:
    """Build a workload from explicit (p, lengths, q) per prompt.

    Draw order with ``numpy.random.default_rng(seed)``: Q [T,Hq,d], K [T,Hkv,d], V [T,Hkv,d]
    as float32 standard normals, each rounded to bf16.  ``q_scale`` multiplies Q before
    rounding (used for sharp-softmax stress inputs).  ``plant_docs`` (one local doc index or
    None per prompt) shifts that document's K rows by PLANT_SHIFT * u_g, where u_g is the mean
    of the bf16 signal-query rows of KV group g, and re-rounds to bf16.
    """
    rng = np.random.default_rng(seed)
    return _draw(rng, prompts, hq, hkv, d, n_signal, seed, name, plant_docs, q_scale)


def _draw(rng, prompts, hq, hkv, d, n_signal, seed, name, plant_docs, q_scale=1.0) -> Workload:
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    seg, seg_ptr, doc, doc_ptr = segment_tables(prompts)
    T = int(seg[-1])
    q32 = rng.standard_normal((T, hq, d), dtype=np.float32)
    if q_scale != 1.0:
        q32 *= np.float32(q_scale)
    Q = f32_to_bf16_bits(q32)
    del q32
    K = f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    V = f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    B = len(prompts)
    ends = [int(seg[seg_ptr[b + 1] - 1]) for b in range(B)]
    for b, (p, lens, q) in enumerate(prompts):
        if q < n_signal:
            raise ValueError("q must be >= n_signal")
    G = hq // hkv
    if plant_docs is not None:
        for b in range(B):
            k = plant_docs[b]
            if k is None:
                continue
            qs = bf16_bits_to_f32(Q[ends[b] - n_signal:ends[b]])  # [S, Hq, d]
            a = int(doc[doc_ptr[b] + k]); e = int(doc[doc_ptr[b] + k + 1])
            for g in range(hkv):
                u = qs[:, g * G:(g + 1) * G, :].reshape(-1, d).mean(axis=0, dtype=np.float32)
                kf = bf16_bits_to_f32(K[a:e, g, :]) + np.float32(PLANT_SHIFT) * u
                K[a:e, g, :] = f32_to_bf16_bits(kf)
    Q_S = np.stack([Q[e - n_signal:e] for e in ends], axis=0)
    return Workload(name=name, seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    n_signal=n_signal, prompts=[(p, list(map(int, l)), q) for (p, l, q) in prompts],
                    segment_offsets=seg, seg_ptr=seg_ptr, doc_offsets=doc, doc_ptr=doc_ptr,
                    Q=Q, K=K, V=V, Q_S=np.ascontiguousarray(Q_S),
                    planted=None if plant_docs is None else list(plant_docs))


def make(name: str, seed: int = 0, q_scale: float = 1.0) -> Workload:
    """Generate a named configuration.

    Draw order: per prompt the document lengths (then, for planted configs, the planted
    index drawn with ``rng.integers(N)``), then Q, K, V for the whole packed token axis.
    """
    c = CONFIGS[name]
    rng = np.random.default_rng(seed)
    prompts, plants = [], []
    for _ in range(c["batch"]):
        kind = c["lens"][0]
        if kind == "fixed":
            lens = np.full(c["n_docs"], c["lens"][1], dtype=np.int64)
        else:
            lens = rng.integers(c["lens"][1], c["lens"][2] + 1, size=c["n_docs"])
        plant = None
        if c.get("plant"):
            plant = int(rng.integers(c["n_docs"]))
            lens[plant] = PLANT_LENGTH
        prompts.append((c["p"], [int(x) for x in lens], c["q"]))
        plants.append(plant)
    w = _draw(rng, prompts, c["hq"], c["hkv"], c["d"], c["n_signal"], seed, name,
              plants if c.get("plant") else None, q_scale)
    w.meta = dict(config=name)
    return w
