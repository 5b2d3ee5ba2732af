"""Seeded synthetic inputs for the INT2 decode workloads.

This module only draws random numbers and shapes them: it holds none of the
quantization or attention arithmetic, and it imports neither the HIP binding
nor the CPU oracle, so both sides can take their inputs from here.

Workloads (sizes as named in the method's serving scenarios):
  tiny          1 seq, 4 q / 2 KV heads, context 1024, page 16, sink 4, recent 128,
                q/K/V ~ N(0,1) bf16 with K channels {5, 37, 70, 101} scaled x20,
                rotation from 4096 seeded calibration tokens.
  qwen3_8b_32k  32 q / 8 KV heads, batch 1, context 32768, page 16, sink 4, recent 128,
                K with lognormal per-(head, channel) scales (sigma 1) and 2 % outlier
                channels x30; q, V ~ N(0,1).
  b1_131k       as above, context 131072, page 64; one decode step appends one token.
  conc_28x100k  32 q / 8 KV heads, batch 28 x 100000-token contexts, sink 4, recent 256,
                page 16, physical pages a seeded random permutation.
  qwen3_32b     64 q / 8 KV heads, batch 64, contexts uniform in [4096, 65536]; half of
                the long sequences share a 16384-token prefix (shared pages), page 16.

bf16 values are produced by torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    page_size: int
    n_sink: int
    n_recent: int
    context: int                     # fixed context, or the upper bound of a random draw
    context_min: int = 0             # >0: contexts uniform in [context_min, context]
    k_dist: str = "lognormal"        # "fixed4" | "lognormal"
    n_calib: int = 2048
    random_pages: bool = True
    shared_prefix: int = 0           # tokens shared (page-aligned) by half of the long sequences
    index: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def seq_lens(self) -> np.ndarray:
        """Context length of every sequence after this step's append."""
        if self.context_min <= 0:
            return np.full(self.batch, self.context, np.int64)
        rng = np.random.default_rng(3000 + self.index)
        return rng.integers(self.context_min, self.context + 1, size=self.batch).astype(np.int64)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 2, 16, 4, 128, 1024, k_dist="fixed4", n_calib=4096,
                     random_pages=True, index=0),
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 1, 32, 8, 16, 4, 128, 32768, index=1),
    "b1_131k": Workload("b1_131k", 1, 32, 8, 64, 4, 128, 131072, index=2),
    "conc_28x100k": Workload("conc_28x100k", 28, 32, 8, 16, 4, 256, 100000, index=3),
    "qwen3_32b": Workload("qwen3_32b", 64, 64, 8, 16, 4, 128, 65536, context_min=4096,
                          shared_prefix=16384, index=4),
}

FIXED_OUTLIER_CHANNELS = (5, 37, 70, 101)


def to_bf16_bits(x) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's RNE cast."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def k_channel_scales(w: Workload) -> np.ndarray:
    """Per (KV head, channel) multiplier of K: float32 [Hkv][128]."""
    if w.k_dist == "fixed4":
        a = np.ones((w.n_kv_heads, HEAD_DIM), np.float32)
        a[:, list(FIXED_OUTLIER_CHANNELS)] = 20.0
        return a
    rng = np.random.default_rng(4000 + w.index)
    a = np.exp(rng.standard_normal((w.n_kv_heads, HEAD_DIM))).astype(np.float32)
    n_out = int(math.ceil(0.02 * HEAD_DIM))
    for h in range(w.n_kv_heads):
        a[h, rng.choice(HEAD_DIM, n_out, replace=False)] *= 30.0
    return a


def normal_bits(seed: int, shape, scale=None) -> np.ndarray:
    """N(0,1) float32 (times an optional broadcast scale) -> bf16 bits, seeded PCG64."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if scale is not None:
        x = x * scale
    return to_bf16_bits(x)


def calibration_tokens(w: Workload, n_tokens: int | None = None):
    """(q, k, v) bf16 bits [N][H][128] for offline calibration (seed 1000 + index)."""
    n = w.n_calib if n_tokens is None else n_tokens
    s = 1000 + w.index
    q = normal_bits(s * 10 + 0, (n, w.n_q_heads, HEAD_DIM))
    k = normal_bits(s * 10 + 1, (n, w.n_kv_heads, HEAD_DIM), k_channel_scales(w)[None])
    v = normal_bits(s * 10 + 2, (n, w.n_kv_heads, HEAD_DIM))
    return q, k, v


def sequence_kv(w: Workload, b: int, length: int, offset: int = 0):
    """(k, v) bf16 bits [length][Hkv][128] of tokens [offset, offset+length) of sequence b.

    Host draw (seed 2000 + 100*index + b); used for small workloads and for
    sampled rows of large ones.  Tokens are drawn in blocks of 4096 so that a
    sub-range is reproducible without drawing the whole sequence.
    """
    scale = k_channel_scales(w)[None]
    ks, vs = [], []
    blk = 4096
    first, last = offset // blk, (offset + length - 1) // blk if length > 0 else offset // blk - 1
    for i in range(first, last + 1):
        seed = (2000 + 100 * w.index + b) * 100003 + i
        kb = normal_bits(seed * 2, (blk, w.n_kv_heads, HEAD_DIM), scale)
        vb = normal_bits(seed * 2 + 1, (blk, w.n_kv_heads, HEAD_DIM))
        ks.append(kb)
        vs.append(vb)
    if not ks:
        z = np.zeros((0, w.n_kv_heads, HEAD_DIM), np.uint16)
        return z, z.copy()
    k = np.concatenate(ks)[offset - first * blk: offset - first * blk + length]
    v = np.concatenate(vs)[offset - first * blk: offset - first * blk + length]
    return k, v


def decode_queries(w: Workload, step: int = 0) -> np.ndarray:
    """q bf16 bits [B][Hq][128] of one decode step."""
    return normal_bits(5000 + 100 * w.index + step, (w.batch, w.n_q_heads, HEAD_DIM))


def page_assignment(w: Workload, seq_lens: np.ndarray, extra_pages: int = 0):
    """Block table [B][max_pages] int32 and the number of physical pages.

    Logical pages of all sequences are laid out, then (if random_pages) the
    physical page numbers are a seeded random permutation.  With a shared
    prefix, the first 16384 tokens of half of the long sequences map to one
    shared set of physical pages.
    """
    P = w.page_size
    npages = [int(math.ceil(int(L) / P)) for L in seq_lens]
    stride = max(npages) if npages else 1
    bt = np.zeros((len(seq_lens), stride), np.int32)
    shared_pages = w.shared_prefix // P if w.shared_prefix else 0
    sharers = []
    if shared_pages:
        long_ids = [b for b, L in enumerate(seq_lens) if L > w.shared_prefix + w.n_recent]
        sharers = long_ids[: len(long_ids) // 2]
    logical = []                      # list of (b, logical page) that own a private page
    for b, n in enumerate(npages):
        for p in range(n):
            if b in sharers and p < shared_pages and b != sharers[0]:
                continue
            logical.append((b, p))
    total = len(logical) + extra_pages
    phys = np.arange(total, dtype=np.int64)
    if w.random_pages:
        phys = np.random.default_rng(6000 + w.index).permutation(total)
    owner = {}
    for i, (b, p) in enumerate(logical):
        bt[b, p] = phys[i]
        owner[(b, p)] = phys[i]
    for b in sharers[1:]:
        for p in range(shared_pages):
            bt[b, p] = owner[(sharers[0], p)]
    return bt, total, sharers


# --------------------------------------------------------------------------
# Device-side draws for the large workloads (torch's GPU generator).  The
# same seeds give the same values on every call, so a sub-range (one
# sequence, one block of tokens) can be re-drawn and copied to the host.
# --------------------------------------------------------------------------

DEVICE_BLOCK = 4096


def sequence_kv_device(w: Workload, b: int, offset: int, length: int, device="cuda"):
    """(k, v) bf16 bit patterns as int16 tensors [length][Hkv][128] on `device`.

    Token block i (DEVICE_BLOCK tokens) of sequence b is drawn from a torch
    generator seeded with (7000 + 100*index + b) * 100003 + i.  With a shared
    prefix, sequences that share it draw their first `shared_prefix` tokens
    from the first sharer's seed.
    """
    scale = torch.from_numpy(k_channel_scales(w)).to(device)[None]
    out_k, out_v = [], []
    first = offset // DEVICE_BLOCK
    last = (offset + length - 1) // DEVICE_BLOCK
    for i in range(first, last + 1):
        bb = b
        if w.shared_prefix and (i + 1) * DEVICE_BLOCK <= w.shared_prefix:
            bb = _shared_owner(w, b)
        gen = torch.Generator(device=device)
        gen.manual_seed((7000 + 100 * w.index + bb) * 100003 + i)
        shape = (DEVICE_BLOCK, w.n_kv_heads, HEAD_DIM)
        k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale
        v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        out_k.append(k.to(torch.bfloat16).view(torch.int16))
        out_v.append(v.to(torch.bfloat16).view(torch.int16))
    k = torch.cat(out_k)[offset - first * DEVICE_BLOCK: offset - first * DEVICE_BLOCK + length]
    v = torch.cat(out_v)[offset - first * DEVICE_BLOCK: offset - first * DEVICE_BLOCK + length]
    return k.contiguous(), v.contiguous()


def _shared_owner(w: Workload, b: int) -> int:
    _, _, sharers = page_assignment(w, w.seq_lens())
    return sharers[0] if b in sharers else b


def decode_queries_device(w: Workload, step: int, device="cuda") -> torch.Tensor:
    """q bf16 bits (int16 tensor) [B][Hq][128] for decode step `step`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(9000 + 100 * w.index + step)
    q = torch.randn((w.batch, w.n_q_heads, HEAD_DIM), generator=gen, device=device)
    return q.to(torch.bfloat16).view(torch.int16).contiguous()


# --------------------------------------------------------------------------
# HQMQ inputs: the secondary codebook is S Haar-random unit quaternions per
# (KV head, role), drawn without calibration; both the library and the CPU
# oracle take them from here.
# --------------------------------------------------------------------------

def hqmq_secondary(seed: int, n_kv_heads: int, n_secondary: int) -> np.ndarray:
    """fp32 [2][Hkv][S][4]: normalised standard-normal 4-vectors (uniform on
    the 3-sphere), role 0 for K and 1 for V."""
    g = np.random.default_rng(seed).standard_normal((2, n_kv_heads, n_secondary, 4))
    return (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)
