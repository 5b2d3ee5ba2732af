"""Plain CPU oracle of the HQMQ KV-cache codec and of decode attention over it.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``__graft_entry__.smoke()``.
It imports nothing from the HIP library and the HIP library imports nothing
from here.

Source (web page; cited by title and section):
  [HQMQ-S]  "Technical summary: Hurwitz quaternion multiplicative quantization
            for KV cache compression" (gist.science, paper 2605.27646),
            sections "Method" 1 (multiplicative codebook), 2 (random
            initialisation), 3 (median-multiple outlier extraction, Med3x),
            and "Memory and latency" (fused decode).

What the page fixes:
  * every 4-element chunk of a K or V vector is a quaternion x, split into
    its radius r = |x| and its direction u = x / r on the 3-sphere;
  * the primary codebook P is the 24 unit Hurwitz quaternions (the binary
    tetrahedral group 2T, the vertices of the 24-cell);
  * the secondary codebook S is S random unit quaternions per (layer, head,
    role), drawn without calibration;
  * the codebook is C = {q_p q_s : q_p in P, q_s in S} (24 S words from S
    stored quaternions), and u is coded by the word c maximising <u, c>;
  * Med3x: with r_med the median chunk norm of the current batch, chunks
    with r > 3 r_med are kept in fp16 and flagged with one bit, the rest are
    coded by HQMQ;
  * the fused kernel decodes K and V inside the attention loop.

What the page leaves open, and the reading taken here (each also listed
with its reason in the design notes of the repository):
  H1  chunk j of a 128-vector is channels 4j .. 4j + 3 = (a, b, c, d) of
      a + b i + c j + d k;
  H2  P is enumerated as: index 2a + s (a = 0..3, s = 0..1) is the unit
      along axis a (1, i, j, k) with sign (-1)^s; index 8 + m (m = 0..15) is
      (1/2)(+-1, +-1, +-1, +-1) with component t negative iff bit t of m is
      set.  Codeword index = 24 s + p for q_p q_s;
  H3  quaternion products use Hamilton's rule, in the order q_p q_s that the
      page writes; the codebook is the fp32 rounding of the fp64 product;
  H4  the argmax is taken in fp32: u = x / r and each score
      ((u0 c0 + u1 c1) + u2 c2) + u3 c3 with every product and sum rounded
      separately; ties go to the lowest index; r = 0 codes index 0;
      r = sqrt(((x0^2 + x1^2) + x2^2) + x3^2) the same way;
  H5  the radius is coded in 8 bits, uniformly over [0, r_max] with r_max
      the fp16 rounding of the record's largest coded radius:
      code = clamp(rint(r * fp32(255 / r_max)), 0, 255), decoded as
      code * r_max / 255;
  H6  at most 10 secondary quaternions, so a codeword index fits 8 bits;
  H7  "the current batch" is all chunks of one role (K or V) over all
      tokens and KV heads of one append call; its median is the lower
      median (element (n - 1) // 2 of the ascending order); the threshold
      is fp32(3 * r_med);
  H8  a record holds at most 3 fp16 chunks; with more candidates the 3 of
      largest radius stay fp16 (ties: lower chunk index), the others are
      coded;
  H9  HQMQ needs no calibration and no rotation; every token is coded when
      it is appended (no bf16 window);
  H10 one (token, KV head, role) record is 96 bytes:
        [0, 32)   codeword index of chunk j at byte j (0 for fp16 chunks)
        [32, 64)  radius code of chunk j at byte 32 + j (0 for fp16 chunks)
        [64, 66)  r_max (fp16); [66, 68) zero
        [68, 72)  flags (uint32, bit j: chunk j is kept in fp16)
        [72, 96)  three fp16 chunk slots: the flagged chunks in ascending
                  chunk order, 4 fp16 each; unused slots zero
      and a page of P tokens holds, per KV head, P tokens x (K record,
      V record): record (page, h, slot, role) at
      ((page Hkv + h) P + slot) 192 + 96 role.

Decode attention is exact given the cache contents: plain softmax attention
in fp64 over the decoded K and V, one query head g reading KV head g // G.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .kvq_oracle import attention, bf16_bits_to_f32, f16_bits_to_f32, f32_to_f16_bits

HEAD_DIM = 128
N_CHUNKS = HEAD_DIM // 4
PRIMARY = 24
MAX_SECONDARY = 10
MAX_OUTLIERS = 3
OUTLIER_FACTOR = 3.0
RECORD_BYTES = 96
TOKEN_BYTES = 2 * RECORD_BYTES
RADIUS_LEVELS = 255
IDX_OFF, RAD_OFF, RMAX_OFF, FLAGS_OFF, OUT_OFF = 0, 32, 64, 68, 72


# --------------------------------------------------------------------------
# Quaternions and the binary tetrahedral group  [HQMQ-S Method 1]
# --------------------------------------------------------------------------

def hamilton(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Hamilton product p q of quaternions (a, b, c, d) = a + b i + c j + d k,
    in fp64, each component summed left to right as written."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    a1, b1, c1, d1 = p[..., 0], p[..., 1], p[..., 2], p[..., 3]
    a2, b2, c2, d2 = q[..., 0], q[..., 1], q[..., 2], q[..., 3]
    return np.stack([
        a1 * a2 - b1 * b2 - c1 * c2 - d1 * d2,
        a1 * b2 + b1 * a2 + c1 * d2 - d1 * c2,
        a1 * c2 - b1 * d2 + c1 * a2 + d1 * b2,
        a1 * d2 + b1 * c2 - c1 * b2 + d1 * a2,
    ], axis=-1)


def binary_tetrahedral() -> np.ndarray:
    """The 24 unit Hurwitz quaternions [24][4] fp64 in the enumeration H2."""
    out = np.zeros((PRIMARY, 4))
    for a in range(4):
        for s in range(2):
            out[2 * a + s, a] = -1.0 if s else 1.0
    for m in range(16):
        for t in range(4):
            out[8 + m, t] = -0.5 if (m >> t) & 1 else 0.5
    return out


def codebook(secondary: np.ndarray) -> np.ndarray:
    """C = {q_p q_s} as fp32 [24 S][4]: word 24 s + p = fp32(q_p q_s)
    [HQMQ-S Method 1; readings H2, H3]."""
    sec = np.asarray(secondary, np.float32)
    assert sec.ndim == 2 and sec.shape[1] == 4 and 1 <= sec.shape[0] <= MAX_SECONDARY
    P = binary_tetrahedral()
    out = np.zeros((PRIMARY * sec.shape[0], 4), np.float32)
    for s in range(sec.shape[0]):
        for p in range(PRIMARY):
            out[PRIMARY * s + p] = hamilton(P[p], sec[s].astype(np.float64)).astype(np.float32)
    return out


# --------------------------------------------------------------------------
# Encoding  [HQMQ-S Method 1 and 3; readings H1, H4, H5, H7, H8]
# --------------------------------------------------------------------------

def chunk_norms(x: np.ndarray) -> np.ndarray:
    """fp32 radii [..., 32] of fp32 vectors [..., 128] (reading H4)."""
    c = np.asarray(x, np.float32).reshape(*np.shape(x)[:-1], N_CHUNKS, 4)
    sq = c * c                                     # each product rounded to fp32
    s = ((sq[..., 0] + sq[..., 1]) + sq[..., 2]) + sq[..., 3]
    return np.sqrt(s).astype(np.float32)


def lower_median(values: np.ndarray) -> np.float32:
    """Element (n - 1) // 2 of the ascending order (reading H7)."""
    v = np.sort(np.asarray(values, np.float32).reshape(-1))
    return v[(v.size - 1) // 2]


def outlier_threshold(norms: np.ndarray) -> np.float32:
    """fp32(3 r_med) over all chunk norms of one role in one call [Med3x]."""
    return np.float32(np.float32(OUTLIER_FACTOR) * lower_median(norms))


def direction_index(u: np.ndarray, cb: np.ndarray) -> int:
    """First index of the largest fp32 score ((u0 c0 + u1 c1) + u2 c2) + u3 c3."""
    u = np.asarray(u, np.float32)
    prod = cb * u[None, :]                          # fp32 products
    sc = ((prod[:, 0] + prod[:, 1]) + prod[:, 2]) + prod[:, 3]
    return int(np.argmax(sc))                       # argmax returns the first maximum


def encode_record(x_bits: np.ndarray, cb: np.ndarray, thr: np.float32) -> np.ndarray:
    """The 96-byte record of one bf16 vector [128] (reading H10)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float32)
    r = chunk_norms(x)
    cand = [j for j in range(N_CHUNKS) if r[j] > thr]
    # capacity: the largest radii stay fp16 (ties: lower chunk index)
    cand.sort(key=lambda j: (-float(r[j]), j))
    fp16_chunks = sorted(cand[:MAX_OUTLIERS])
    coded = [j for j in range(N_CHUNKS) if j not in fp16_chunks]
    r_max = max((float(r[j]) for j in coded), default=0.0)
    r_max_bits = int(f32_to_f16_bits(np.float32(r_max)))
    r_max_h = f16_bits_to_f32(np.uint16(r_max_bits))
    rec = np.zeros(RECORD_BYTES, np.uint8)
    inv = np.float32(np.float32(RADIUS_LEVELS) / r_max_h) if r_max_h > 0 else np.float32(0)
    for j in coded:
        if r[j] > 0:
            u = x[4 * j:4 * j + 4] / r[j]           # four fp32 divisions
            rec[IDX_OFF + j] = direction_index(u, cb)
        if r_max_h > 0:
            t = np.float32(r[j] * inv)
            rec[RAD_OFF + j] = int(min(max(np.rint(t), 0.0), float(RADIUS_LEVELS)))
    rec[RMAX_OFF:RMAX_OFF + 2] = np.array([r_max_bits], np.uint16).view(np.uint8)
    flags = 0
    for e, j in enumerate(fp16_chunks):
        flags |= 1 << j
        h = f32_to_f16_bits(x[4 * j:4 * j + 4])
        rec[OUT_OFF + 8 * e:OUT_OFF + 8 * e + 8] = h.view(np.uint8)
    rec[FLAGS_OFF:FLAGS_OFF + 4] = np.array([flags], np.uint32).view(np.uint8)
    return rec


def decode_record(rec: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """fp64 vector [128] of one record: r_hat c for coded chunks (r_hat =
    code r_max / 255), the fp16 values for kept chunks."""
    rec = np.asarray(rec, np.uint8)
    r_max = float(f16_bits_to_f32(rec[RMAX_OFF:RMAX_OFF + 2].view(np.uint16))[0])
    flags = int(rec[FLAGS_OFF:FLAGS_OFF + 4].view(np.uint32)[0])
    out = np.zeros(HEAD_DIM)
    e = 0
    for j in range(N_CHUNKS):
        if flags >> j & 1:
            out[4 * j:4 * j + 4] = f16_bits_to_f32(
                rec[OUT_OFF + 8 * e:OUT_OFF + 8 * e + 8].view(np.uint16))
            e += 1
        else:
            r_hat = int(rec[RAD_OFF + j]) * r_max / RADIUS_LEVELS
            out[4 * j:4 * j + 4] = r_hat * cb[int(rec[IDX_OFF + j])].astype(np.float64)
    return out


# --------------------------------------------------------------------------
# The paged cache  [HQMQ-S "Memory and latency"; readings H9, H10]
# --------------------------------------------------------------------------

@dataclass
class HqmqDims:
    n_q_heads: int
    n_kv_heads: int
    page_size: int
    n_secondary: int
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def record_offset(d: HqmqDims, page: int, h: int, slot: int, role: int) -> int:
    return ((page * d.n_kv_heads + h) * d.page_size + slot) * TOKEN_BYTES + role * RECORD_BYTES


class HqmqCache:
    """pool uint8 [num_pages][Hkv][P][2][96]; block_table int32 [B][stride]
    maps logical page pos // P of sequence b to a physical page."""

    def __init__(self, d: HqmqDims, batch: int, num_pages: int, block_table: np.ndarray,
                 codebooks: np.ndarray, fill: int = 0):
        self.d = d
        self.B = batch
        self.block_table = np.asarray(block_table, np.int32)
        self.pool = np.full(num_pages * d.n_kv_heads * d.page_size * TOKEN_BYTES, fill, np.uint8)
        self.cb = np.asarray(codebooks, np.float32)     # [2][Hkv][24 S][4]
        assert self.cb.shape == (2, d.n_kv_heads, PRIMARY * d.n_secondary, 4)

    def append(self, starts, k_new: list, v_new: list):
        """One append call: k_new[b] / v_new[b] bf16 bits [n_b][Hkv][128] go to
        positions starts[b] .. starts[b] + n_b - 1.  The Med3x median runs
        over all chunks of each role in the call."""
        d = self.d
        thr = []
        for role, xs in enumerate((k_new, v_new)):
            vals = [chunk_norms(bf16_bits_to_f32(x)) for x in xs if len(x)]
            thr.append(outlier_threshold(np.concatenate([v.reshape(-1) for v in vals]))
                       if vals else np.float32(0))
        for b in range(self.B):
            for i in range(len(k_new[b])):
                pos = int(starts[b]) + i
                page = int(self.block_table[b, pos // d.page_size])
                for h in range(d.n_kv_heads):
                    for role, xs in enumerate((k_new, v_new)):
                        rec = encode_record(xs[b][i, h], self.cb[role, h], thr[role])
                        off = record_offset(d, page, h, pos % d.page_size, role)
                        self.pool[off:off + RECORD_BYTES] = rec
        return thr

    def record(self, b: int, pos: int, h: int, role: int) -> np.ndarray:
        d = self.d
        page = int(self.block_table[b, pos // d.page_size])
        off = record_offset(d, page, h, pos % d.page_size, role)
        return self.pool[off:off + RECORD_BYTES]

    def decoded(self, b: int, length: int, h: int):
        """(K, V) fp64 [length][128] of sequence b, KV head h."""
        K = np.stack([decode_record(self.record(b, p, h, 0), self.cb[0, h])
                      for p in range(length)]) if length else np.zeros((0, HEAD_DIM))
        V = np.stack([decode_record(self.record(b, p, h, 1), self.cb[1, h])
                      for p in range(length)]) if length else np.zeros((0, HEAD_DIM))
        return K, V

    def decode(self, seq_len, q_bits: np.ndarray) -> np.ndarray:
        """Decode attention of q [B][Hq][128] (bf16 bits) over positions
        [0, seq_len[b]): fp32 out [B][Hq][128]."""
        d = self.d
        out = np.zeros((self.B, d.n_q_heads, HEAD_DIM), np.float32)
        for b in range(self.B):
            L = int(seq_len[b])
            for h in range(d.n_kv_heads):
                K, V = self.decoded(b, L, h)
                for g in range(h * d.group, (h + 1) * d.group):
                    q = bf16_bits_to_f32(q_bits[b, g]).astype(np.float64)
                    out[b, g] = attention(q, K, V, d.sm_scale).astype(np.float32)
        return out


def bits_per_element() -> float:
    """Bits per cached K or V element of the record layout (reading H10)."""
    return RECORD_BYTES * 8 / HEAD_DIM
