"""Plain, slow CPU oracle of OSCAR-style INT2 KV-cache decode (NumPy, fp64).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg.  It imports nothing from the HIP library
and the HIP library imports nothing from here.

Sources (web pages; cited by title and section):
  [OSCAR-S]  "Technical summary: OSCAR - Offline Spectral Covariance-Aware
             Rotation for 2-bit KV cache quantization" (gist.science,
             paper 2605.17757), sections 1, 2.1, 2.2-A (offline calibration,
             items 1-4), 2.2-B (online serving), 3, 4.
  [OSCAR-N]  tilnote.io blog note on OSCAR (Together AI): sections
             "attention-aware rotation" and "why it matters for serving".

Conventions (readings where the pages are silent; all are listed with their
reasons in the design notes of the repository):
  * head_dim d = 128; one quantization group = one (token, KV head) vector.
  * Rotated vectors use x' = R^T x, so q' . k' = q . k, and the output of
    attention in rotated space is mapped back with o = R_V o'.
  * R = U H P with U the eigenbasis (descending eigenvalues, sign rule),
    H the 128x128 Sylvester Hadamard scaled by 1/sqrt(128), P the 7-bit
    bit-reversal permutation.
  * Asymmetric 2-bit quantizer with fp16 scale s = (max - min)/3 and fp16
    zero z = min, codes = clamp(rint((x - z)/s), 0, 3) in pinned fp32 steps.
  * The first n_sink tokens and the last n_recent tokens are kept in bf16
    (rotated); everything in between is INT2, in pages of P tokens.

Every function below that fixes a number the GPU library must reproduce bit
for bit (rotation, quantization, packing, cache placement) is written as the
sequence of rounding steps it performs.  Decode attention is exact given the
cache contents, so it is plain softmax attention in fp64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128
CHUNK_TOKENS = 16          # a page is a whole number of 16-token chunks
CHUNK_BYTES = 1152         # 512 K codes + 512 V codes + 64 K params + 64 V params
K_CODES_OFF = 0
V_CODES_OFF = 512
K_PARAMS_OFF = 1024
V_PARAMS_OFF = 1088

LOG2E = 1.4426950408889634


# --------------------------------------------------------------------------
# Number formats (IEEE round-to-nearest-even conversions)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    bfloat16 keeps the top 16 bits of a float32; rounding adds 0x7FFF plus the
    lowest kept bit before truncating.  Finite inputs only.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    rounding = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of float32 values (numpy cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


# --------------------------------------------------------------------------
# The fixed rotation R = U H P   [OSCAR-S 2.2-A items 2-3]
# --------------------------------------------------------------------------

def popcount(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.int64).copy()
    n = np.zeros_like(a)
    while np.any(a):
        n += a & 1
        a >>= 1
    return n


def hadamard(n: int = HEAD_DIM) -> np.ndarray:
    """Sylvester Hadamard matrix in natural order, scaled to be orthogonal.

    H[i][j] = (-1)^popcount(i & j) / sqrt(n).  [OSCAR-S 2.2-A item 3: the
    Hadamard factor H_Had that evens out per-channel importance.]
    """
    i = np.arange(n)
    sign = np.where(popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)
    return sign / math.sqrt(n)


def hadamard_blocks(n: int = HEAD_DIM, block: int = HEAD_DIM) -> np.ndarray:
    """Block-diagonal Hadamard: n / block copies of hadamard(block) on the
    diagonal (block = n is the full transform).  [OSCAR-S 2.2-A item 3 does
    not fix the transform's size; a block Hadamard is the reading under which
    smaller quantization groups keep their channel mixing local.]"""
    assert n % block == 0
    H = np.zeros((n, n))
    Hb = hadamard(block)
    for k in range(n // block):
        H[k * block:(k + 1) * block, k * block:(k + 1) * block] = Hb
    return H


def bitrev(i: int, bits: int = 7) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def bitrev_permutation(n: int = HEAD_DIM) -> np.ndarray:
    """P[i][j] = 1 iff j = bitrev(i).  An involution, so P = P^T.

    [OSCAR-S 2.2-A item 3: P_br interleaves high- and low-variance channels.]
    """
    bits = int(round(math.log2(n)))
    P = np.zeros((n, n))
    for i in range(n):
        P[i, bitrev(i, bits)] = 1.0
    return P


def eigenbasis(C: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Eigen-decomposition of a symmetric matrix [OSCAR-S 2.2-A item 2].

    Columns ordered by descending eigenvalue (a stable order on ties); each
    column's largest-magnitude entry (lowest index on ties) made positive.
    """
    w, U = np.linalg.eigh(np.asarray(C, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    w = w[order]
    U = U[:, order].copy()
    for c in range(U.shape[1]):
        k = int(np.argmax(np.abs(U[:, c])))
        if U[k, c] < 0:
            U[:, c] = -U[:, c]
    return w, U


def composite_rotation(U: np.ndarray, hadamard_block: int = HEAD_DIM) -> np.ndarray:
    """R = U . H_Had . P_br in fp64 [OSCAR-S 2.2-A item 3, the formula R_K = U_Q H P];
    H_Had is the full Sylvester transform, or its block-diagonal form."""
    n = U.shape[0]
    return U @ hadamard_blocks(n, hadamard_block) @ bitrev_permutation(n)


# --------------------------------------------------------------------------
# Offline calibration [OSCAR-S 2.2-A items 1-4; OSCAR-N attention-aware rotation]
# --------------------------------------------------------------------------

def query_covariance(q_group: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n q_n^T, pooled over the query heads of one KV head.

    q_group: [N, G, d] fp64.  Uncentered second moment; the pages write
    (1/N) sum q_n^T q_n with q_n a row vector, i.e. the outer product.
    """
    N, G, d = q_group.shape
    C = np.zeros((d, d))
    for g in range(G):
        C += q_group[:, g, :].T @ q_group[:, g, :]
    return C / (N * G)


def causal_attention_outputs(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             sm_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Causal softmax attention of one query head over N calibration tokens.

    Returns (S, O) with S the N x N row-stochastic score matrix (token n sees
    tokens 0..n) and O = S V.  The causal mask is a reading: the pages do not
    say which scores S are.
    """
    N = q.shape[0]
    logits = sm_scale * (q @ k.T)
    logits[np.triu_indices(N, 1)] = -np.inf
    logits -= logits.max(axis=1, keepdims=True)
    S = np.exp(logits)
    S /= S.sum(axis=1, keepdims=True)
    return S, S @ v


def score_covariance(q_group: np.ndarray, k: np.ndarray, v: np.ndarray,
                     sm_scale: float) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V = (1/N) O^T O, pooled over the group's query heads."""
    N, G, d = q_group.shape
    C = np.zeros((d, d))
    for g in range(G):
        _, O = causal_attention_outputs(q_group[:, g, :], k, v, sm_scale)
        C += O.T @ O
    return C / (N * G)


def nearest_rank_quantile(values: np.ndarray, p: float) -> float:
    """Nearest-rank p-quantile: the ceil(p*n)-th smallest value (rank clamped to [1, n])."""
    a = np.sort(np.asarray(values, dtype=np.float32).ravel())
    n = a.size
    k = min(max(int(math.ceil(p * n)), 1), n)
    return float(a[k - 1])


@dataclass
class Calibration:
    R_K: np.ndarray      # float32 [Hkv][128][128], applied as R^T x
    R_V: np.ndarray
    clip_K: float        # float32 value
    clip_V: float
    eig_Q: np.ndarray    # [Hkv][128] descending
    eig_S: np.ndarray


def calibrate(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
              n_q_heads: int, n_kv_heads: int, sm_scale: float,
              clip_quantile: float = 0.999, hadamard_block: int = HEAD_DIM) -> Calibration:
    """Offline calibration of one layer [OSCAR-S 2.2-A items 1-4].

    q_bits [N][Hq][128], k_bits / v_bits [N][Hkv][128] bf16 bit patterns.
    One R_K and one R_V per KV head; one clip threshold for K and one for V
    per layer, the nearest-rank quantile of |rotated calibration values| over
    all tokens, KV heads and channels.
    """
    G = n_q_heads // n_kv_heads
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    k = bf16_bits_to_f32(k_bits).astype(np.float64)
    v = bf16_bits_to_f32(v_bits).astype(np.float64)
    d = q.shape[-1]
    R_K = np.zeros((n_kv_heads, d, d), np.float32)
    R_V = np.zeros((n_kv_heads, d, d), np.float32)
    eQ = np.zeros((n_kv_heads, d))
    eS = np.zeros((n_kv_heads, d))
    for h in range(n_kv_heads):
        qg = q[:, h * G:(h + 1) * G, :]
        wq, UQ = eigenbasis(query_covariance(qg))
        ws, US = eigenbasis(score_covariance(qg, k[:, h, :], v[:, h, :], sm_scale))
        R_K[h] = composite_rotation(UQ, hadamard_block).astype(np.float32)
        R_V[h] = composite_rotation(US, hadamard_block).astype(np.float32)
        eQ[h], eS[h] = wq, ws
    rk = np.stack([rotate(k_bits[:, h, :], R_K[h]) for h in range(n_kv_heads)])
    rv = np.stack([rotate(v_bits[:, h, :], R_V[h]) for h in range(n_kv_heads)])
    clip_K = nearest_rank_quantile(np.abs(bf16_bits_to_f32(rk)), clip_quantile)
    clip_V = nearest_rank_quantile(np.abs(bf16_bits_to_f32(rv)), clip_quantile)
    return Calibration(R_K, R_V, clip_K, clip_V, eQ, eS)


# --------------------------------------------------------------------------
# Online path, step 1: rotation of a new K or V head-vector (pinned rounding)
# --------------------------------------------------------------------------

def rotate(x_bits: np.ndarray, R: np.ndarray) -> np.ndarray:
    """r = bf16(fp32(R^T x)) with a pinned fp64 accumulation order.

    For output channel i: acc = 0; for j = 0..127: acc += x_j * R[j][i] in
    fp64.  A bf16 x fp32 product is exact in fp64, so fused or unfused
    multiply-add give the same sum.  Then round to fp32, then to bf16.
    [OSCAR-S 2.2-B: history is stored after the fixed rotation.]
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    Rd = np.asarray(R, dtype=np.float32).astype(np.float64)
    acc = np.zeros(x.shape, np.float64)
    for j in range(x.shape[-1]):
        acc += x[..., j:j + 1] * Rd[j]
    return f32_to_bf16_bits(acc.astype(np.float32))


# --------------------------------------------------------------------------
# Online path, step 2: clip + asymmetric INT2 quantization (pinned fp32 steps)
# --------------------------------------------------------------------------

def quantize_groups(r_bits: np.ndarray, clip: float, group: int):
    """quantize() on each contiguous group of `group` channels of the rotated
    vectors [..., 128] separately: codes uint8 [..., 128] and fp16 bits of
    (scale, zero) [..., 128 / group], group k covering channels
    [k group, (k + 1) group).  [OSCAR-S 2.2-A item 3: P_br balances the
    dynamic range inside the quantization groups; with group < 128 each group
    has its own scale and zero.]"""
    r = np.asarray(r_bits, np.uint16)
    ng = HEAD_DIM // group
    parts = [quantize(r[..., k * group:(k + 1) * group], clip) for k in range(ng)]
    codes = np.concatenate([p[0] for p in parts], axis=-1)
    s = np.stack([p[1] for p in parts], axis=-1)
    z = np.stack([p[2] for p in parts], axis=-1)
    return codes, s, z


def quantize(r_bits: np.ndarray, clip: float):
    """Quantize rotated bf16 vectors [..., n] (one group each) to 2-bit codes +
    fp16 (scale, zero).

    [OSCAR-S 1 and 2.2-B: INT2 = 4 levels; 2.2-A item 4: per-layer clipping of
    rotated activations.]  Steps, all IEEE fp32 with RNE:
      x  = min(max(r, -c), c) + 0      (also turns -0 into +0)
      mn = min x, mx = max x, s = (mx - mn) / 3
      s_h = fp16(s), z_h = fp16(mn)
      if s_h == 0: codes = 0
      else: inv = 1 / s_h; t = (x - z_h) * inv (two roundings); code = clamp(rint(t), 0, 3)
    Returns (codes uint8 [..., n], s_h bits uint16 [...], z_h bits uint16 [...]).
    """
    r = bf16_bits_to_f32(r_bits)
    c = np.float32(clip)
    x = np.minimum(np.maximum(r, -c), c) + np.float32(0.0)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s = (mx - mn) / np.float32(3.0)
    s_bits = f32_to_f16_bits(s)
    z_bits = f32_to_f16_bits(mn)
    sf = f16_bits_to_f32(s_bits)
    zf = f16_bits_to_f32(z_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1.0) / sf
        t = (x - zf[..., None]).astype(np.float32) * inv[..., None]
        codes = np.clip(np.rint(t), 0, 3)
    codes = np.where((sf == 0)[..., None], 0, codes).astype(np.uint8)
    return codes, s_bits, z_bits


def dequantize(codes: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray) -> np.ndarray:
    """x_hat = z + code * s in fp64 (exact for these operands)."""
    s = f16_bits_to_f32(s_bits).astype(np.float64)
    z = f16_bits_to_f32(z_bits).astype(np.float64)
    return z[..., None] + codes.astype(np.float64) * s[..., None]


def dequantize_groups(codes: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray) -> np.ndarray:
    """x_hat = z_k + code * s_k on every channel of group k: codes [..., 128],
    s_bits / z_bits [..., 128 / group]."""
    ng = s_bits.shape[-1]
    gs = HEAD_DIM // ng
    s = np.repeat(f16_bits_to_f32(s_bits).astype(np.float64), gs, axis=-1)
    z = np.repeat(f16_bits_to_f32(z_bits).astype(np.float64), gs, axis=-1)
    return z + codes.astype(np.float64) * s


# --------------------------------------------------------------------------
# Online path, step 3: byte layout of one 16-token chunk (one KV head)
# --------------------------------------------------------------------------
# Four consecutive channels 4g..4g+3 of one token share a byte; channel 4g+k
# sits in bits 2k..2k+1.  K bytes are token-major; V bytes are grouped so that
# the eight bytes at 512 + 32*(g % 16) + 8*(t // 4) hold channel groups g and
# g + 16 of tokens 4*(t//4) .. 4*(t//4)+3.  Per-token (scale, zero) fp16 pairs.

def k_byte_offset(t: int, g: int) -> int:
    return K_CODES_OFF + 32 * t + g


def v_byte_offset(t: int, g: int) -> int:
    return V_CODES_OFF + 32 * (g & 15) + 8 * (t >> 2) + 4 * (g >> 4) + (t & 3)


def param_offset(kind: int, t: int, group: int = HEAD_DIM, k: int = 0) -> int:
    """(scale, zero) of quantization group k of slot t: kind 0 = K, 1 = V;
    bytes [off, off+2) scale, [off+2, off+4) zero (little endian).  With
    ng = 128 / group pairs per slot the K pairs fill [1024, 1024 + 64 ng) and
    the V pairs the next 64 ng bytes, slot-major (group 128: 1024 + 4 t and
    1088 + 4 t)."""
    ng = HEAD_DIM // group
    return K_CODES_OFF + 1024 + kind * 64 * ng + 4 * (t * ng + k)


def chunk_bytes(group: int = HEAD_DIM) -> int:
    """Bytes of one 16-token chunk: 1024 code bytes + 2 x 16 x (128 / group) x 4."""
    return 1024 + 128 * (HEAD_DIM // group)


_T = np.arange(CHUNK_TOKENS)[:, None]
_G = np.arange(HEAD_DIM // 4)[None, :]
K_BYTE_TABLE = (K_CODES_OFF + 32 * _T + _G).astype(np.int64)                       # [16][32]
V_BYTE_TABLE = (V_CODES_OFF + 32 * (_G & 15) + 8 * (_T >> 2) + 4 * (_G >> 4) + (_T & 3)).astype(np.int64)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., 128] codes in {0..3} -> [..., 32] bytes (channel 4g+k at bits 2k)."""
    c = codes.astype(np.uint8).reshape(codes.shape[:-1] + (HEAD_DIM // 4, 4))
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., 32] bytes -> [..., 128] codes."""
    p = packed.astype(np.uint8)
    out = np.stack([(p >> (2 * k)) & 3 for k in range(4)], axis=-1)
    return out.reshape(packed.shape[:-1] + (HEAD_DIM,)).astype(np.uint8)


# --------------------------------------------------------------------------
# The paged mixed-precision cache [OSCAR-S 2.2-B; OSCAR-N serving section]
# --------------------------------------------------------------------------

@dataclass
class Dims:
    n_q_heads: int
    n_kv_heads: int
    page_size: int
    n_sink: int
    n_recent: int
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    head_dim: int = HEAD_DIM
    quant_group: int = HEAD_DIM          # channels per (scale, zero) pair: 32, 64 or 128

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


class OracleCache:
    """Caller-visible state of the cache, byte for byte.

    pool   uint8 [num_pages][Hkv][P/16][chunk_bytes(quant_group)]  INT2 history
    sink   uint16 (bf16) [B][Hkv][n_sink][2][128]  rotated K (index 0) and V (1)
    recent uint16 (bf16) [B][Hkv][n_recent][2][128] ring: position pos lives in
           slot (pos - n_sink) mod n_recent
    block_table int32 [B][stride]: logical page pos // P -> physical page.

    Segments of a sequence of length L: sink [0, min(L, n_sink)), INT2
    [n_sink, max(n_sink, L - W)), recent [max(n_sink, L - W), L).
    """

    def __init__(self, dims: Dims, batch: int, num_pages: int, block_table: np.ndarray,
                 fill: int = 0):
        d = dims
        self.d = d
        self.batch = batch
        self.num_pages = num_pages
        self.block_table = np.asarray(block_table, dtype=np.int32)
        cpp = d.page_size // CHUNK_TOKENS
        self.pool = np.full((num_pages, d.n_kv_heads, cpp, chunk_bytes(d.quant_group)), fill,
                            np.uint8)
        self.sink = np.full((batch, d.n_kv_heads, max(d.n_sink, 0), 2, HEAD_DIM), fill * 0x0101, np.uint16)
        self.recent = np.full((batch, d.n_kv_heads, d.n_recent, 2, HEAD_DIM), fill * 0x0101, np.uint16)

    # -- chunk addressing --------------------------------------------------
    def _chunk_bases(self, b: int, h: int, positions: np.ndarray) -> np.ndarray:
        """Flat byte offset in `pool` of the chunk holding each position."""
        P = self.d.page_size
        cpp = P // CHUNK_TOKENS
        pages = self.block_table[b, positions // P].astype(np.int64)
        chunk_in_page = (positions % P) // CHUNK_TOKENS
        return ((pages * self.d.n_kv_heads + h) * cpp + chunk_in_page) * chunk_bytes(
            self.d.quant_group)

    def write_int2(self, b: int, h: int, kind: int, positions, r_bits: np.ndarray, clip: float):
        """Quantize rotated bf16 vectors r_bits [n][128] and store them at `positions`."""
        positions = np.asarray(positions, dtype=np.int64)
        if positions.size == 0:
            return
        gs = self.d.quant_group
        codes, s, z = quantize_groups(r_bits, clip, gs)              # s, z [n][ng]
        packed = pack_codes(codes)                                   # [n][32]
        base = self._chunk_bases(b, h, positions)                    # [n]
        t = positions % CHUNK_TOKENS
        table = K_BYTE_TABLE if kind == 0 else V_BYTE_TABLE
        flat = self.pool.reshape(-1)
        flat[base[:, None] + table[t]] = packed
        for k in range(HEAD_DIM // gs):
            off = base + np.array([param_offset(kind, int(tt), gs, k) for tt in t], np.int64)
            sb = s[:, k].astype(np.uint16)
            zb = z[:, k].astype(np.uint16)
            flat[off + 0] = (sb & 0xFF).astype(np.uint8)
            flat[off + 1] = (sb >> 8).astype(np.uint8)
            flat[off + 2] = (zb & 0xFF).astype(np.uint8)
            flat[off + 3] = (zb >> 8).astype(np.uint8)

    def read_int2(self, b: int, h: int, kind: int, positions) -> np.ndarray:
        """Dequantized fp64 vectors [n][128] of INT2 positions."""
        positions = np.asarray(positions, dtype=np.int64)
        base = self._chunk_bases(b, h, positions)
        t = positions % CHUNK_TOKENS
        table = K_BYTE_TABLE if kind == 0 else V_BYTE_TABLE
        flat = self.pool.reshape(-1)
        codes = unpack_codes(flat[base[:, None] + table[t]])
        gs = self.d.quant_group
        ng = HEAD_DIM // gs
        s = np.zeros((positions.size, ng), np.uint16)
        z = np.zeros((positions.size, ng), np.uint16)
        for k in range(ng):
            off = base + np.array([param_offset(kind, int(tt), gs, k) for tt in t], np.int64)
            s[:, k] = flat[off].astype(np.uint16) | (flat[off + 1].astype(np.uint16) << 8)
            z[:, k] = flat[off + 2].astype(np.uint16) | (flat[off + 3].astype(np.uint16) << 8)
        return dequantize_groups(codes, s, z)

    # -- append -------------------------------------------------------------
    def append(self, R_K, R_V, clip_K, clip_V, b: int, start: int,
               k_new: np.ndarray, v_new: np.ndarray):
        """Append L tokens (bf16 [L][Hkv][128]) to sequence b, whose length is `start`.

        First the ring tokens that fall out of the recent window are quantized
        from their stored bf16 values into INT2; then every new token is
        rotated and placed: sink, INT2 directly (if it is already older than
        the window at the end of this append), or the ring.
        """
        d = self.d
        L = k_new.shape[0]
        end = start + L
        W, ns = d.n_recent, d.n_sink
        R = (R_K, R_V)
        clip = (clip_K, clip_V)
        # 1. tokens that were in the ring before this append and leave the window
        evict = np.array([p for p in range(max(ns, start - W), start) if p < end - W], dtype=np.int64)
        if evict.size:
            slots = (evict - ns) % W
            for h in range(d.n_kv_heads):
                for kind in range(2):
                    self.write_int2(b, h, kind, evict, self.recent[b, h, slots, kind], clip[kind])
        # 2. new tokens
        pos = start + np.arange(L)
        to_sink = pos < ns
        to_int2 = (pos >= ns) & (pos < end - W)
        to_ring = (pos >= ns) & (pos >= end - W)
        for h in range(d.n_kv_heads):
            for kind, x in enumerate((k_new, v_new)):
                r = rotate(x[:, h, :], R[kind][h])                       # [L][128]
                if to_sink.any():
                    self.sink[b, h, pos[to_sink], kind] = r[to_sink]
                if to_int2.any():
                    self.write_int2(b, h, kind, pos[to_int2], r[to_int2], clip[kind])
                if to_ring.any():
                    self.recent[b, h, (pos[to_ring] - ns) % W, kind] = r[to_ring]

    # -- decode ---------------------------------------------------------------
    def gather(self, b: int, h: int, length: int) -> tuple[np.ndarray, np.ndarray]:
        """Dequantized rotated keys and values [length][128] fp64 of sequence b."""
        d = self.d
        ns, W = d.n_sink, d.n_recent
        K = np.zeros((length, HEAD_DIM))
        V = np.zeros((length, HEAD_DIM))
        n_sink_here = min(length, ns)
        for pos in range(n_sink_here):
            K[pos] = bf16_bits_to_f32(self.sink[b, h, pos, 0])
            V[pos] = bf16_bits_to_f32(self.sink[b, h, pos, 1])
        int2_end = max(ns, length - W)
        pos_int2 = np.arange(ns, int2_end)
        if pos_int2.size:
            K[ns:int2_end] = self.read_int2(b, h, 0, pos_int2)
            V[ns:int2_end] = self.read_int2(b, h, 1, pos_int2)
        for pos in range(max(ns, length - W), length):
            slot = (pos - ns) % W
            K[pos] = bf16_bits_to_f32(self.recent[b, h, slot, 0])
            V[pos] = bf16_bits_to_f32(self.recent[b, h, slot, 1])
        return K, V

    def decode(self, R_K, R_V, seq_len, q_bits: np.ndarray, heads=None) -> np.ndarray:
        """Decode attention for every sequence: out fp32 [B][Hq][128].

        q' = R_K^T q, logits = sm_scale * q' . k_hat', softmax, o' = sum p v_hat',
        o = R_V o' (fp64 throughout).  `heads` optionally restricts the work to
        a list of (b, kv_head) pairs (other rows are left as NaN).
        """
        d = self.d
        G = d.group
        out = np.full((self.batch, d.n_q_heads, HEAD_DIM), np.nan, np.float32)
        pairs = heads if heads is not None else [(b, h) for b in range(self.batch)
                                                  for h in range(d.n_kv_heads)]
        for b, h in pairs:
            K, V = self.gather(b, h, int(seq_len[b]))
            for g in range(h * G, (h + 1) * G):
                q = bf16_bits_to_f32(q_bits[b, g]).astype(np.float64)
                qr = np.asarray(R_K[h], np.float64).T @ q
                o_rot = attention(qr, K, V, d.sm_scale)
                out[b, g] = (np.asarray(R_V[h], np.float64) @ o_rot).astype(np.float32)
        return out


def decode_multi(cache: "OracleCache", R_K, R_V, seq_len, n_query: int,
                 q_bits: np.ndarray) -> np.ndarray:
    """Multi-query attention over the cache: out fp32 [B][M][Hq][128].

    The M = n_query queries of sequence b sit at its last M positions
    L - M .. L - 1 (their keys and values already appended, so the cache
    length L includes them; L >= M); query m attends causally to the stored
    keys and values of positions 0 .. L - M + m, dequantized as in decode; a
    query with no such position (L - M + m < 0, a sequence shorter than M)
    attends to nothing and gives 0, like the decode of an empty sequence.
    Speculative verification and chunked prefill over the INT2 cache
    [OSCAR-S 2.2-B: the same mixed-precision cache serves every query].
    q' = R_K^T q, softmax over the visible positions, o = R_V o' (fp64).
    """
    d = cache.d
    G = d.group
    B = cache.batch
    out = np.full((B, n_query, d.n_q_heads, HEAD_DIM), np.nan, np.float32)
    for b in range(B):
        L = int(seq_len[b])
        for h in range(d.n_kv_heads):
            K, V = cache.gather(b, h, L)
            for m in range(n_query):
                visible = max(0, L - n_query + m + 1)
                for g in range(h * G, (h + 1) * G):
                    q = bf16_bits_to_f32(q_bits[b, m, g]).astype(np.float64)
                    qr = np.asarray(R_K[h], np.float64).T @ q
                    o_rot = attention(qr, K[:visible], V[:visible], d.sm_scale)
                    out[b, m, g] = (np.asarray(R_V[h], np.float64) @ o_rot).astype(np.float32)
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Plain softmax attention of one query over [n][d] keys/values in fp64."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    logits = sm_scale * (K @ q)
    p = np.exp(logits - logits.max())
    return (p @ V) / p.sum()


def append_token_by_token(cache: OracleCache, R_K, R_V, clip_K, clip_V, b: int, start: int,
                          k_new: np.ndarray, v_new: np.ndarray):
    """The same append as `OracleCache.append`, one token per call."""
    for n in range(k_new.shape[0]):
        cache.append(R_K, R_V, clip_K, clip_V, b, start + n, k_new[n:n + 1], v_new[n:n + 1])


# --------------------------------------------------------------------------
# Byte accounting [OSCAR-S 4, memory; OSCAR-N serving section]
# --------------------------------------------------------------------------

def segment_counts(length: int, n_sink: int, n_recent: int) -> tuple[int, int, int]:
    """(#sink, #INT2, #recent) tokens of a sequence of the given length."""
    ns = min(length, n_sink)
    n_int2 = max(0, length - n_recent - n_sink)
    return ns, n_int2, length - ns - n_int2


def int2_bits_per_element() -> float:
    """2 code bits + two fp16 numbers per 128 channels = 2.25 bits."""
    return 2.0 + 32.0 / HEAD_DIM
