"""Pins of the HQMQ oracle (oracle/hqmq_oracle.py) against facts that the
page and the mathematics fix, not against the oracle's own formulas:
quaternion algebra (i j = k, norm multiplicativity, associativity), the
binary tetrahedral group (closure, 60-degree neighbours, the 24-cell's
45-degree covering radius), the product order q_p q_s, hand-derived
radius codes and Med3x decisions, and decode attention on a cache that
encodes exactly, against torch's scaled-dot-product attention.

Source: "Technical summary: Hurwitz quaternion multiplicative quantization
for KV cache compression" (gist.science 2605.27646), Method sections 1-3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import hqmq_oracle as H
from oracle.kvq_oracle import bf16_bits_to_f32, f32_to_bf16_bits
from long_context_decode_kvq_amd.workloads import hqmq_secondary

ONE = np.array([1.0, 0, 0, 0])
I_ = np.array([0, 1.0, 0, 0])
J_ = np.array([0, 0, 1.0, 0])
K_ = np.array([0, 0, 0, 1.0])


# ------------------------------------------------------------ quaternions

def test_hamilton_units():
    """i^2 = j^2 = k^2 = ijk = -1 and the cyclic products."""
    for u in (I_, J_, K_):
        assert np.array_equal(H.hamilton(u, u), -ONE)
    assert np.array_equal(H.hamilton(H.hamilton(I_, J_), K_), -ONE)
    assert np.array_equal(H.hamilton(I_, J_), K_)
    assert np.array_equal(H.hamilton(J_, K_), I_)
    assert np.array_equal(H.hamilton(K_, I_), J_)
    assert np.array_equal(H.hamilton(J_, I_), -K_)
    assert np.array_equal(H.hamilton(K_, J_), -I_)
    assert np.array_equal(H.hamilton(I_, K_), -J_)
    assert np.array_equal(H.hamilton(ONE, I_), I_)


def test_hamilton_norm_multiplicative_and_associative():
    rng = np.random.default_rng(0)
    for _ in range(50):
        p, q, r = rng.standard_normal((3, 4))
        pq = H.hamilton(p, q)
        assert abs(np.linalg.norm(pq) - np.linalg.norm(p) * np.linalg.norm(q)) < 1e-12
        assert np.allclose(H.hamilton(pq, r), H.hamilton(p, H.hamilton(q, r)), atol=1e-12)
        # conjugation reverses the order: conj(pq) = conj(q) conj(p)
        cj = lambda x: x * np.array([1, -1, -1, -1])
        assert np.allclose(cj(pq), H.hamilton(cj(q), cj(p)), atol=1e-12)


# ---------------------------------------------- binary tetrahedral group

def test_binary_tetrahedral_enumeration():
    P = H.binary_tetrahedral()
    assert P.shape == (24, 4)
    assert np.array_equal(P[0], ONE) and np.array_equal(P[1], -ONE)
    assert np.array_equal(P[2], I_) and np.array_equal(P[3], -I_)
    assert np.array_equal(P[4], J_) and np.array_equal(P[7], -K_)
    assert np.array_equal(P[8], [0.5, 0.5, 0.5, 0.5])
    assert np.array_equal(P[8 + 0b0101], [-0.5, 0.5, -0.5, 0.5])
    assert np.array_equal(P[23], [-0.5, -0.5, -0.5, -0.5])
    assert len({tuple(x) for x in P}) == 24
    assert np.allclose(np.linalg.norm(P, axis=1), 1.0)


def test_binary_tetrahedral_is_a_group_with_60_degree_neighbours():
    P = H.binary_tetrahedral()
    members = {tuple(x) for x in P}
    for a in P:
        for b in P:
            assert tuple(H.hamilton(a, b)) in members            # closed (exact arithmetic)
        assert tuple(a * np.array([1, -1, -1, -1])) in members   # inverses
    G = P @ P.T
    for i in range(24):
        others = np.delete(G[i], i)
        assert others.max() == 0.5                               # nearest at 60 degrees
        assert np.sum(others == 0.5) == 8                        # 24-cell: 8 neighbours


def test_covering_radius_of_the_24_cell_is_45_degrees():
    """Every unit direction lies within 45 degrees of a vertex of the 24-cell
    and the deep holes (the dual 24-cell) sit at exactly 45 degrees."""
    P = H.binary_tetrahedral()
    rng = np.random.default_rng(1)
    u = rng.standard_normal((20000, 4))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    assert (u @ P.T).max(axis=1).min() >= 1 / math.sqrt(2) - 1e-12
    hole = np.array([1.0, 1.0, 0, 0]) / math.sqrt(2)
    assert abs((P @ hole).max() - 1 / math.sqrt(2)) < 1e-15


# -------------------------------------------------------------- codebook

def test_codebook_product_order_is_primary_times_secondary():
    """With q_s = i: word p = q_p i, so +j gives j i = -k (not i j = +k)."""
    cb = H.codebook(np.array([[0, 1, 0, 0]], np.float32))
    assert np.array_equal(cb[4], [0, 0, 0, -1])                  # (+j) i = -k
    assert np.array_equal(cb[2], [-1, 0, 0, 0])                  # i i = -1
    assert np.array_equal(cb[6], [0, 0, 1, 0])                   # k i = j
    # identity secondary: the codebook is 2T itself, word 24 s + p
    cb2 = H.codebook(np.array([[0, 1, 0, 0], [1, 0, 0, 0]], np.float32))
    assert np.array_equal(cb2[24:], H.binary_tetrahedral().astype(np.float32))


def test_codebook_is_24_rotated_copies_of_the_24_cell():
    """Right multiplication by a unit quaternion is an isometry: each block
    of 24 words has the Gram matrix of 2T and unit norms."""
    sec = hqmq_secondary(3, 1, 10)[0, 0]
    cb = H.codebook(sec).astype(np.float64)
    assert cb.shape == (240, 4)
    P = H.binary_tetrahedral()
    for s in range(10):
        blk = cb[24 * s:24 * s + 24]
        assert np.abs(blk @ blk.T - P @ P.T).max() < 1e-6
    assert np.abs(np.linalg.norm(cb, axis=1) - 1).max() < 1e-6


# -------------------------------------------------------------- encoding

def test_chunk_norms_closed_form():
    x = np.zeros(128, np.float32)
    x[0:4] = [3, 4, 0, 0]
    x[4:8] = [1, 1, 1, 1]
    x[8:12] = [0, 0, -6, 8]
    r = H.chunk_norms(x)
    assert r[0] == 5 and r[1] == 2 and r[2] == 10 and r[3] == 0


def test_lower_median():
    assert H.lower_median(np.array([4, 1, 3, 2], np.float32)) == 2        # not 2.5
    assert H.lower_median(np.array([5, 1, 3], np.float32)) == 3
    v = np.random.default_rng(2).random(1001).astype(np.float32)
    assert H.lower_median(v) == np.median(v)                               # odd n
    assert H.outlier_threshold(np.array([1, 2, 3], np.float32)) == 6


def _bf16(x):
    b = f32_to_bf16_bits(np.asarray(x, np.float32))
    assert np.array_equal(bf16_bits_to_f32(b), np.asarray(x, np.float32))
    return b


def test_record_of_a_hand_derived_vector():
    """Radii 4, 2, 1, 1/2 along +1: r_max = 4, codes rint(r 255/4) = 255,
    rint(127.5) = 128 (tie to even), rint(63.75) = 64, rint(31.875) = 32;
    every direction is the word +1 (index 0 with the identity secondary),
    a chunk along -i is word 3, along (1/2)(1,1,1,1) word 8."""
    cb = H.codebook(np.array([[1, 0, 0, 0]], np.float32))
    x = np.zeros(128, np.float32)
    x[0:4] = [4, 0, 0, 0]
    x[4:8] = [2, 0, 0, 0]
    x[8:12] = [1, 0, 0, 0]
    x[12:16] = [0.5, 0, 0, 0]
    x[16:20] = [0, -1, 0, 0]
    x[20:24] = [0.5, 0.5, 0.5, 0.5]
    rec = H.encode_record(_bf16(x), cb, np.float32(100.0))
    assert list(rec[H.RAD_OFF:H.RAD_OFF + 6]) == [255, 128, 64, 32, 64, 64]
    assert list(rec[H.IDX_OFF:H.IDX_OFF + 6]) == [0, 0, 0, 0, 3, 8]
    assert not rec[H.IDX_OFF + 6:H.IDX_OFF + 32].any()                     # zero chunks
    assert not rec[H.RAD_OFF + 6:H.RAD_OFF + 32].any()
    assert rec[H.RMAX_OFF:H.RMAX_OFF + 2].view(np.uint16)[0] == 0x4400     # fp16 4.0
    assert rec[H.FLAGS_OFF:].view(np.uint8).sum() == 0


def test_med3x_outliers_and_capacity():
    """Candidates are chunks with r > thr (strict); with four candidates of
    radii 10, 20, 30, 20 the three largest stay fp16 (the tie keeps the
    lower chunk index) and the fourth is coded."""
    cb = H.codebook(np.array([[1, 0, 0, 0]], np.float32))
    x = np.zeros(128, np.float32)
    x[4 * 1] = 10
    x[4 * 5] = 20
    x[4 * 9 + 2] = -30
    x[4 * 12 + 3] = 20
    x[4 * 20] = 6        # r = thr exactly: not a candidate
    rec = H.encode_record(_bf16(x), cb, np.float32(6.0))
    flags = int(rec[H.FLAGS_OFF:H.FLAGS_OFF + 4].view(np.uint32)[0])
    assert flags == (1 << 5) | (1 << 9) | (1 << 12)
    slots = rec[H.OUT_OFF:H.OUT_OFF + 24].view(np.uint16).view(np.float16).astype(np.float32)
    assert np.array_equal(slots, [20, 0, 0, 0, 0, 0, -30, 0, 0, 0, 0, 20])
    # coded chunks: r_max = 10 (chunk 1), chunk 20 has r = 6 -> rint(153) = 153
    assert rec[H.RAD_OFF + 1] == 255 and rec[H.RAD_OFF + 20] == 153
    assert rec[H.RAD_OFF + 5] == 0 and rec[H.IDX_OFF + 9] == 0             # fp16 chunks: 0
    d = H.decode_record(rec, cb)
    assert d[20] == 20 and d[38] == -30 and d[51] == 20                    # kept exactly
    assert d[4] == 10 and abs(d[80] - 153 * 10 / 255) < 1e-12
    # a tie at the capacity cut: radii 20, 20, 30, 20 keep 30 and the two
    # lower-index 20s
    y = np.zeros(128, np.float32)
    y[4 * 1] = y[4 * 5] = y[4 * 12 + 3] = 20
    y[4 * 9 + 2] = -30
    rec = H.encode_record(_bf16(y), cb, np.float32(6.0))
    assert int(rec[H.FLAGS_OFF:H.FLAGS_OFF + 4].view(np.uint32)[0]) == (1 << 1) | (1 << 5) | (1 << 9)
    assert rec[H.RAD_OFF + 12] == 255
    # a chunk with r equal to the threshold and no other candidate: coded
    z = np.zeros(128, np.float32)
    z[4 * 3 + 1] = 6
    z[4 * 7] = 2
    rec = H.encode_record(_bf16(z), cb, np.float32(6.0))
    assert int(rec[H.FLAGS_OFF:H.FLAGS_OFF + 4].view(np.uint32)[0]) == 0
    assert rec[H.RAD_OFF + 3] == 255 and rec[H.IDX_OFF + 3] == 2           # +i


def test_radius_code_uses_the_stored_fp16_r_max():
    """r_max = fp32 sqrt(2) is stored as fp16 1.4140625 (0x3DA8); a chunk of
    radius 0.224609375 codes as rint(0.224609375 * fp32(255 / 1.4140625)) =
    rint(40.504) = 41 (against the unrounded r_max it would be 40)."""
    cb = H.codebook(np.array([[1, 0, 0, 0]], np.float32))
    x = np.zeros(128, np.float32)
    x[0:2] = [1, 1]
    x[4] = 0.224609375
    rec = H.encode_record(_bf16(x), cb, np.float32(100.0))
    assert rec[H.RMAX_OFF:H.RMAX_OFF + 2].view(np.uint16)[0] == 0x3DA8
    assert rec[H.RAD_OFF] == 255 and rec[H.RAD_OFF + 1] == 41


def test_encoder_direction_is_the_best_word():
    """u equal to a word (power-of-two radius) gives that word; random
    directions get a word within fp32 rounding of the fp64 best, and within
    the covering bound."""
    sec = hqmq_secondary(4, 1, 3)[0, 0]
    cb = H.codebook(sec)
    for w in (0, 5, 30, 71):
        x = np.float32(2.0) * cb[w]
        assert H.direction_index(x / np.float32(2.0), cb) == w
    rng = np.random.default_rng(5)
    cb64 = cb.astype(np.float64)
    for _ in range(2000):
        u = rng.standard_normal(4).astype(np.float32)
        u = (u / np.float32(np.linalg.norm(u))).astype(np.float32)
        w = H.direction_index(u, cb)
        sc = cb64 @ u.astype(np.float64)
        assert sc[w] >= sc.max() - 1e-6
        assert sc[w] >= 1 / math.sqrt(2) - 1e-6


def test_coded_chunk_error_bound():
    """|x_hat - x| <= r_max / 510 + r sqrt(2 - 2 <u, c>) per coded chunk,
    with <u, c> >= cos 45 degrees."""
    sec = hqmq_secondary(6, 1, 10)[0, 0]
    cb = H.codebook(sec)
    rng = np.random.default_rng(7)
    for _ in range(30):
        xb = f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
        x = bf16_bits_to_f32(xb).astype(np.float64)
        rec = H.encode_record(xb, cb, np.float32(1e9))
        d = H.decode_record(rec, cb)
        r = H.chunk_norms(x.astype(np.float32)).astype(np.float64)
        r_max = float(np.float16(r.max()))
        for j in range(32):
            err = np.linalg.norm(d[4 * j:4 * j + 4] - x[4 * j:4 * j + 4])
            bound = r_max / 510 * 1.001 + r[j] * math.sqrt(2 - 2 / math.sqrt(2)) + 1e-6
            assert err <= bound


# ---------------------------------------------------------------- decode

def _exact_vectors(rng, n, Hkv, P):
    """bf16 vectors that HQMQ codes exactly: every chunk is r c for a word c
    of 2T (identity secondary) with one power-of-two r per vector, so the
    record has r_max = r and code 255 everywhere."""
    Pq = P.astype(np.float32)
    words = rng.integers(0, 24, size=(n, Hkv, 32))
    r = np.float32(2.0) ** rng.integers(-2, 3, size=(n, Hkv, 1, 1)).astype(np.float32)
    x = (Pq[words] * r).reshape(n, Hkv, 128).astype(np.float32)
    return _bf16(x)


@pytest.mark.parametrize("Hq,Hkv,P", [(4, 2, 16), (2, 2, 32)])
def test_decode_on_an_exact_cache_is_plain_attention(Hq, Hkv, P):
    rng = np.random.default_rng(8)
    d = H.HqmqDims(Hq, Hkv, P, 1)
    lens = [37, 5]
    npg = [-(-L // P) for L in lens]
    bt = np.full((2, max(npg)), -1, np.int32)
    perm = rng.permutation(sum(npg))
    bt[0, :npg[0]] = perm[:npg[0]]
    bt[1, :npg[1]] = perm[npg[0]:]
    ident = np.tile(np.array([1, 0, 0, 0], np.float32), (2, Hkv, 1, 1))
    cbs = np.stack([np.stack([H.codebook(ident[r, h]) for h in range(Hkv)]) for r in range(2)])
    cache = H.HqmqCache(d, 2, sum(npg), bt, cbs, fill=0xA5)
    P2 = H.binary_tetrahedral()
    ks = [_exact_vectors(rng, L, Hkv, P2) for L in lens]
    vs = [_exact_vectors(rng, L, Hkv, P2) for L in lens]
    cache.append([0, 0], [k[:20] for k in ks], [v[:20] for v in vs])
    cache.append([20, min(20, lens[1])], [k[20:] for k in ks], [v[20:] for v in vs])
    q = f32_to_bf16_bits(rng.standard_normal((2, Hq, 128)).astype(np.float32))
    out = cache.decode(lens, q)
    for b, L in enumerate(lens):
        K = torch.from_numpy(bf16_bits_to_f32(ks[b]).astype(np.float64))     # [L][Hkv][128]
        V = torch.from_numpy(bf16_bits_to_f32(vs[b]).astype(np.float64))
        Q = torch.from_numpy(bf16_bits_to_f32(q[b]).astype(np.float64))      # [Hq][128]
        G = Hq // Hkv
        Kx = K.permute(1, 0, 2).repeat_interleave(G, 0)                      # [Hq][L][128]
        Vx = V.permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[:, None, :], Kx, Vx, scale=1 / math.sqrt(128))[:, 0]
        assert np.abs(out[b] - ref.numpy()).max() <= 1e-5 * max(1.0, np.abs(ref.numpy()).max())


def test_decode_uniform_keys_average_the_values():
    """Equal keys give equal weights: the output is the mean of the decoded
    values, whatever the query."""
    rng = np.random.default_rng(9)
    d = H.HqmqDims(2, 1, 16, 2)
    sec = hqmq_secondary(10, 1, 2)
    cbs = np.stack([np.stack([H.codebook(sec[r, 0])]) for r in range(2)])
    bt = np.array([[1, 0]], np.int32)
    cache = H.HqmqCache(d, 1, 2, bt, cbs)
    L = 23
    k = np.tile(f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32)), (L, 1, 1))
    v = f32_to_bf16_bits(rng.standard_normal((L, 1, 128)).astype(np.float32))
    cache.append([0], [k], [v])
    q = f32_to_bf16_bits(rng.standard_normal((1, 2, 128)).astype(np.float32))
    out = cache.decode([L], q)
    _, V = cache.decoded(0, L, 0)
    assert np.abs(out[0, 0] - V.mean(0)).max() < 1e-6
    assert np.abs(out[0, 1] - V.mean(0)).max() < 1e-6


def test_append_median_spans_the_whole_call():
    """The Med3x median is taken over every chunk of a role in one call: a
    chunk that is an outlier against a call of small vectors is coded when
    appended with large ones."""
    d = H.HqmqDims(1, 1, 16, 1)
    cbs = np.stack([np.stack([H.codebook(np.array([[1, 0, 0, 0]], np.float32))])] * 2)
    small = np.zeros((1, 1, 128), np.float32)
    small[..., :] = 1.0                                  # every chunk r = 2
    big = np.full((1, 1, 128), 8.0, np.float32)          # every chunk r = 16
    mixed = small.copy()
    mixed[0, 0, :4] = 8.0                                # chunk 0 r = 16 > 3 * 2
    bt = np.array([[0]], np.int32)
    c1 = H.HqmqCache(d, 1, 1, bt, cbs)
    c1.append([0], [_bf16(mixed)], [_bf16(mixed)])
    assert int(c1.record(0, 0, 0, 0)[H.FLAGS_OFF]) == 1
    c2 = H.HqmqCache(d, 1, 1, np.array([[0]], np.int32), cbs)
    c2.append([0], [_bf16(np.concatenate([mixed, big, big]))],
              [_bf16(np.concatenate([mixed, big, big]))])
    assert int(c2.record(0, 0, 0, 0)[H.FLAGS_OFF]) == 0   # median 16: no outlier


def test_bits_per_element():
    assert H.bits_per_element() == 6.0
