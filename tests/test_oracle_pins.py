"""Pins of the CPU oracle to things other than itself.

Each test ties one oracle function to a closed form, a library routine, a
hand-derived fixture, a brute-force evaluation or an invariant fixed by the
method's definition (OSCAR technical summary, sec. 2.2-A/B; tilnote OSCAR
note, attention-aware rotation).  A dropped term, a wrong sign, a transposed
operand or a wrong index anywhere in the oracle should fail one of these.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def bf16(x):
    """Test-side bf16 rounding through torch (independent of the oracle's)."""
    import torch
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- formats

def test_bf16_rounding_matches_torch():
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10 ** rng.uniform(-5, 5, 20000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.001953125])])
    assert np.array_equal(O.f32_to_bf16_bits(x), bf16(x))


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    assert O.f32_to_bf16_bits(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert O.f32_to_bf16_bits(np.float32(1 + 3 * 2 ** -8)) == 0x3F82


# ---------------------------------------------------------------- rotation parts

def test_hadamard_is_sylvester_from_scipy():
    H = O.hadamard(128)
    assert np.array_equal(H * math.sqrt(128), scipy.linalg.hadamard(128).astype(np.float64))
    S = np.rint(H * math.sqrt(128)).astype(np.int64)
    assert np.array_equal(S @ S.T, 128 * np.eye(128, dtype=np.int64))


def test_bitrev_against_string_reversal():
    for i in range(128):
        assert O.bitrev(i) == int(format(i, "07b")[::-1], 2)
    P = O.bitrev_permutation(128)
    assert np.array_equal(P, P.T)
    assert np.array_equal(P @ P, np.eye(128))
    assert P[1, 64] == 1 and P[3, 96] == 1 and P[5, 80] == 1


def test_eigenbasis_recovers_constructed_spectrum():
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    lam = np.linspace(5.0, 0.1, 128) + rng.uniform(0, 1e-3, 128)
    C = Q @ np.diag(lam) @ Q.T
    w, U = O.eigenbasis(C)
    assert np.all(np.diff(w) < 0)
    assert np.allclose(w, np.sort(lam)[::-1], atol=1e-12)
    # each column equals +-Q[:, j] of the same eigenvalue
    order = np.argsort(-lam)
    M = U.T @ Q[:, order]
    assert np.allclose(np.abs(np.diag(M)), 1.0, atol=1e-8)
    assert np.linalg.norm(C @ U - U @ np.diag(w)) <= 1e-10 * np.linalg.norm(C)


def test_eigen_order_and_sign_rule_on_diagonal():
    C = np.diag(np.arange(1.0, 129.0))
    w, U = O.eigenbasis(C)
    assert w[0] == 128.0 and w[-1] == 1.0
    # column 0 is e_127 with a positive entry, column 127 is e_0
    assert U[127, 0] == 1.0 and U[0, 127] == 1.0
    assert np.all(U >= 0)


def test_composite_rotation_orthogonal_and_hadamard_only_case():
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    R = O.composite_rotation(Q)
    assert np.abs(R.T @ R - np.eye(128)).max() < 1e-12
    R32 = R.astype(np.float32).astype(np.float64)
    assert np.abs(R32.T @ R32 - np.eye(128)).max() < 1e-6
    # U = I: R = H P, every entry +-1/sqrt(128): a unit vector is spread evenly
    RH = O.composite_rotation(np.eye(128))
    assert np.allclose(np.abs(RH), 1 / math.sqrt(128), atol=0)


def test_composite_rotation_with_identity_basis_is_hadamard_then_bitrev():
    """U = I: R = H P, so column j of R is column bitrev(j) of the Sylvester H."""
    Hs = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128)
    R = O.composite_rotation(np.eye(128))
    for j in range(128):
        assert np.array_equal(R[:, j], Hs[:, int(format(j, "07b")[::-1], 2)])


def test_rotation_direction_spreads_dominant_query_direction():
    """x' = R^T x puts a query along the top eigenvector of C_Q into eigen-
    coordinate 0, which the Hadamard then spreads evenly over all 128 channels
    (the stated purpose of H_Had).  With R x instead of R^T x this fails."""
    v = rng.standard_normal(128)
    v /= np.linalg.norm(v)
    N, G = 512, 2
    a = rng.standard_normal((N, G, 1)) * 4.0
    q = a * v + 0.01 * rng.standard_normal((N, G, 128))
    qb = bf16(q.astype(np.float32))
    C = O.query_covariance(O.bf16_bits_to_f32(qb).astype(np.float64))
    _, U = O.eigenbasis(C)
    R = O.composite_rotation(U).astype(np.float32)
    x = bf16((5.0 * v).astype(np.float32))
    r = O.bf16_bits_to_f32(O.rotate(x[None], R))[0].astype(np.float64)
    assert np.abs(np.abs(r) - 5.0 / math.sqrt(128)).max() < 0.02
    wrong = np.asarray(R, np.float64) @ O.bf16_bits_to_f32(x).astype(np.float64)
    assert np.abs(np.abs(wrong) - 5.0 / math.sqrt(128)).max() > 0.1


# ---------------------------------------------------------------- calibration statistics

def test_query_covariance_bruteforce():
    q = rng.standard_normal((7, 3, 128))
    C = O.query_covariance(q)
    B = np.zeros((128, 128))
    for n in range(7):
        for g in range(3):
            for i in range(128):
                B[i] += q[n, g, i] * q[n, g]
    assert np.allclose(C, B / 21, rtol=0, atol=1e-12)


def test_score_covariance_equals_VtStSV():
    """C_S = (1/N) V^T S^T S V with S built entry by entry (causal softmax)."""
    N, d = 9, 128
    q = rng.standard_normal((N, 2, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    sm = 1 / math.sqrt(d)
    C = O.score_covariance(q, k, v, sm)
    ref = np.zeros((d, d))
    for g in range(2):
        S = np.zeros((N, N))
        for n in range(N):
            e = [math.exp(sm * float(q[n, g] @ k[j])) for j in range(n + 1)]
            tot = sum(e)
            for j in range(n + 1):
                S[n, j] = e[j] / tot
        ref += v.T @ S.T @ S @ v
    assert np.allclose(C, ref / (N * 2), rtol=1e-10, atol=1e-12)


def test_nearest_rank_quantile():
    vals = np.arange(1, 1001, dtype=np.float32)[::-1]
    assert O.nearest_rank_quantile(vals, 0.999) == 999.0
    assert O.nearest_rank_quantile(vals, 1.0) == 1000.0
    assert O.nearest_rank_quantile(vals, 0.5) == 500.0
    assert O.nearest_rank_quantile(vals, 0.0) == 1.0


def test_calibrate_clip_p1_is_max_and_R_orthogonal():
    N, Hq, Hkv = 64, 4, 2
    q = bf16(rng.standard_normal((N, Hq, 128)).astype(np.float32))
    k = bf16(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * 3)
    v = bf16(rng.standard_normal((N, Hkv, 128)).astype(np.float32))
    cal = O.calibrate(q, k, v, Hq, Hkv, 1 / math.sqrt(128), clip_quantile=1.0)
    rk = np.stack([O.rotate(k[:, h], cal.R_K[h]) for h in range(Hkv)])
    assert cal.clip_K == float(np.abs(O.bf16_bits_to_f32(rk)).max())
    for R in (cal.R_K, cal.R_V):
        for h in range(Hkv):
            Rd = R[h].astype(np.float64)
            assert np.abs(Rd.T @ Rd - np.eye(128)).max() < 1e-6
    assert np.all(np.diff(cal.eig_Q, axis=1) <= 0)


def test_calibrate_wiring_closed_form():
    """R_K[h] = U_Q(h) H P and R_V[h] = U_S(h) H P, with U_Q from the pooled
    queries of KV head h's own query heads (h G .. h G + G - 1), U_S from the
    attention outputs of those queries over head h's keys and values, and
    one clip per tensor (p = 1: the largest |rotated value|), on data whose
    eigenbases are known in closed form (tests/calib_fixture.py)."""
    from calib_fixture import ClosedFormCalibration
    fx = ClosedFormCalibration(n_q_heads=4, n_kv_heads=2)
    cal = O.calibrate(fx.q, fx.k, fx.v, 4, 2, 1 / math.sqrt(128), clip_quantile=1.0)
    for h in range(2):
        assert np.abs(cal.R_K[h] - fx.R_K[h].astype(np.float32)).max() <= 1e-7, f"R_K[{h}]"
        assert np.abs(cal.R_V[h] - fx.R_V[h].astype(np.float32)).max() <= 1e-7, f"R_V[{h}]"
        assert np.allclose(cal.eig_Q[h], fx.eig_Q[h], rtol=1e-12, atol=0)
        assert np.allclose(cal.eig_S[h], fx.eig_S[h], rtol=1e-9, atol=0)
    assert cal.clip_K == fx.clip_K
    assert cal.clip_V == fx.clip_V
    assert fx.clip_K != fx.clip_V


def test_calibrate_wiring_eight_heads_per_kv_head():
    """The same closed form with G = 4 and three KV heads (query heads
    4h .. 4h + 3 belong to KV head h)."""
    from calib_fixture import ClosedFormCalibration
    fx = ClosedFormCalibration(n_q_heads=12, n_kv_heads=3, seed=7)
    cal = O.calibrate(fx.q, fx.k, fx.v, 12, 3, 1 / math.sqrt(128), clip_quantile=1.0)
    for h in range(3):
        assert np.abs(cal.R_K[h] - fx.R_K[h].astype(np.float32)).max() <= 1e-7, f"R_K[{h}]"
        assert np.abs(cal.R_V[h] - fx.R_V[h].astype(np.float32)).max() <= 1e-7, f"R_V[{h}]"
        assert np.allclose(cal.eig_Q[h], fx.eig_Q[h], rtol=1e-12, atol=0)
    assert (cal.clip_K, cal.clip_V) == (fx.clip_K, fx.clip_V)


# ---------------------------------------------------------------- pinned rotation

def test_rotate_identity_permutation_and_hadamard():
    x = bf16(rng.standard_normal((5, 128)).astype(np.float32))
    assert np.array_equal(O.rotate(x, np.eye(128, dtype=np.float32)), x)
    perm = rng.permutation(128)
    Pm = np.zeros((128, 128), np.float32)
    Pm[perm, np.arange(128)] = 1.0          # x'_i = x_perm[i]
    assert np.array_equal(O.rotate(x, Pm), x[:, perm])
    # e_j through the Hadamard: every entry bf16(+-fp32(1/sqrt(128)))
    Hf = O.hadamard(128).astype(np.float32)
    e = np.zeros((1, 128), np.float32)
    e[0, 7] = 1.0
    r = O.bf16_bits_to_f32(O.rotate(bf16(e), Hf))[0]
    mag = O.bf16_bits_to_f32(bf16(np.float32(1 / math.sqrt(128))))
    assert np.array_equal(np.abs(r), np.full(128, mag, np.float32))
    assert np.array_equal(np.sign(r), np.sign(Hf[7]))


def test_rotate_matches_exact_rational_within_one_ulp():
    """Against the correctly rounded exact dot product (Python fractions)."""
    R = np.linalg.qr(rng.standard_normal((128, 128)))[0].astype(np.float32)
    x = bf16(rng.standard_normal((6, 128)).astype(np.float32))
    got = O.bf16_bits_to_f32(O.rotate(x, R)).astype(np.float64)
    xf = O.bf16_bits_to_f32(x)
    same = 0
    for n in range(6):
        for i in range(128):
            s = sum(Fraction(float(xf[n, j])) * Fraction(float(R[j, i])) for j in range(128))
            exact = O.bf16_bits_to_f32(bf16(np.float32(float(s))))
            same += int(exact == got[n, i])
            ulp = 2.0 ** (math.floor(math.log2(abs(float(exact)))) - 7) if exact != 0 else 2 ** -133
            assert abs(got[n, i] - exact) <= ulp
    assert same >= 6 * 128 - 2


# ---------------------------------------------------------------- quantizer

def _golden_quantizer_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "quantizer_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, clip, pat, sbits, zbits, codes, err = [c.strip() for c in line.split("|")]
        cases.append((name, float(clip), [float(t) for t in pat.split()], int(sbits, 16),
                      int(zbits, 16), [int(c) for c in codes.split()], float(err)))
    return cases


@pytest.mark.parametrize("case", _golden_quantizer_cases(), ids=lambda c: c[0])
def test_quantizer_golden(case):
    name, clip, pat, sbits, zbits, cpat, maxerr = case
    r = np.array([pat[i % len(pat)] for i in range(128)], np.float32)
    codes, s, z = O.quantize(bf16(r)[None], clip)
    assert int(s[0]) == sbits and int(z[0]) == zbits
    assert list(codes[0]) == [cpat[i % len(cpat)] for i in range(128)]
    xc = np.clip(r, -clip, clip).astype(np.float64)
    assert np.abs(O.dequantize(codes, s, z)[0] - xc).max() == maxerr


def test_quantizer_error_bound_and_codes_range():
    r = bf16((rng.standard_normal((4000, 128)) * rng.uniform(0.01, 50, (4000, 1))).astype(np.float32))
    clip = 20.0
    codes, s, z = O.quantize(r, clip)
    assert codes.max() <= 3
    x = np.clip(O.bf16_bits_to_f32(r).astype(np.float64), -clip, clip)
    xh = O.dequantize(codes, s, z)
    sh = O.f16_bits_to_f32(s).astype(np.float64)[:, None]
    zh = O.f16_bits_to_f32(z).astype(np.float64)[:, None]
    mn = x.min(1, keepdims=True)
    sx = (x.max(1, keepdims=True) - mn) / 3
    inside = (x >= zh) & (x <= zh + 3 * sh)
    err = np.abs(x - xh)
    assert np.all(err[inside] <= (sh / 2 * (1 + 2 ** -18) + 0 * x)[inside])
    bound_out = sh / 2 + np.abs(mn - zh) + 3 * np.abs(sx - sh)
    assert np.all(err <= bound_out * (1 + 1e-6) + 0 * x)


# ---------------------------------------------------------------- packing and chunk layout

def test_pack_unpack_exhaustive_bytes():
    allb = np.arange(256, dtype=np.uint8)
    packed = np.tile(allb, 1)[: 256].reshape(8, 32)
    assert np.array_equal(O.pack_codes(O.unpack_codes(packed)), packed)
    codes = np.array([i % 4 for i in range(128)], np.uint8)
    assert np.all(O.pack_codes(codes) == 0xE4)
    one = np.zeros(128, np.uint8)
    one[5] = 2                                  # channel 5 -> byte 1, bits 2..3
    p = O.pack_codes(one)
    assert p[1] == 0x08 and p.sum() == 0x08


def test_chunk_layout_bijection_and_literals():
    k = O.K_BYTE_TABLE.ravel()
    v = O.V_BYTE_TABLE.ravel()
    assert sorted(k) == list(range(0, 512))
    assert sorted(v) == list(range(512, 1024))
    assert O.k_byte_offset(3, 5) == 101
    assert O.v_byte_offset(5, 17) == 512 + 32 * 1 + 8 * 1 + 4 * 1 + 1
    assert O.v_byte_offset(15, 31) == 512 + 32 * 15 + 8 * 3 + 4 + 3 == 1023
    offs = sorted(O.param_offset(kind, t) + j for kind in (0, 1) for t in range(16) for j in range(4))
    assert offs == list(range(1024, 1152))


# ---------------------------------------------------------------- cache and decode

def _rand_R(n):
    return np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(n)]).astype(np.float32)


def _tiny_setup(Hq=4, Hkv=2, P=16, ns=4, W=8, B=2, lens=(70, 45), fill=0):
    d = O.Dims(Hq, Hkv, P, ns, W)
    npages = [math.ceil(L / P) for L in lens]
    total = sum(npages) + 3
    perm = rng.permutation(total)
    bt = np.zeros((B, max(npages)), np.int32)
    i = 0
    for b, n in enumerate(npages):
        for p in range(n):
            bt[b, p] = perm[i]
            i += 1
    cache = O.OracleCache(d, B, total, bt, fill=fill)
    R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
    return d, cache, R_K, R_V


def test_bulk_append_equals_token_by_token():
    lens = (70, 45)
    d, c1, R_K, R_V = _tiny_setup(lens=lens)
    _, c2, _, _ = _tiny_setup(lens=lens)
    c2.block_table = c1.block_table.copy()
    c2.pool[:] = c1.pool
    for b, L in enumerate(lens):
        k = bf16(rng.standard_normal((L, 2, 128)).astype(np.float32) * 3)
        v = bf16(rng.standard_normal((L, 2, 128)).astype(np.float32))
        # c1: ragged bulk pieces (one longer than the window); c2: one token at a time
        cuts = [0, 3, 5, 30, 31, L]
        for a, e in zip(cuts[:-1], cuts[1:]):
            c1.append(R_K, R_V, 2.5, 2.0, b, a, k[a:e], v[a:e])
        O.append_token_by_token(c2, R_K, R_V, 2.5, 2.0, b, 0, k, v)
    assert np.array_equal(c1.pool, c2.pool)
    assert np.array_equal(c1.sink, c2.sink)
    assert np.array_equal(c1.recent, c2.recent)


def test_untouched_bytes_keep_sentinel():
    lens = (70, 45)
    d, c, R_K, R_V = _tiny_setup(lens=lens, fill=0xA5)
    for b, L in enumerate(lens):
        k = bf16(rng.standard_normal((L, 2, 128)).astype(np.float32))
        c.append(R_K, R_V, 3.0, 3.0, b, 0, k, k)
    flat = c.pool.reshape(c.num_pages, 2, -1)
    written = np.zeros(flat.shape, bool)
    for b, L in enumerate(lens):
        for pos in range(d.n_sink, L - d.n_recent):
            page = c.block_table[b, pos // 16]
            t = pos % 16
            for h in range(2):
                written[page, h, O.K_BYTE_TABLE[t]] = True
                written[page, h, O.V_BYTE_TABLE[t]] = True
                for kind in (0, 1):
                    o = O.param_offset(kind, t)
                    written[page, h, o:o + 4] = True
    assert np.all(flat[~written] == 0xA5)


def test_decode_matches_bruteforce_dense_attention():
    Hq, Hkv, P, ns, W = 4, 2, 16, 3, 8
    d = O.Dims(Hq, Hkv, P, ns, W)
    L = 61
    npg = math.ceil(L / P)
    bt = np.array([rng.permutation(npg + 2)[:npg]], np.int32)
    cache = O.OracleCache(d, 1, npg + 2, bt)
    R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
    cK, cV = 2.0, 1.5
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32) * 2)
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    cache.append(R_K, R_V, cK, cV, 0, 0, k[:20], v[:20])
    cache.append(R_K, R_V, cK, cV, 0, 20, k[20:], v[20:])
    q = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
    got = cache.decode(R_K, R_V, [L], q)
    G = Hq // Hkv
    for h in range(Hkv):
        keys, vals = [], []
        for pos in range(L):
            rk = O.rotate(k[pos, h][None], R_K[h])
            rv = O.rotate(v[pos, h][None], R_V[h])
            if ns <= pos < L - W:
                kc, ks, kz = O.quantize(rk, cK)
                vc, vs, vz = O.quantize(rv, cV)
                keys.append(O.dequantize(kc, ks, kz)[0])
                vals.append(O.dequantize(vc, vs, vz)[0])
            else:
                keys.append(O.bf16_bits_to_f32(rk[0]).astype(np.float64))
                vals.append(O.bf16_bits_to_f32(rv[0]).astype(np.float64))
        for g in range(h * G, (h + 1) * G):
            qv = O.bf16_bits_to_f32(q[0, g]).astype(np.float64)
            qr = [sum(float(R_K[h][j, i]) * qv[j] for j in range(128)) for i in range(128)]
            logits = [d.sm_scale * sum(qr[i] * keys[t][i] for i in range(128)) for t in range(L)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            orot = [sum(w[t] * vals[t][i] for t in range(L)) / sum(w) for i in range(128)]
            o = [sum(float(R_V[h][i, j]) * orot[j] for j in range(128)) for i in range(128)]
            assert np.allclose(got[0, g], np.array(o, np.float32), rtol=1e-5, atol=1e-6)


def test_rotation_invariance_fp64():
    """attn(q, K, V) = R_V attn(R_K^T q, R_K^T K, R_V^T V) (orthogonal R)."""
    Rk = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    Rv = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    q = rng.standard_normal(128)
    K = rng.standard_normal((50, 128)) * 2
    V = rng.standard_normal((50, 128))
    sm = 1 / math.sqrt(128)
    ref = O.attention(q, K, V, sm)
    rot = Rv @ O.attention(Rk.T @ q, K @ Rk, V @ Rv, sm)
    assert np.abs(ref - rot).max() < 1e-12


def test_all_bf16_cache_reduces_to_plain_attention():
    """len <= n_sink + W: no INT2; output equals unrotated attention up to bf16 rounding."""
    Hq, Hkv = 2, 1
    d = O.Dims(Hq, Hkv, 16, 4, 64)
    L = 60
    cache = O.OracleCache(d, 1, 4, np.zeros((1, 4), np.int32))
    cal_q = bf16(rng.standard_normal((64, Hq, 128)).astype(np.float32))
    cal_k = bf16(rng.standard_normal((64, Hkv, 128)).astype(np.float32))
    cal = O.calibrate(cal_q, cal_k, cal_k, Hq, Hkv, d.sm_scale)
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    cache.append(cal.R_K, cal.R_V, cal.clip_K, cal.clip_V, 0, 0, k, v)
    assert np.all(cache.pool == 0)
    q = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
    got = cache.decode(cal.R_K, cal.R_V, [L], q)
    for g in range(Hq):
        ref = O.attention(O.bf16_bits_to_f32(q[0, g]).astype(np.float64),
                          O.bf16_bits_to_f32(k[:, 0]).astype(np.float64),
                          O.bf16_bits_to_f32(v[:, 0]).astype(np.float64), d.sm_scale)
        e = np.abs(got[0, g] - ref).max() / np.abs(ref).max()
        assert e < 2e-2


def test_decode_invariant_under_page_permutation_and_G1_is_MHA():
    lens = (70,)
    for Hq, Hkv in ((4, 2), (2, 2)):
        d = O.Dims(Hq, Hkv, 16, 4, 8)
        k = bf16(rng.standard_normal((70, Hkv, 128)).astype(np.float32))
        v = bf16(rng.standard_normal((70, Hkv, 128)).astype(np.float32))
        q = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
        R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
        outs = []
        for perm in (np.arange(5), np.array([4, 0, 3, 1, 2])):
            c = O.OracleCache(d, 1, 5, perm[None, :].astype(np.int32))
            c.append(R_K, R_V, 3.0, 3.0, 0, 0, k, v)
            outs.append(c.decode(R_K, R_V, [70], q))
        assert np.array_equal(outs[0], outs[1])
        if Hq == Hkv:   # G = 1: head g reads KV head g only
            c2 = O.OracleCache(O.Dims(1, 1, 16, 4, 8), 1, 5, np.arange(5)[None].astype(np.int32))
            c2.append(R_K[1:2], R_V[1:2], 3.0, 3.0, 0, 0, k[:, 1:2], v[:, 1:2])
            single = c2.decode(R_K[1:2], R_V[1:2], [70], q[:, 1:2])
            assert np.array_equal(single[0, 0], outs[0][0, 1])


def test_segment_counts_and_bits_per_element():
    assert O.segment_counts(100000, 4, 256) == (4, 99740, 256)
    assert O.segment_counts(100, 4, 256) == (4, 0, 96)
    assert O.segment_counts(2, 4, 256) == (2, 0, 0)
    assert O.int2_bits_per_element() == 2.25
    # bytes per (token, KV head): 2 * (32 + 4) INT2 vs 2 * 256 bf16 -> 7.1x less
    assert 2 * 256 / (2 * (32 + 4)) == pytest.approx(7.111, rel=1e-3)


# ---------------------------------------------------------------- multi-query attention

def test_decode_multi_one_query_is_decode():
    d, oc, (R_K, R_V) = _multi_setup()
    q = bf16(rng.standard_normal((2, 1, 4, 128)).astype(np.float32))
    a = O.decode_multi(oc, R_K, R_V, [70, 45], 1, q)
    b = oc.decode(R_K, R_V, [70, 45], q[:, 0])
    assert np.array_equal(a[:, 0], b)


def _multi_setup(lens=(70, 45), W=8, ns=4):
    d = O.Dims(4, 2, 16, ns, W)
    npg = [math.ceil(L / 16) for L in lens]
    bt = np.zeros((len(lens), max(npg)), np.int32)
    perm = rng.permutation(sum(npg))
    i = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[i:i + n]
        i += n
    oc = O.OracleCache(d, len(lens), sum(npg), bt)
    R_K, R_V = _rand_R(2), _rand_R(2)
    for b, L in enumerate(lens):
        k = bf16(rng.standard_normal((L, 2, 128)).astype(np.float32) * 2)
        v = bf16(rng.standard_normal((L, 2, 128)).astype(np.float32))
        oc.append(R_K, R_V, 6.0, 6.0, b, 0, k, v)
    return d, oc, (R_K, R_V)


def test_decode_multi_bf16_cache_is_causal_sdpa():
    """With R = I and every position in bf16 (L <= n_sink + W), multi-query
    attention is scaled-dot-product attention with a bottom-right causal mask
    (torch, float64): query m of M sees the first L - M + m + 1 keys."""
    import torch
    Hq, Hkv, L, M, W, ns = 6, 2, 37, 5, 40, 4
    G = Hq // Hkv
    d = O.Dims(Hq, Hkv, 16, ns, W)
    npg = math.ceil(L / 16)
    oc = O.OracleCache(d, 1, npg, np.arange(npg, dtype=np.int32)[None])
    I = np.stack([np.eye(128, dtype=np.float32)] * Hkv)
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    oc.append(I, I, 8.0, 8.0, 0, 0, k, v)
    q = bf16(rng.standard_normal((1, M, Hq, 128)).astype(np.float32))
    got = O.decode_multi(oc, I, I, [L], M, q)[0]                         # [M][Hq][128]
    to64 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double()
    qt, kt, vt = to64(q[0]), to64(k), to64(v)                            # [M][Hq][d], [L][Hkv][d]
    mask = torch.zeros(M, L, dtype=torch.bool)
    for m in range(M):
        mask[m, :L - M + m + 1] = True
    for g in range(Hq):
        h = g // G
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[:, g][None, None], kt[:, h][None, None], vt[:, h][None, None], attn_mask=mask,
            scale=d.sm_scale)[0, 0]
        assert np.allclose(got[:, g], ref.numpy().astype(np.float32), rtol=0, atol=1e-6)


def test_decode_multi_rows_differ_only_by_visible_prefix():
    """Across the M queries the visible prefix grows by one position: giving
    every query the same vector, row m equals a one-query decode of a cache
    truncated to L - M + m + 1 positions when all of them are still bf16."""
    Hq, Hkv, L, M = 4, 2, 20, 4
    d = O.Dims(Hq, Hkv, 16, 4, 32)
    npg = math.ceil(L / 16)
    oc = O.OracleCache(d, 1, npg, np.arange(npg, dtype=np.int32)[None])
    R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    oc.append(R_K, R_V, 8.0, 8.0, 0, 0, k, v)
    q1 = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
    q = np.repeat(q1[:, None], M, axis=1)
    got = O.decode_multi(oc, R_K, R_V, [L], M, q)[0]
    for m in range(M):
        ref = oc.decode(R_K, R_V, [L - M + m + 1], q1)[0]
        assert np.allclose(got[m], ref, rtol=0, atol=1e-6), m


def test_decode_multi_sequence_shorter_than_the_queries():
    """L < M: query m sees positions 0 .. L - M + m, none when that is
    negative (output 0); the others equal the truncated one-query decodes."""
    Hq, Hkv, L, M = 4, 2, 2, 4
    d = O.Dims(Hq, Hkv, 16, 4, 8)
    oc = O.OracleCache(d, 1, 1, np.zeros((1, 1), np.int32))
    R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    oc.append(R_K, R_V, 8.0, 8.0, 0, 0, k, v)
    q1 = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
    got = O.decode_multi(oc, R_K, R_V, [L], M, np.repeat(q1[:, None], M, axis=1))[0]
    assert np.array_equal(got[0], np.zeros((Hq, 128), np.float32))
    assert np.array_equal(got[1], np.zeros((Hq, 128), np.float32))
    assert np.allclose(got[2], oc.decode(R_K, R_V, [1], q1)[0], rtol=0, atol=1e-6)
    assert np.allclose(got[3], oc.decode(R_K, R_V, [2], q1)[0], rtol=0, atol=1e-6)


# ---------------------------------------------------------------- quantization groups < 128

def test_block_hadamard_is_blockwise_sylvester():
    for blk in (32, 64, 128):
        H = O.hadamard_blocks(128, blk)
        assert np.abs(H @ H.T - np.eye(128)).max() < 1e-12
        ref = scipy.linalg.hadamard(blk) / math.sqrt(blk)
        for k in range(128 // blk):
            assert np.array_equal(H[k * blk:(k + 1) * blk, k * blk:(k + 1) * blk], ref)
        off = H.copy()
        for k in range(128 // blk):
            off[k * blk:(k + 1) * blk, k * blk:(k + 1) * blk] = 0
        assert not off.any()
    assert np.array_equal(O.hadamard_blocks(128, 128), O.hadamard(128))


def test_bitrev_spreads_one_hadamard_block_over_every_group():
    """U = I, Hadamard blocks of 32: x = e_j with j in the first block lights
    up H coordinates 0..31 only, and x' = R^T x = P H x puts coordinate
    y = bitrev7(i) at channel i, i.e. at the channels i = 0 mod 4 -- eight in
    each quantization group of 32, each of magnitude 1/sqrt(32)."""
    R = O.composite_rotation(np.eye(128), 32).astype(np.float32)
    e = np.zeros((1, 128), np.float32)
    e[0, 9] = 1.0
    r = O.bf16_bits_to_f32(O.rotate(bf16(e), R))[0]
    nz = np.flatnonzero(r)
    assert np.array_equal(nz, np.arange(0, 128, 4))
    mag = O.bf16_bits_to_f32(bf16(np.float32(1 / math.sqrt(32))))
    assert np.all(np.abs(r[nz]) == mag)
    for g in range(4):
        assert np.count_nonzero(r[32 * g:32 * (g + 1)]) == 8


def _golden_by_name():
    return {c[0]: c for c in _golden_quantizer_cases()}


@pytest.mark.parametrize("group,names", [
    (32, ("grid", "constant", "ties", "third")),
    (64, ("ties", "grid")),
    (32, ("negzero", "third", "constant", "grid")),
])
def test_quantizer_groups_are_independent_golden(group, names):
    """Each group of `group` channels holds one hand-derived case (all with the
    same clip): every group gets exactly that case's scale, zero and codes,
    so nothing leaks between groups."""
    gold = _golden_by_name()
    clip = 8.0 if "grid" not in names else 4.0
    parts = []
    for n in names:
        pat = np.resize(np.asarray(gold[n][2], np.float32), group)
        parts.append(pat)
    x = bf16(np.concatenate(parts)[None])
    codes, s, z = O.quantize_groups(x, clip, group)
    for k, n in enumerate(names):
        _, _, _, sbits, zbits, cpat, _ = gold[n]
        assert (int(s[0, k]), int(z[0, k])) == (sbits, zbits), (n, k)
        assert np.array_equal(codes[0, k * group:(k + 1) * group],
                              np.resize(np.asarray(cpat, np.uint8), group)), (n, k)


def test_quantizer_groups_128_is_quantize_and_bound_holds_per_group():
    x = bf16((rng.standard_normal((50, 128)) * rng.uniform(0.1, 5, (50, 1))).astype(np.float32))
    c1, s1, z1 = O.quantize(x, 6.0)
    c2, s2, z2 = O.quantize_groups(x, 6.0, 128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2[:, 0]) and np.array_equal(z1, z2[:, 0])
    for g in (32, 64):
        c, s, z = O.quantize_groups(x, 6.0, g)
        xh = O.dequantize_groups(c, s, z)
        xc = np.minimum(np.maximum(O.bf16_bits_to_f32(x).astype(np.float64), -6.0), 6.0)
        sh = np.repeat(O.f16_bits_to_f32(s).astype(np.float64), g, axis=-1)
        zh = np.repeat(O.f16_bits_to_f32(z).astype(np.float64), g, axis=-1)
        inside = (xc >= zh) & (xc <= zh + 3 * sh)
        assert np.all(np.abs(xc - xh)[inside] <= (sh / 2 * (1 + 2 ** -18))[inside])
        # finer groups never quantize worse than the whole vector on average
        err_g = np.abs(xc - xh).mean()
        err_128 = np.abs(xc - O.dequantize(c1, s1, z1)).mean()
        assert err_g <= err_128


def test_group_chunk_layout_covers_the_chunk_once():
    for g in (32, 64, 128):
        ng = 128 // g
        cb = O.chunk_bytes(g)
        assert cb == 1024 + 128 * ng
        offs = sorted(O.param_offset(kind, t, g, k) + j for kind in (0, 1) for t in range(16)
                      for k in range(ng) for j in range(4))
        assert offs == list(range(1024, cb))
    assert O.param_offset(0, 3) == 1024 + 12 and O.param_offset(1, 3) == 1088 + 12
    # slot-major pairs: slot t's ng pairs are contiguous (literal layout)
    assert O.param_offset(0, 3, 32, 2) == 1024 + 4 * (3 * 4 + 2)
    assert O.param_offset(1, 15, 32, 3) == 1024 + 256 + 4 * (15 * 4 + 3) == 1532
    assert O.param_offset(1, 1, 64, 1) == 1024 + 128 + 4 * 3


@pytest.mark.parametrize("group", [32, 64])
def test_group_cache_decode_is_dense_attention_over_groupwise_dequantized(group):
    """Bulk == token-by-token bytes with quantization groups, and decode equal
    to dense attention over K/V dequantized group by group straight from
    quantize_groups of the rotated tokens (no cache involved)."""
    Hq, Hkv, P, ns, W, L = 4, 2, 16, 4, 8, 90
    d = O.Dims(Hq, Hkv, P, ns, W, quant_group=group)
    npg = math.ceil(L / P)
    bt = rng.permutation(npg).astype(np.int32)[None]
    R_K, R_V = _rand_R(Hkv), _rand_R(Hkv)
    k = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32) * 2)
    v = bf16(rng.standard_normal((L, Hkv, 128)).astype(np.float32))
    c1 = O.OracleCache(d, 1, npg, bt)
    c2 = O.OracleCache(d, 1, npg, bt)
    c1.append(R_K, R_V, 5.0, 5.0, 0, 0, k, v)
    O.append_token_by_token(c2, R_K, R_V, 5.0, 5.0, 0, 0, k, v)
    assert np.array_equal(c1.pool, c2.pool) and np.array_equal(c1.recent, c2.recent)
    q = bf16(rng.standard_normal((1, Hq, 128)).astype(np.float32))
    got = c1.decode(R_K, R_V, [L], q)[0]
    G = Hq // Hkv
    for h in range(Hkv):
        Kr = np.zeros((L, 128))
        Vr = np.zeros((L, 128))
        for pos in range(L):
            rk, rv = O.rotate(k[pos:pos + 1, h], R_K[h]), O.rotate(v[pos:pos + 1, h], R_V[h])
            if ns <= pos < L - W:
                Kr[pos] = O.dequantize_groups(*O.quantize_groups(rk, 5.0, group))[0]
                Vr[pos] = O.dequantize_groups(*O.quantize_groups(rv, 5.0, group))[0]
            else:
                Kr[pos], Vr[pos] = O.bf16_bits_to_f32(rk)[0], O.bf16_bits_to_f32(rv)[0]
        for g in range(h * G, (h + 1) * G):
            qr = R_K[h].astype(np.float64).T @ O.bf16_bits_to_f32(q[0, g]).astype(np.float64)
            lg = d.sm_scale * (Kr @ qr)
            p = np.exp(lg - lg.max())
            ref = R_V[h].astype(np.float64) @ ((p @ Vr) / p.sum())
            assert np.allclose(got[g], ref, rtol=0, atol=1e-5)


def test_calibrate_block_hadamard_closed_form():
    from calib_fixture import ClosedFormCalibration
    fx = ClosedFormCalibration(n_q_heads=4, n_kv_heads=2, hadamard_block=32)
    cal = O.calibrate(fx.q, fx.k, fx.v, 4, 2, 1 / math.sqrt(128), clip_quantile=1.0,
                      hadamard_block=32)
    for h in range(2):
        assert np.abs(cal.R_K[h] - fx.R_K[h].astype(np.float32)).max() <= 1e-7
        assert np.abs(cal.R_V[h] - fx.R_V[h].astype(np.float32)).max() <= 1e-7
    assert (cal.clip_K, cal.clip_V) == (fx.clip_K, fx.clip_V)
