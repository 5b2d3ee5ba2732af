"""CPU tests of the libkvq2 boundary: the library loads, exports every symbol
declared in include/kvq2.h, rejects bad arguments before any HIP call, and its
host calibration agrees with the oracle's (no GPU needed)."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle as O
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import to_bf16_bits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ERR_ARG, ERR_UNSUP, ERR_WS, ERR_NUM = -1, -2, -3, -4


def _lib():
    if not os.path.exists(kvq2._LIB_PATH):
        pytest.fail("libkvq2.so is not built: run python -m long_context_decode_kvq_amd.build")
    return kvq2.lib()


def test_exports_every_declared_symbol():
    L = _lib()
    header = open(os.path.join(ROOT, "include", "kvq2.h")).read()
    names = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(kvq_\w+)\s*\(", header, re.M))
    assert names == set(kvq2.EXPORTS)
    probe = open(os.path.join(ROOT, "include", "kvq2_probe.h")).read()
    pnames = set(re.findall(r"^\s*int\s+(kvq_\w+)\s*\(", probe, re.M))
    assert pnames == set(kvq2.PROBE_EXPORTS)
    for n in kvq2.PROBE_EXPORTS:
        assert hasattr(L, n)
    for n in names:
        assert hasattr(L, n), n
    assert L.kvq_status_string(0) == b"KVQ_OK"
    for rc in (ERR_ARG, ERR_UNSUP, ERR_WS, ERR_NUM, -5):
        assert L.kvq_status_string(rc).startswith(b"KVQ_ERR_")


# Fake but 16-byte-aligned device addresses: validation must reject the call
# before anything dereferences them or touches HIP.
FAKE = 0x7F0000000000


def _args(**over):
    d = kvq2.dims(over.pop("Hq", 32), over.pop("Hkv", 8), over.pop("P", 16), over.pop("ns", 4),
                  over.pop("W", 256))
    for k in list(over):
        if hasattr(d, k):
            setattr(d, k, over.pop(k))
    lay = kvq2.KvqLayer(FAKE, FAKE + 0x100000, over.pop("clip_K", 4.0), over.pop("clip_V", 4.0))
    cch = kvq2.KvqCache(FAKE + 0x200000, 100, FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000,
                        over.pop("bt_stride", 8))
    return d, lay, cch


def _decode(d, lay, cch, batch=2, seq=FAKE, max_len=100, q=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30):
    return _lib().kvq_decode_attention(C.byref(d), C.byref(lay), C.byref(cch), batch, seq, max_len,
                                       q, out, ws, wsb, None)


def _append(d, lay, cch, batch=2, sp=FAKE, cu=FAKE, total=4, mx=2, k=FAKE, v=FAKE):
    return _lib().kvq_quantize_append(C.byref(d), C.byref(lay), C.byref(cch), batch, sp, cu, total,
                                      mx, k, v, None)


def _step(d, lay, cch, batch=2, sp=FAKE, cu=FAKE, total=4, mx=2, k=FAKE, v=FAKE, seq=FAKE,
          max_len=100, q=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30):
    return _lib().kvq_decode_step(C.byref(d), C.byref(lay), C.byref(cch), batch, sp, cu, total, mx,
                                  k, v, seq, max_len, q, out, ws, wsb, None)


@pytest.mark.parametrize("over,rc", [
    (dict(head_dim=64), ERR_UNSUP),
    (dict(P=8), ERR_UNSUP),
    (dict(P=128), ERR_UNSUP),
    (dict(Hq=34, Hkv=8), ERR_ARG),
    (dict(Hq=34, Hkv=2), ERR_UNSUP),          # group 17 > 16
    (dict(ns=-1), ERR_ARG),
    (dict(W=0), ERR_ARG),
    (dict(clip_K=0.0), ERR_ARG),
    (dict(clip_V=16385.0), ERR_ARG),
    (dict(clip_K=float("nan")), ERR_ARG),
    (dict(bt_stride=0), ERR_ARG),
    (dict(quant_group=16), ERR_UNSUP),
    (dict(quant_group=96), ERR_UNSUP),
    (dict(hadamard_block=8), ERR_UNSUP),
])
def test_validation_rejects_before_launch(over, rc):
    d, lay, cch = _args(**dict(over))
    assert _decode(d, lay, cch) == rc
    d, lay, cch = _args(**dict(over))
    assert _append(d, lay, cch) == rc
    d, lay, cch = _args(**dict(over))
    assert _step(d, lay, cch) == rc


def test_validation_pointer_and_size_errors():
    d, lay, cch = _args()
    assert _decode(d, lay, cch, q=FAKE + 2) == ERR_ARG            # misaligned
    assert _decode(d, lay, cch, out=0) == ERR_ARG                 # null
    assert _decode(d, lay, cch, seq=0) == ERR_ARG
    assert _decode(d, lay, cch, batch=0) == ERR_ARG
    assert _decode(d, lay, cch, max_len=8 * 16 + 1) == ERR_ARG    # beyond the block table
    need = _lib().kvq_decode_workspace_bytes(C.byref(d), 2, 100)
    assert need > 0
    assert _decode(d, lay, cch, wsb=need - 1) == ERR_WS
    assert _decode(d, lay, cch, ws=0) == ERR_WS
    assert _append(d, lay, cch, mx=5) == ERR_ARG                   # max_new > total_new
    assert _append(d, lay, cch, k=FAKE + 8) == ERR_ARG
    assert _append(d, lay, cch, cu=0) == ERR_ARG
    assert _append(d, lay, cch, total=0, mx=0) == 0                # nothing to do, no launch
    cch.sink = 0
    assert _append(d, lay, cch) == ERR_ARG                         # n_sink > 0 needs a sink
    lay2 = kvq2.KvqLayer(FAKE + 4, FAKE, 4.0, 4.0)
    d, _, cch = _args()
    assert _decode(d, lay2, cch) == ERR_ARG


def test_decode_step_validates_both_halves_before_launch():
    d, lay, cch = _args()
    need = _lib().kvq_decode_workspace_bytes(C.byref(d), 2, 100)
    # append half
    assert _step(d, lay, cch, mx=5) == ERR_ARG
    assert _step(d, lay, cch, k=FAKE + 8) == ERR_ARG
    assert _step(d, lay, cch, sp=0) == ERR_ARG
    # decode half (also when there is nothing to append)
    assert _step(d, lay, cch, q=FAKE + 2) == ERR_ARG
    assert _step(d, lay, cch, seq=0) == ERR_ARG
    assert _step(d, lay, cch, max_len=8 * 16 + 1) == ERR_ARG
    assert _step(d, lay, cch, wsb=need - 1) == ERR_WS
    assert _step(d, lay, cch, total=0, mx=0, ws=0) == ERR_WS
    assert _step(d, lay, cch, batch=0) == ERR_ARG


def test_decode_rejects_batches_beyond_32bit_tile_counts():
    # 1024 sequences x 8 KV heads x 4M tokens: the batch's tile count does
    # not fit the decode's 32-bit counters; refused before any launch.
    L = 1 << 22
    d, lay, cch = _args(bt_stride=L // 16)
    assert _decode(d, lay, cch, batch=1024, max_len=L) == ERR_UNSUP
    assert _decode(d, lay, cch, batch=1024, max_len=L, ws=0) == ERR_UNSUP


def test_workspace_bytes_grow_with_batch_and_length():
    d = kvq2.dims(32, 8, 16, 4, 256)
    f = lambda b, n: _lib().kvq_decode_workspace_bytes(C.byref(d), b, n)
    assert f(1, 0) > 0
    assert f(28, 100000) >= f(1, 100000)
    assert f(1, 131072) >= f(1, 1024)
    bad = kvq2.dims(32, 8, 16, 4, 256, head_dim=64)
    assert _lib().kvq_decode_workspace_bytes(C.byref(bad), 1, 10) == 0


# ---------------------------------------------------------------- host calibration

def _aniso_calibration(N=1024, Hq=4, Hkv=2, seed=7):
    """Queries and values with distinct per-channel variances: well separated
    eigenvalues, so the eigenbasis is unique up to the sign rule."""
    rng = np.random.default_rng(seed)
    scale = np.linspace(0.5, 4.0, 128).astype(np.float32)
    q = to_bf16_bits(rng.standard_normal((N, Hq, 128)).astype(np.float32) * scale[rng.permutation(128)])
    k = to_bf16_bits(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * 2.0)
    v = to_bf16_bits(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * scale[::-1])
    return q, k, v


def test_calibrate_matches_oracle_on_separated_spectrum():
    q, k, v = _aniso_calibration()
    d = kvq2.dims(4, 2, 16, 4, 128)
    R_K, R_V, cK, cV = kvq2.calibrate(d, q, k, v, 0.999)
    cal = O.calibrate(q, k, v, 4, 2, 1 / math.sqrt(128), 0.999)
    for R in (R_K, R_V):
        for h in range(2):
            Rd = R[h].astype(np.float64)
            assert np.abs(Rd.T @ Rd - np.eye(128)).max() < 1e-6
    assert np.abs(R_K - cal.R_K).max() < 1e-4
    # C_S eigen gaps are smaller than C_Q's: allow a looser match of R_V
    assert np.abs(R_V - cal.R_V).max() < 5e-3
    # clip thresholds: the same order statistic of |bf16 rotated values|
    ulp = lambda x: 2.0 ** (math.floor(math.log2(x)) - 7)
    assert abs(cK - cal.clip_K) <= ulp(cal.clip_K)
    assert abs(cV - cal.clip_V) <= ulp(cal.clip_V)


def test_calibrate_closed_form_wiring():
    """kvq_calibrate on data whose eigenbases are known in closed form
    (tests/calib_fixture.py): R_K[h] = U_Q(h) H P and R_V[h] = U_S(h) H P
    for KV head h's own query heads, one clip per tensor."""
    from calib_fixture import ClosedFormCalibration
    for Hq, Hkv, seed in ((4, 2, 2024), (12, 3, 7)):
        fx = ClosedFormCalibration(n_q_heads=Hq, n_kv_heads=Hkv, seed=seed)
        d = kvq2.dims(Hq, Hkv, 16, 4, 128)
        R_K, R_V, cK, cV = kvq2.calibrate(d, fx.q, fx.k, fx.v, 1.0)
        for h in range(Hkv):
            assert np.abs(R_K[h] - fx.R_K[h]).max() <= 1e-6, f"R_K[{h}]"
            assert np.abs(R_V[h] - fx.R_V[h]).max() <= 1e-6, f"R_V[{h}]"
        assert (cK, cV) == (fx.clip_K, fx.clip_V)


@pytest.mark.parametrize("hb", [32, 64])
def test_calibrate_block_hadamard_matches_oracle(hb):
    """kvq_calibrate with a block-diagonal Hadamard (dims.hadamard_block): the
    closed-form fixture built for that block size, and the oracle's
    calibration on the separated spectrum."""
    from calib_fixture import ClosedFormCalibration
    fx = ClosedFormCalibration(n_q_heads=4, n_kv_heads=2, seed=11, hadamard_block=hb)
    d = kvq2.dims(4, 2, 16, 4, 128, quant_group=hb, hadamard_block=hb)
    R_K, R_V, cK, cV = kvq2.calibrate(d, fx.q, fx.k, fx.v, 1.0)
    for h in range(2):
        assert np.abs(R_K[h] - fx.R_K[h]).max() <= 1e-6, f"R_K[{h}]"
        assert np.abs(R_V[h] - fx.R_V[h]).max() <= 1e-6, f"R_V[{h}]"
    assert (cK, cV) == (fx.clip_K, fx.clip_V)
    q, k, v = _aniso_calibration()
    R_K, R_V, cK, cV = kvq2.calibrate(d, q, k, v, 0.999)
    cal = O.calibrate(q, k, v, 4, 2, 1 / math.sqrt(128), 0.999, hadamard_block=hb)
    assert np.abs(R_K - cal.R_K).max() < 1e-4
    assert np.abs(R_V - cal.R_V).max() < 5e-3


def test_pool_layout_of_quantization_groups():
    """Chunk sizes of the pool for groups of 128, 64 and 32 channels agree
    between the binding and the oracle's layout."""
    for g, nbytes in ((0, 1152), (128, 1152), (64, 1280), (32, 1536)):
        assert kvq2.chunk_bytes(g) == nbytes
        assert O.chunk_bytes(g or 128) == nbytes


def test_calibrate_invariants_on_isotropic_data():
    """iid queries: C_Q ~ I and the eigenbasis is noise; check invariants only."""
    rng = np.random.default_rng(3)
    N, Hq, Hkv = 256, 2, 1
    q = to_bf16_bits(rng.standard_normal((N, Hq, 128)).astype(np.float32))
    k = to_bf16_bits(rng.standard_normal((N, Hkv, 128)).astype(np.float32))
    d = kvq2.dims(Hq, Hkv, 16, 4, 128)
    R_K, R_V, cK, cV = kvq2.calibrate(d, q, k, k, 1.0)
    qf = O.bf16_bits_to_f32(q).astype(np.float64)
    C_Q = O.query_covariance(qf[:, 0:2, :])
    # R^T C_Q R = (H P)^T Lambda (H P): its diagonal is constant = trace/128
    M = R_K[0].astype(np.float64).T @ C_Q @ R_K[0].astype(np.float64)
    assert np.allclose(np.diag(M), np.trace(C_Q) / 128, rtol=1e-5)
    rk = O.rotate(k[:, 0], R_K[0])
    assert cK == float(np.abs(O.bf16_bits_to_f32(rk)).max())     # p = 1 -> max


def test_calibrate_rejects_bad_input():
    q, k, v = _aniso_calibration(N=32)
    d = kvq2.dims(4, 2, 16, 4, 128)
    for p in (0.0, 1.5, float("nan")):
        with pytest.raises(kvq2.KvqError, match="ARG"):
            kvq2.calibrate(d, q, k, v, p)
    bad = q.copy()
    bad[3, 1, 7] = 0x7F80              # +inf
    with pytest.raises(kvq2.KvqError, match="NUMERIC"):
        kvq2.calibrate(d, bad, k, v, 0.999)
    huge = to_bf16_bits(np.full((32, 2, 128), 30000.0, np.float32))
    with pytest.raises(kvq2.KvqError, match="NUMERIC"):          # clip > 16384
        kvq2.calibrate(d, q, huge, v, 0.999)


def _noalloc(d, lay, cch, batch=2, seq=FAKE, max_len=100, q=FAKE, out=FAKE):
    return _lib().kvq_decode_attention_noalloc(C.byref(d), C.byref(lay), C.byref(cch), batch, seq,
                                               max_len, q, out, None)


def test_noalloc_decode_validates_before_launch():
    """The no-alloc decode checks what kvq_decode_attention checks, and
    refuses a decode whose workspace exceeds its 64 MiB scratch, all before
    any HIP call."""
    d, lay, cch = _args()
    assert _noalloc(d, lay, cch, q=FAKE + 2) == ERR_ARG
    assert _noalloc(d, lay, cch, out=0) == ERR_ARG
    assert _noalloc(d, lay, cch, seq=0) == ERR_ARG
    assert _noalloc(d, lay, cch, batch=0) == ERR_ARG
    assert _noalloc(d, lay, cch, max_len=8 * 16 + 1) == ERR_ARG
    d, lay, cch = _args(P=8)
    assert _noalloc(d, lay, cch) == ERR_UNSUP
    # 2000 sequences of 64 query heads: the rotated queries alone take 67 MB
    d, lay, cch = _args(Hq=64, Hkv=8)
    need = _lib().kvq_decode_workspace_bytes(C.byref(d), 2000, 100)
    assert need > 64 << 20
    assert _noalloc(d, lay, cch, batch=2000) == ERR_WS
    assert b"64 MiB" in _lib().kvq_last_error()


# ---------------------------------------------------------------- prefix-aware decode

def _groups(n_groups=1, n_members=4, arrays=True):
    p = FAKE + 0x600000 if arrays else None
    return kvq2.KvqPrefixGroups(n_groups, n_members, p, p and p + 0x1000, p and p + 0x2000)


def _prefix(d, lay, cch, g, batch=2, seq=FAKE, max_len=100, q=FAKE, out=FAKE, ws=FAKE,
            wsb=1 << 30):
    return _lib().kvq_decode_prefix_attention(C.byref(d), C.byref(lay), C.byref(cch), batch, seq,
                                              max_len, q, out, None if g is None else C.byref(g),
                                              ws, wsb, None)


def test_prefix_decode_validates_before_launch():
    d, lay, cch = _args()
    assert _prefix(d, lay, cch, None) == ERR_ARG
    assert _prefix(d, lay, cch, _groups(n_groups=-1)) == ERR_ARG
    assert _prefix(d, lay, cch, _groups(n_groups=257)) == ERR_ARG
    assert _prefix(d, lay, cch, _groups(n_members=-1)) == ERR_ARG
    assert _prefix(d, lay, cch, _groups(arrays=False)) == ERR_ARG
    assert _prefix(d, lay, cch, _groups(), q=FAKE + 2) == ERR_ARG      # the decode's own checks
    assert _prefix(d, lay, cch, _groups(), seq=0) == ERR_ARG
    need = _lib().kvq_decode_prefix_workspace_bytes(C.byref(d), 2, 100, C.byref(_groups()))
    assert _prefix(d, lay, cch, _groups(), wsb=need - 1) == ERR_WS
    assert _prefix(d, lay, cch, _groups(), ws=0) == ERR_WS


def test_prefix_workspace_bytes():
    d = kvq2.dims(64, 8, 16, 4, 128)
    f = lambda g: _lib().kvq_decode_prefix_workspace_bytes(C.byref(d), 64, 65536, g)
    plain = _lib().kvq_decode_workspace_bytes(C.byref(d), 64, 65536)
    assert f(C.byref(_groups(n_groups=0, n_members=0, arrays=False))) == plain
    one, two = f(C.byref(_groups(1, 32))), f(C.byref(_groups(2, 32)))
    assert plain < one <= two
    assert f(None) == 0 and f(C.byref(_groups(n_groups=300))) == 0
    # quantization groups narrower than the head: the groups are not used
    dn = kvq2.dims(64, 8, 16, 4, 128, quant_group=32)
    g = C.byref(_groups(1, 32))
    assert (_lib().kvq_decode_prefix_workspace_bytes(C.byref(dn), 64, 65536, g)
            == _lib().kvq_decode_workspace_bytes(C.byref(dn), 64, 65536))
