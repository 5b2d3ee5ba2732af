"""GPU parity of multi-query INT2 attention (kvq_decode_multi_attention)
against the oracle's decode_multi, through the C ABI: the M queries of each
sequence sit at its last M positions and attend causally over the sink, the
INT2 pages and the recent window (speculative verification / chunked
prefill over the same cache).  Outputs within 2e-3 max normwise relative
error per row; M = 1 is bit-identical to kvq_decode_attention.  Query blocks
wider than one pass (8 rows of queries x heads on the matrix cores, 16 on
the VALU kernel) take several passes over the pages."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import TOL, Scenario, dev_u16, rel_err, say
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["mfma", "valu"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
    return request.param


def _multi(sc, M, q_seed=5):
    q = normal_bits(sc.seed * 31 + q_seed, (sc.B, M, sc.od.n_q_heads, 128))
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    maxL = max(sc.cur)
    ws = torch.zeros(kvq2.decode_multi_workspace_bytes(sc.kd, sc.B, maxL, M), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((sc.B, M, sc.od.n_q_heads, 128), float("nan"), device="cuda")
    kvq2.decode_multi_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, M, dev_u16(q), out,
                                ws)
    torch.cuda.synchronize()
    ref = O.decode_multi(sc.oc, sc.R_K, sc.R_V, sc.cur, M, q)
    return out.cpu().numpy(), ref, q


CASES = [
    # Hq, Hkv, P, n_sink, W, lens, M          rows = M * Hq / Hkv
    (4, 2, 16, 4, 32, [300, 77, 2, 0], 4),     # 8 rows; a sequence shorter than M, an empty one
    (8, 8, 32, 0, 16, [200, 33], 2),           # G = 1: 2 rows, no sink, page 32
    (8, 2, 16, 4, 8, [100, 50], 2),            # G = 4: 8 rows
    (4, 2, 16, 4, 4, [150], 4),                # M = W: the whole recent window is queries
    (6, 2, 64, 20, 16, [500, 130], 3),         # G = 3: 9 rows, page 64, sink > 16 (MFMA: 2 passes)
    (4, 2, 16, 4, 16, [260, 40], 8),           # 16 rows (MFMA: two passes of 8; VALU: one)
    (8, 2, 16, 4, 16, [300, 50, 7], 8),        # 32 rows (MFMA: four passes; VALU: two)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[0]}x{c[1]}_P{c[2]}_w{c[4]}_M{c[6]}")
def test_multi_query_matches_oracle(case, kernel):
    Hq, Hkv, P, ns, W, lens, M = case
    say(f"[multi] {case} kernel={kernel}")
    sc = Scenario(Hq, Hkv, P, ns, W, lens, seed=7 * M + Hq)
    sc.fill_to(pieces=2)
    got, ref, _ = _multi(sc, M)
    assert np.isfinite(got).all()
    e = rel_err(got, ref)
    say(f"  rel_err={e:.3e}")
    assert e <= TOL


def test_multi_query_one_query_is_decode(kernel):
    sc = Scenario(4, 2, 16, 4, 16, [400, 90], seed=9)
    sc.fill_to(pieces=1)
    got, ref, q = _multi(sc, 1)
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    ws = torch.zeros(kvq2.decode_workspace_bytes(sc.kd, sc.B, max(sc.cur)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((sc.B, 4, 128), dtype=torch.float32, device="cuda")
    kvq2.decode_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, max(sc.cur), dev_u16(q[:, 0]),
                          out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(got[:, 0], out.cpu().numpy())
    assert rel_err(got, ref) <= TOL


def test_multi_query_verify_loop():
    """Speculative verification: append M draft tokens, verify them in one
    call, keep going; bytes and outputs against the oracle every round."""
    M = 4
    sc = Scenario(8, 2, 16, 4, 16, [240, 190], seed=13)
    sc.append([200, 150])
    for rnd in range(5):
        sc.append([M, M])
        assert sc.cache_bytes_equal() == (True, True, True), f"round {rnd}"
        got, ref, _ = _multi(sc, M, q_seed=rnd)
        assert rel_err(got, ref) <= TOL, f"round {rnd}"
