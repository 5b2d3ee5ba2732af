"""GPU parity of quantization groups narrower than the head (32 or 64
channels per (scale, zero) pair; OSCAR technical summary, sec. 2.2-B), with a
full or a block-diagonal Hadamard in the rotation, through the C ABI.

The cache bytes after ragged bulk appends and token-by-token steps must equal
the oracle's (pool chunks of 1024 + 128 * (128 / group) bytes), and decode,
decode-step and multi-query outputs must match the oracle within 2e-3 max
normwise relative error.  Up to four query rows per KV head run on the
matrix-core kernel (one QK column block per group, one PV operand per
group), more on the VALU kernel; both kernels are tested."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import TOL, Scenario, dev_u16, rel_err, say
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

pytestmark = pytest.mark.gpu

LAYOUTS = [(32, 32), (64, 64), (32, 128)]      # (quant_group, hadamard_block)


@pytest.fixture(params=["mfma", "valu"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
    return request.param


def _ids(v):
    return f"g{v[0]}_hb{v[1]}"


CASES = [
    # Hq, Hkv, P, n_sink, W, lens
    (8, 2, 16, 4, 32, [700, 130, 17, 0]),      # G = 4, an empty and a short sequence
    (8, 8, 64, 0, 16, [1100, 45]),             # G = 1, no sink, page 64
    (4, 2, 16, 4, 32, [650, 3, 130]),          # G = 2
    (32, 2, 32, 20, 64, [900]),                # G = 16
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=_ids)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[0]}x{c[1]}_P{c[2]}")
def test_group_cache_bytes_and_decode(case, layout, kernel):
    Hq, Hkv, P, ns, W, lens = case
    g, hb = layout
    say(f"[groups] {case} group={g} hadamard_block={hb} kernel={kernel}")
    sc = Scenario(Hq, Hkv, P, ns, W, lens, seed=3 * g + Hq, fill=0x33, quant_group=g,
                  hadamard_block=hb)
    assert sc.dc.pool.shape[-1] == O.chunk_bytes(g)
    sc.fill_to(pieces=3)
    assert sc.cache_bytes_equal() == (True, True, True)
    got, ref, _ = sc.decode()
    assert np.isfinite(got).all()
    e = rel_err(got, ref)
    say(f"  rel_err={e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("layout", LAYOUTS[:2], ids=_ids)
def test_group_decode_steps(layout, kernel):
    """Token-by-token decode steps (append then attention in one call) over
    ring evictions into INT2 chunks of the narrower layout."""
    g, hb = layout
    sc = Scenario(8, 2, 16, 4, 8, [300, 60], seed=17 + g, quant_group=g, hadamard_block=hb)
    sc.append([250, 40])
    for i in range(20):
        got, ref = sc.step([1, 1], q_seed=i)
        assert rel_err(got, ref) <= TOL, f"step {i}"
    assert sc.cache_bytes_equal() == (True, True, True)


@pytest.mark.parametrize("layout", LAYOUTS[:2], ids=_ids)
def test_group_multi_query(layout, kernel):
    g, hb = layout
    M = 4
    sc = Scenario(8, 2, 16, 4, 16, [400, 90, 3], seed=29 + g, quant_group=g, hadamard_block=hb)
    sc.fill_to(pieces=2)
    q = normal_bits(sc.seed * 31 + 5, (sc.B, M, sc.od.n_q_heads, 128))
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    maxL = max(sc.cur)
    ws = torch.zeros(kvq2.decode_multi_workspace_bytes(sc.kd, sc.B, maxL, M), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((sc.B, M, sc.od.n_q_heads, 128), float("nan"), device="cuda")
    kvq2.decode_multi_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, M, dev_u16(q), out,
                                ws)
    torch.cuda.synchronize()
    ref = O.decode_multi(sc.oc, sc.R_K, sc.R_V, sc.cur, M, q)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= TOL
