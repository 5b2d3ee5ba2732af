"""GPU test of kvq_decode_attention_noalloc (the decode without a caller
workspace, for callers that cannot allocate) through the C ABI: two calls in
a row, the second on a smaller batch, each with outputs identical to
kvq_decode_attention's on the same inputs and within the decode tolerance of
the CPU oracle, for both decode kernels and a 16-head group (whose decode
keeps arrival counters in the scratch)."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Scenario, dev_u16, rel_err, say
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["mfma", "valu"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
    return request.param


def _both(sc, q_seed):
    """(no-alloc output, workspace output, oracle output) on the same query."""
    q = normal_bits(sc.seed * 31 + q_seed, (sc.B, sc.od.n_q_heads, 128))
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    maxL = max(sc.cur)
    ws = torch.zeros(kvq2.decode_workspace_bytes(sc.kd, sc.B, maxL), dtype=torch.uint8,
                     device="cuda")
    out_ws = torch.full((sc.B, sc.od.n_q_heads, 128), float("nan"), device="cuda")
    out_na = torch.full((sc.B, sc.od.n_q_heads, 128), float("nan"), device="cuda")
    qd = dev_u16(q)
    kvq2.decode_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, qd, out_ws, ws)
    kvq2.decode_attention_noalloc(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, qd, out_na)
    torch.cuda.synchronize()
    ref = sc.oc.decode(sc.R_K, sc.R_V, sc.cur, q)
    return out_na.cpu().numpy(), out_ws.cpu().numpy(), ref


@pytest.mark.parametrize("shape", [(8, 2, 16, 4, 32), (16, 1, 16, 4, 8)],
                         ids=["h8x2_P16", "h16x1_P16"])
def test_noalloc_decode_twice_second_smaller(shape, kernel):
    Hq, Hkv, P, ns, W = shape
    big = Scenario(Hq, Hkv, P, ns, W, [900, 500, 77, 0], seed=61)
    big.fill_to(pieces=2)
    small = Scenario(Hq, Hkv, P, ns, W, [130, 20], seed=62)
    small.fill_to(pieces=1)
    for name, sc in (("first, 4 sequences", big), ("second, 2 shorter sequences", small)):
        got, want, ref = _both(sc, q_seed=7)
        say(f"  {shape} {kernel} {name}: rel_err {rel_err(got, ref):.3e}")
        assert np.isfinite(got).all()
        assert np.array_equal(got, want), f"{name}: no-alloc output differs from the workspace call"
        assert rel_err(got, ref) <= TOL
