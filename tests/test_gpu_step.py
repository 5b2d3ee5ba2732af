"""GPU parity of the fused decode step (kvq_decode_step) through the C ABI:
the same cache bytes and output bits as kvq_quantize_append followed by
kvq_decode_attention, and outputs within the decode tolerance of the CPU
oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Scenario, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["mfma", "valu"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
    return request.param


STEP_CASES = [
    # Hq, Hkv, P, n_sink, W, lens, prefill
    (4, 2, 16, 4, 8, [40, 20, 9], [30, 11, 3]),         # G = 2, evictions every step
    (8, 1, 32, 0, 16, [120, 50], [100, 20]),            # G = 8, no sink
    (6, 2, 16, 3, 32, [333, 64], [300, 30]),            # G = 3 (padded group)
    (16, 1, 16, 4, 1, [40, 8], [30, 2]),                # G = 16 (VALU decode), W = 1
    (8, 2, 32, 4, 8, [40, 0, 13, 20], [30, 0, 9, 19]),  # an empty sequence; one that stops growing
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"h{c[0]}x{c[1]}_P{c[2]}_s{c[3]}_w{c[4]}")
def test_decode_step_equals_append_then_decode(case, kernel):
    Hq, Hkv, P, ns, W, lens, prefill = case
    say(f"[case] {case} kernel={kernel}")
    a = Scenario(Hq, Hkv, P, ns, W, lens, seed=3 * Hq + P)
    b = Scenario(Hq, Hkv, P, ns, W, lens, seed=3 * Hq + P)
    a.append(prefill)
    b.append(prefill)
    for step in range(5):
        counts = [1 if a.cur[i] < lens[i] else 0 for i in range(len(lens))]
        if step == 3:
            counts[-1] = 0                       # one sequence without a new token
        a.append(counts)
        out_a, ref, _ = a.decode(q_seed=step)
        out_b, ref_b = b.step(counts, q_seed=step)
        assert np.array_equal(ref, ref_b)
        torch.cuda.synchronize()
        assert torch.equal(a.dc.pool, b.dc.pool), f"step {step}: pool bytes differ"
        assert torch.equal(a.dc.recent, b.dc.recent), f"step {step}: ring differs"
        assert torch.equal(a.dc.sink, b.dc.sink), f"step {step}: sink differs"
        assert np.array_equal(out_a, out_b), f"step {step}: outputs differ"
        assert b.cache_bytes_equal() == (True, True, True), f"step {step}"
        assert rel_err(out_b, ref_b) <= TOL, f"step {step}"


def test_decode_step_large_append_and_empty_append():
    """More than 1024 new tokens (append then decode in stream order) and no
    new tokens (decode only) through the same entry point."""
    a = Scenario(4, 2, 16, 4, 16, [900, 700], seed=41)
    b = Scenario(4, 2, 16, 4, 16, [900, 700], seed=41)
    for counts in ([600, 500], [0, 0], [300, 200]):
        a.append(counts)
        out_a, ref, _ = a.decode(q_seed=sum(counts))
        out_b, ref_b = b.step(counts, q_seed=sum(counts))
        torch.cuda.synchronize()
        assert torch.equal(a.dc.pool, b.dc.pool)
        assert torch.equal(a.dc.recent, b.dc.recent)
        assert np.array_equal(out_a, out_b)
        assert b.cache_bytes_equal() == (True, True, True)
        assert rel_err(out_b, ref_b) <= TOL
