"""The library's calls under HIP graph capture: a captured decode replays to
the eager result every time (several replays with eager work in between),
and a captured run of fused decode steps (append + decode) leaves the same
cache bytes and outputs as the same steps run eagerly.  No memset nodes are
recorded by the library (its scratch clearing is a fill kernel)."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Scenario, dev_u16, rel_err
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["mfma", "valu"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
    return request.param


def test_captured_decode_replays_match_eager(kernel):
    sc = Scenario(8, 2, 16, 4, 16, [700, 300, 45], seed=23)
    sc.fill_to(pieces=2)
    q = dev_u16(normal_bits(77, (sc.B, 8, 128)))
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    ws = torch.zeros(kvq2.decode_workspace_bytes(sc.kd, sc.B, max(sc.cur)), dtype=torch.uint8,
                     device="cuda")
    out_eager = torch.empty((sc.B, 8, 128), device="cuda")
    kvq2.decode_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, max(sc.cur), q, out_eager, ws)
    torch.cuda.synchronize()
    want = out_eager.cpu().numpy()
    out_g = torch.zeros((sc.B, 8, 128), device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        kvq2.decode_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, max(sc.cur), q, out_g, ws,
                              cap)
    for r in range(4):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_g.cpu().numpy(), want), f"replay {r}"
        # eager work on the same workspace between replays
        kvq2.decode_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, max(sc.cur), q,
                              out_eager, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out_eager.cpu().numpy(), want)


def test_captured_decode_steps_match_eager():
    lens = [300, 120]
    a = Scenario(8, 2, 16, 4, 8, lens, seed=31)
    b = Scenario(8, 2, 16, 4, 8, lens, seed=31)
    a.append([280, 100])
    b.append([280, 100])
    n = 4
    B = 2
    st = [torch.tensor([280 + k, 100 + k], dtype=torch.int32, device="cuda") for k in range(n)]
    sq = [torch.tensor([281 + k, 101 + k], dtype=torch.int32, device="cuda") for k in range(n)]
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    kn = [dev_u16(np.stack([a.k_all[i][280 + k if i == 0 else 100 + k] for i in range(B)]))
          for k in range(n)]
    vn = [dev_u16(np.stack([a.v_all[i][280 + k if i == 0 else 100 + k] for i in range(B)]))
          for k in range(n)]
    qs = [dev_u16(normal_bits(500 + k, (B, 8, 128))) for k in range(n)]
    maxL = 300
    ws_a = torch.zeros(kvq2.decode_workspace_bytes(a.kd, B, maxL), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    outs_a = [torch.empty((B, 8, 128), device="cuda") for _ in range(n)]
    outs_b = [torch.empty((B, 8, 128), device="cuda") for _ in range(n)]
    for k in range(n):                      # eager
        kvq2.decode_step(a.kd, a.layer, a.dc.handle, B, st[k], cu, B, 1, kn[k], vn[k], sq[k], maxL,
                         qs[k], outs_a[k], ws_a)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):   # captured, replayed once
        for k in range(n):
            kvq2.decode_step(b.kd, b.layer, b.dc.handle, B, st[k], cu, B, 1, kn[k], vn[k], sq[k],
                             maxL, qs[k], outs_b[k], ws_b, cap)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(a.dc.pool, b.dc.pool)
    assert torch.equal(a.dc.recent, b.dc.recent)
    assert torch.equal(a.dc.sink, b.dc.sink)
    for k in range(n):
        assert torch.equal(outs_a[k], outs_b[k]), f"step {k}"
    # and against the oracle after the last step
    for i in range(B):
        b.oc.append(b.R_K, b.R_V, b.clip_K, b.clip_V, i, b.cur[i],
                    b.k_all[i][b.cur[i]:b.cur[i] + n], b.v_all[i][b.cur[i]:b.cur[i] + n])
        b.cur[i] += n
    assert b.cache_bytes_equal() == (True, True, True)
    ref = b.oc.decode(b.R_K, b.R_V, b.cur, qs[-1].cpu().numpy().view(np.uint16))
    assert rel_err(outs_b[-1].cpu().numpy(), ref) <= TOL
