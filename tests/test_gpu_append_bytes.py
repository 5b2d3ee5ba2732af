"""Byte-exact GPU parity of the quantize-append path on the hand-derived
quantizer cases of tests/golden/quantizer_cases.txt (OSCAR technical summary,
sec. 1 and 2.2-B: four INT2 levels, asymmetric scale and zero; sec. 2.2-A
item 4: the per-layer clip), through all three append kernels.

R_K = R_V = I, so the rotated vector is the input itself (bf16 in, bf16 out)
and the quantizer sees exactly the golden patterns: a grid that quantizes
exactly, clipped values, a constant group (s = 0), -0, rounding ties and an
inexact scale.  One sequence is bulk-appended in one call of more than 8192
tokens (256 tokens per work-group), one in two calls of 1500 tokens (16 per
work-group), and one token by token through the one-token-per-wave step
kernel, where every token reaches INT2 by eviction from the one-slot recent
window.  Every INT2 slot must decode to the golden scale, zero and codes, and
the pool, ring and sink must equal the oracle's bytes.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import dev_u16, say
from long_context_decode_kvq_amd import kvq2

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.txt")


def _cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, clip, pat, sbits, zbits, codes, _ = [c.strip() for c in line.split("|")]
        out.append((name, float(clip), [float(t) for t in pat.split()], int(sbits, 16),
                    int(zbits, 16), [int(c) for c in codes.split()]))
    return out


CASES = _cases()
CLIPS = sorted({c[1] for c in CASES})


def _bf16_exact(vals):
    """bf16 bit patterns of values that are exact in bf16 (checked)."""
    x = np.asarray(vals, np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x)
    return bits


@pytest.mark.parametrize("clip", CLIPS, ids=[f"clip{c:g}" for c in CLIPS])
def test_golden_quantizer_cases_through_every_append_kernel(clip):
    cases = [c for c in CASES if c[1] == clip]
    vecs = np.stack([_bf16_exact(np.resize(np.asarray(c[2], np.float32), 128)) for c in cases])
    lens = [8200, 3000, 40]                     # bulk kernel, medium kernel, step kernel
    B, P = len(lens), 16
    d = O.Dims(1, 1, P, 0, 1)
    kd = kvq2.dims(1, 1, P, 0, 1)
    npg = [(L + P - 1) // P for L in lens]
    bt = np.full((B, max(npg)), -1, np.int32)
    perm = np.random.default_rng(1).permutation(sum(npg))
    o = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[o:o + n]
        o += n
    oc = O.OracleCache(d, B, sum(npg), np.where(bt < 0, 0, bt), fill=0x5A)
    dc = kvq2.DeviceCache(kd, B, sum(npg), bt, fill=0x5A)
    eye = torch.eye(128, dtype=torch.float32, device="cuda")[None].contiguous()
    lay = kvq2.layer(eye, eye, clip, clip)
    I = np.eye(128, dtype=np.float32)[None]
    # token n of sequence b: K takes case (n + b) mod m, V case (n + b + 1) mod m
    m = len(cases)
    kv = []
    for b, L in enumerate(lens):
        n = np.arange(L)
        kv.append((vecs[(n + b) % m][:, None, :], vecs[(n + b + 1) % m][:, None, :]))

    def append(b_counts, starts):
        cu = np.zeros(B + 1, np.int32)
        cu[1:] = np.cumsum(b_counts)
        if cu[-1] == 0:
            return
        ks = np.concatenate([kv[b][0][starts[b]:starts[b] + c] for b, c in enumerate(b_counts)])
        vs = np.concatenate([kv[b][1][starts[b]:starts[b] + c] for b, c in enumerate(b_counts)])
        for b, c in enumerate(b_counts):
            if c:
                oc.append(I, I, clip, clip, b, starts[b], kv[b][0][starts[b]:starts[b] + c],
                          kv[b][1][starts[b]:starts[b] + c])
        kvq2.quantize_append(kd, lay, dc.handle, B,
                             torch.tensor(starts, dtype=torch.int32, device="cuda"),
                             torch.from_numpy(cu).cuda(), int(cu[-1]), int(max(b_counts)),
                             dev_u16(ks), dev_u16(vs))

    append([8200, 0, 0], [0, 0, 0])                       # > 8192 new tokens: 256 per work-group
    append([0, 1500, 0], [8200, 0, 0])                    # 1025 .. 8192: 16 per work-group
    append([0, 1500, 0], [8200, 1500, 0])
    for t in range(40):                                   # one token per call: step kernel
        append([0, 0, 1], [8200, 3000, t])
    torch.cuda.synchronize()
    pool = dc.pool.cpu().numpy()
    assert np.array_equal(pool, oc.pool), "pool bytes differ from the oracle"
    assert np.array_equal(dc.recent.cpu().numpy().view(np.uint16), oc.recent)

    # Every INT2 position decodes to its golden scale, zero and codes.
    flat = pool.reshape(-1)
    for b, L in enumerate(lens):
        for pos in range(L - 1):                          # the last token is still in the ring
            base = int(bt[b, pos // P]) * 1152
            t = pos % 16
            for kind, idx in ((0, (pos + b) % m), (1, (pos + b + 1) % m)):
                _, _, _, sbits, zbits, codes = cases[idx]
                table = O.K_BYTE_TABLE if kind == 0 else O.V_BYTE_TABLE
                got = O.unpack_codes(flat[base + table[t]])
                off = base + O.param_offset(kind, t)
                s = int(flat[off]) | int(flat[off + 1]) << 8
                z = int(flat[off + 2]) | int(flat[off + 3]) << 8
                assert (s, z) == (sbits, zbits), (cases[idx][0], b, pos, kind, hex(s), hex(z))
                assert np.array_equal(got, np.resize(np.asarray(codes, np.uint8), 128)), \
                    (cases[idx][0], b, pos, kind)
    say(f"  clip {clip:g}: {sum(lens) - B} INT2 positions x (K, V) match the golden cases "
        f"{[c[0] for c in cases]}")
