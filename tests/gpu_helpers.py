"""Shared set-up of the GPU parity tests: one scenario is built twice, by the
CPU oracle and by libkvq2 through its C ABI, from the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as O
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

TOL = 2e-3          # max normwise relative error of decode outputs (fp32 accumulation)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||out - ref||_inf / ||ref||_inf (rows with ref = 0 use absolute error)."""
    out = out.reshape(-1, out.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


def random_block_table(rng, lens, P, extra=3):
    npg = [max(1, math.ceil(L / P)) for L in lens]
    total = sum(npg) + extra
    perm = rng.permutation(total)
    bt = np.full((len(lens), max(npg)), -1, np.int32)
    i = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[i:i + n]
        i += n
    return bt, total


class Scenario:
    """Same cache built by the oracle and on the GPU."""

    def __init__(self, Hq, Hkv, P, ns, W, lens, seed=0, fill=0, k_scale=2.0, clip=None,
                 quant_group=128, hadamard_block=128):
        self.rng = np.random.default_rng(seed)
        self.seed = seed
        self.lens = list(lens)
        B = len(lens)
        self.B = B
        self.od = O.Dims(Hq, Hkv, P, ns, W, quant_group=quant_group)
        self.kd = kvq2.dims(Hq, Hkv, P, ns, W, quant_group=quant_group,
                            hadamard_block=hadamard_block)
        self.bt, self.num_pages = random_block_table(self.rng, lens, P)
        # rotations from the oracle's calibration on seeded tokens
        cq = normal_bits(seed * 7 + 1, (256, Hq, 128))
        ck = normal_bits(seed * 7 + 2, (256, Hkv, 128), np.float32(k_scale))
        cv = normal_bits(seed * 7 + 3, (256, Hkv, 128))
        cal = O.calibrate(cq, ck, cv, Hq, Hkv, self.od.sm_scale, 0.999,
                          hadamard_block=hadamard_block)
        self.R_K, self.R_V = cal.R_K, cal.R_V
        self.clip_K = cal.clip_K if clip is None else clip
        self.clip_V = cal.clip_V if clip is None else clip
        self.oc = O.OracleCache(self.od, B, self.num_pages, np.where(self.bt < 0, 0, self.bt), fill=fill)
        self.dc = kvq2.DeviceCache(self.kd, B, self.num_pages, self.bt, fill=fill)
        self.dR_K = torch.from_numpy(self.R_K).cuda()
        self.dR_V = torch.from_numpy(self.R_V).cuda()
        self.layer = kvq2.layer(self.dR_K, self.dR_V, self.clip_K, self.clip_V)
        self.cur = [0] * B
        maxL = max(max(lens), 1)
        self.k_all = [normal_bits(seed * 1000 + 10 * b + 1, (maxL, Hkv, 128), np.float32(k_scale))
                      for b in range(B)]
        self.v_all = [normal_bits(seed * 1000 + 10 * b + 2, (maxL, Hkv, 128)) for b in range(B)]

    def append(self, counts):
        """Append counts[b] new tokens to every sequence on both sides."""
        B = self.B
        start = np.array(self.cur, np.int32)
        cu = np.zeros(B + 1, np.int32)
        cu[1:] = np.cumsum(counts)
        total = int(cu[-1])
        if total == 0:
            return
        ks = np.concatenate([self.k_all[b][self.cur[b]:self.cur[b] + counts[b]] for b in range(B)])
        vs = np.concatenate([self.v_all[b][self.cur[b]:self.cur[b] + counts[b]] for b in range(B)])
        for b in range(B):
            if counts[b]:
                self.oc.append(self.R_K, self.R_V, self.clip_K, self.clip_V, b, self.cur[b],
                               self.k_all[b][self.cur[b]:self.cur[b] + counts[b]],
                               self.v_all[b][self.cur[b]:self.cur[b] + counts[b]])
        kvq2.quantize_append(self.kd, self.layer, self.dc.handle, B,
                             torch.from_numpy(start).cuda(), torch.from_numpy(cu).cuda(),
                             total, int(max(counts)), dev_u16(ks), dev_u16(vs))
        for b in range(B):
            self.cur[b] += counts[b]

    def fill_to(self, pieces=3):
        """Bulk-append every sequence to its full length in ragged pieces."""
        rem = [L - c for L, c in zip(self.lens, self.cur)]
        for i in range(pieces):
            counts = [r // pieces + (r % pieces if i == pieces - 1 else 0) for r in rem]
            self.append(counts)

    def cache_bytes_equal(self):
        torch.cuda.synchronize()
        pool = self.dc.pool.cpu().numpy()
        sink = self.dc.sink.cpu().numpy().view(np.uint16)
        rec = self.dc.recent.cpu().numpy().view(np.uint16)
        ok_pool = np.array_equal(pool, self.oc.pool)
        ok_sink = self.od.n_sink == 0 or np.array_equal(sink, self.oc.sink)
        ok_rec = np.array_equal(rec, self.oc.recent)
        return ok_pool, ok_sink, ok_rec

    def step(self, counts, q_seed=99):
        """append(counts) and decode(q_seed) in one kvq_decode_step call."""
        B = self.B
        start = np.array(self.cur, np.int32)
        cu = np.zeros(B + 1, np.int32)
        cu[1:] = np.cumsum(counts)
        total = int(cu[-1])
        k_dev = v_dev = None
        if total:
            ks = np.concatenate([self.k_all[b][self.cur[b]:self.cur[b] + counts[b]] for b in range(B)])
            vs = np.concatenate([self.v_all[b][self.cur[b]:self.cur[b] + counts[b]] for b in range(B)])
            k_dev, v_dev = dev_u16(ks), dev_u16(vs)
        for b in range(B):
            if counts[b]:
                self.oc.append(self.R_K, self.R_V, self.clip_K, self.clip_V, b, self.cur[b],
                               self.k_all[b][self.cur[b]:self.cur[b] + counts[b]],
                               self.v_all[b][self.cur[b]:self.cur[b] + counts[b]])
            self.cur[b] += counts[b]
        q = normal_bits(self.seed * 31 + q_seed, (B, self.od.n_q_heads, 128))
        seq = torch.tensor(self.cur, dtype=torch.int32, device="cuda")
        maxL = max(self.cur)
        ws = torch.zeros(kvq2.decode_workspace_bytes(self.kd, B, maxL), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((B, self.od.n_q_heads, 128), dtype=torch.float32, device="cuda")
        kvq2.decode_step(self.kd, self.layer, self.dc.handle, B, torch.from_numpy(start).cuda(),
                         torch.from_numpy(cu).cuda(), total, int(max(counts)), k_dev, v_dev, seq,
                         maxL, dev_u16(q), out, ws)
        torch.cuda.synchronize()
        ref = self.oc.decode(self.R_K, self.R_V, self.cur, q)
        return out.cpu().numpy(), ref

    def decode(self, q_seed=99):
        q = normal_bits(self.seed * 31 + q_seed, (self.B, self.od.n_q_heads, 128))
        seq = torch.tensor(self.cur, dtype=torch.int32, device="cuda")
        maxL = max(self.cur)
        ws = torch.zeros(kvq2.decode_workspace_bytes(self.kd, self.B, maxL), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((self.B, self.od.n_q_heads, 128), dtype=torch.float32, device="cuda")
        kvq2.decode_attention(self.kd, self.layer, self.dc.handle, self.B, seq, maxL, dev_u16(q),
                              out, ws)
        torch.cuda.synchronize()
        ref = self.oc.decode(self.R_K, self.R_V, self.cur, q)
        return out.cpu().numpy(), ref, ws
