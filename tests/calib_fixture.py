"""Calibration data whose OSCAR rotations are known in closed form.

OSCAR technical summary, sec. 2.2-A items 1-3: for each KV head h,
R_K = U_Q H P_br with U_Q the eigenbasis of the pooled query covariance of
h's query heads, and R_V = U_S H P_br with U_S the eigenbasis of the
covariance of the attention outputs (V^T S^T S V).

Construction (all values exact in bf16), N = 128 calibration tokens:
  * query head g of KV head h, token n:  q = c_g * alpha_n * e_{pi_h(n)}
    with alpha_n = 1024 + 8 n and c_g = 2^g;
  * key of KV head h, token n:           k = e_{pi_h(n)}
  * value of KV head h, token n:         v = beta_{h,n} * e_{rho_h(n)}
    with beta_{h,n} = 1 + a_h(n) / 128, a_h a permutation of 0..127.
Keys are orthonormal and every query is parallel to its own key, so the
causal softmax of every query row puts weight 1 - O(n e^-90) on its own
token: S = I and the attention outputs are the values.  Hence
  C_Q(h) = diag over pi_h(n) of (sum_g c_g^2 / G) alpha_n^2 / N,
  C_S(h) = diag over rho_h(n) of beta_{h,n}^2 / N,
and the eigenbases are signed permutation matrices (all signs + by the
largest-entry rule): column j of U_Q is e_{pi_h(127 - j)} (alpha grows with
n) and column j of U_S is e_{rho_h(m_j)} with m_j the token of the j-th
largest beta.  Each KV head has its own permutations, so a wrong head slice,
a swapped U_Q / U_S or a clip threshold taken from the other tensor changes
the result.  The Hadamard and the bit reversal are built here from scipy and
string reversal, independently of the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.linalg

N_TOKENS = 128
D = 128


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns through torch's conversion (round to nearest even)."""
    import torch
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def hadamard_bitrev(block: int = D) -> np.ndarray:
    """H P_br in fp64: column k is column bitrev7(k) of the Sylvester Hadamard
    / sqrt(128), or of its block-diagonal form with blocks of `block`."""
    H = np.zeros((D, D))
    Hb = scipy.linalg.hadamard(block).astype(np.float64) / math.sqrt(block)
    for i in range(D // block):
        H[i * block:(i + 1) * block, i * block:(i + 1) * block] = Hb
    cols = [int(format(k, "07b")[::-1], 2) for k in range(D)]
    return H[:, cols]


class ClosedFormCalibration:
    def __init__(self, n_q_heads: int = 4, n_kv_heads: int = 2, seed: int = 2024,
                 hadamard_block: int = D):
        Hq, Hkv = n_q_heads, n_kv_heads
        G = Hq // Hkv
        rng = np.random.default_rng(seed)
        self.G = G
        self.pi = [rng.permutation(D) for _ in range(Hkv)]
        self.rho = [rng.permutation(D) for _ in range(Hkv)]
        self.a = [rng.permutation(D) for _ in range(Hkv)]
        n = np.arange(N_TOKENS)
        self.alpha = 1024.0 + 8.0 * n
        self.beta = [1.0 + a / 128.0 for a in self.a]
        q = np.zeros((N_TOKENS, Hq, D), np.float32)
        k = np.zeros((N_TOKENS, Hkv, D), np.float32)
        v = np.zeros((N_TOKENS, Hkv, D), np.float32)
        for h in range(Hkv):
            for t in range(N_TOKENS):
                k[t, h, self.pi[h][t]] = 1.0
                v[t, h, self.rho[h][t]] = self.beta[h][t]
                for g in range(G):
                    q[t, h * G + g, self.pi[h][t]] = 2.0 ** g * self.alpha[t]
        self.q, self.k, self.v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        # the construction is exact in bf16
        import torch
        back = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert np.array_equal(back(self.q), q) and np.array_equal(back(self.v), v)
        HP = hadamard_bitrev(hadamard_block)
        self.R_K = np.zeros((Hkv, D, D))
        self.R_V = np.zeros((Hkv, D, D))
        self.eig_Q = np.zeros((Hkv, D))
        self.eig_S = np.zeros((Hkv, D))
        pool = sum(4.0 ** g for g in range(G)) / G
        for h in range(Hkv):
            UQ = np.zeros((D, D))
            for j in range(D):
                UQ[self.pi[h][D - 1 - j], j] = 1.0
            order = np.argsort(-self.beta[h], kind="stable")
            US = np.zeros((D, D))
            for j in range(D):
                US[self.rho[h][order[j]], j] = 1.0
            self.R_K[h] = UQ @ HP
            self.R_V[h] = US @ HP
            self.eig_Q[h] = pool * self.alpha[::-1] ** 2 / N_TOKENS
            self.eig_S[h] = self.beta[h][order] ** 2 / N_TOKENS
        # clip at p = 1: every nonzero rotated key entry is +-fp32(1/sqrt(block))
        # times 1; the largest rotated value entry is beta_max times it (fp64
        # product, then fp32, then bf16)
        c32 = np.float64(np.float32(1.0 / math.sqrt(hadamard_block)))
        to_f = lambda x: float(back(bf16_bits(np.float32(x)))[()])
        self.clip_K = to_f(c32)
        self.clip_V = to_f(np.float32(max(b.max() for b in self.beta) * c32))
