"""Proxy-compensated block-sparse attention forward, float64 (CPU).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it.

Follows the proxy route of the PrimTS page ("proxy-compensated block-sparse
attention", flashinfer pull request 4872: the description's proxy paragraph
and the Sol-Attn scope note).  Selected KV blocks are attended exactly.
Every other semantic KV block n of the row stands in through two summaries
that the caller supplies: the arithmetic mean of its keys (Kbar_n) and the
sum of its values (Vsum_n).  The softmax denominator counts such a block at
its token mass c_n, the number of tokens in it (the true length of the final,
partial block).  For a query row with scaled scores s_j on exact keys and
sbar_n = scale * q.Kbar_n on omitted blocks:

    O   = (sum_j e^{s_j} v_j + sum_n e^{sbar_n} Vsum_n)
          / (sum_j e^{s_j} + sum_n c_n e^{sbar_n})
    LSE = log(sum_j e^{s_j} + sum_n c_n e^{sbar_n})

This is attention with each omitted block's c_n tokens replaced by copies of
(Kbar_n, Vsum_n / c_n).  A block on the row's exact list is never also
counted as a proxy, and a row whose blocks are all exact has no proxy term.
Proxies are defined with no element mask (the pages restrict them to dense
masks), so the mask list's blocks are attended exactly like the full list's.
"""
from __future__ import annotations

import numpy as np

from .metadata import cdiv


def block_summaries(k: np.ndarray, v: np.ndarray, block_kv: int):
    """Mean K and summed V per semantic KV block: k, v [B,Sk,Hkv,D] ->
    (Kbar, Vsum) [B,N,Hkv,D] float64, N = ceil(Sk/block_kv); the last block
    averages and sums over its true length."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sk, Hkv, D = k.shape
    N = cdiv(Sk, block_kv)
    kbar = np.zeros((B, N, Hkv, D))
    vsum = np.zeros((B, N, Hkv, D))
    for n in range(N):
        sl = slice(n * block_kv, min((n + 1) * block_kv, Sk))
        kbar[:, n] = k[:, sl].mean(axis=1)
        vsum[:, n] = v[:, sl].sum(axis=1)
    return kbar, vsum


def proxy_attention(q, k, v, full, part, kbar, vsum, block_q: int, block_kv: int,
                    scale: float, q_blocks=None):
    """q [B,Sq,H,D], k/v [B,Sk,Hkv,D], full/part bool [B,H,M,N] (together the
    exact blocks of each Q-block row), kbar/vsum [B,N,Hkv,D].  Returns O
    [B,Sq,H,D] and LSE [B,H,Sq] float64 (natural log); q_blocks optionally
    limits the work to some (b, h, i), the rest left NaN."""
    q, k, v, kbar, vsum = (np.asarray(x, np.float64) for x in (q, k, v, kbar, vsum))
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    M, N = cdiv(Sq, block_q), cdiv(Sk, block_kv)
    if full.shape != (B, H, M, N) or part.shape != (B, H, M, N):
        raise ValueError(f"block masks must be {(B, H, M, N)}")
    if kbar.shape != (B, N, Hkv, D) or vsum.shape != (B, N, Hkv, D):
        raise ValueError(f"summaries must be {(B, N, Hkv, D)}")
    mass = np.array([min(block_kv, Sk - n * block_kv) for n in range(N)], np.float64)
    O = np.full((B, Sq, H, D), np.nan)
    LSE = np.full((B, H, Sq), np.nan)
    if q_blocks is None:
        q_blocks = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    for (b, h, i) in q_blocks:
        hk = h // (H // Hkv)
        rows = np.arange(i * block_q, min((i + 1) * block_q, Sq))
        exact = np.asarray(full[b, h, i], bool) | np.asarray(part[b, h, i], bool)
        cols = np.concatenate([np.arange(n * block_kv, min((n + 1) * block_kv, Sk))
                               for n in np.flatnonzero(exact)] + [np.zeros(0, np.int64)])
        omitted = np.flatnonzero(~exact)
        qr = q[b, rows, h]                                   # [r, D]
        s = scale * qr @ k[b, cols, hk].T                    # [r, exact keys]
        sbar = scale * qr @ kbar[b, omitted, hk].T           # [r, omitted blocks]
        if s.shape[1] + sbar.shape[1] == 0:
            O[b, rows, h] = 0.0
            LSE[b, h, rows] = -np.inf
            continue
        m = np.concatenate([s, sbar], axis=1).max(axis=1, keepdims=True)
        e = np.exp(s - m)
        ebar = np.exp(sbar - m)
        den = e.sum(axis=1) + ebar @ mass[omitted]
        num = e @ v[b, cols, hk] + ebar @ vsum[b, omitted, hk]
        O[b, rows, h] = num / den[:, None]
        LSE[b, h, rows] = m[:, 0] + np.log(den)
    return O, LSE


def proxy_attention_bwd(q, k, v, full, part, kbar, vsum, block_q: int, block_kv: int,
                        scale: float, dout):
    """Gradients of proxy_attention's O, for the upstream gradient dout
    [B,Sq,H,D], with respect to q, k, v, kbar and vsum (float64).  The
    forward's definition differentiated (the same pages; the backward is the
    derivative of the forward): per query row, with P_j = e^{s_j} / den on
    exact keys and Pbar_n = e^{sbar_n} / den on omitted blocks,

        dv_j    += P_j dO                 dvsum_n += Pbar_n dO
        dS_j     = P_j (dO.v_j - D)       dSbar_n  = Pbar_n (dO.vsum_n - c_n D)
        dq       = scale (sum_j dS_j k_j + sum_n dSbar_n kbar_n)
        dk_j    += scale dS_j q           dkbar_n += scale dSbar_n q

    where D = dO.O and c_n is block n's token mass.  Rows are summed over the
    Q heads that share a KV head.  Returns (dq, dk, dv, dkbar, dvsum)."""
    q, k, v, kbar, vsum, dout = (np.asarray(x, np.float64) for x in (q, k, v, kbar, vsum, dout))
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    M, N = cdiv(Sq, block_q), cdiv(Sk, block_kv)
    mass = np.array([min(block_kv, Sk - n * block_kv) for n in range(N)], np.float64)
    O, LSE = proxy_attention(q, k, v, full, part, kbar, vsum, block_q, block_kv, scale)
    dq = np.zeros_like(q)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    dkbar, dvsum = np.zeros_like(kbar), np.zeros_like(vsum)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            for i in range(M):
                rows = np.arange(i * block_q, min((i + 1) * block_q, Sq))
                exact = np.asarray(full[b, h, i], bool) | np.asarray(part[b, h, i], bool)
                cols = np.concatenate([np.arange(n * block_kv, min((n + 1) * block_kv, Sk))
                                       for n in np.flatnonzero(exact)] + [np.zeros(0, np.int64)])
                omitted = np.flatnonzero(~exact)
                if cols.size + omitted.size == 0:
                    continue
                qr, g = q[b, rows, h], dout[b, rows, h]
                lse = LSE[b, h, rows][:, None]
                Dr = (g * O[b, rows, h]).sum(axis=1, keepdims=True)
                kc, vc = k[b, cols, hk], v[b, cols, hk]
                kb, vb = kbar[b, omitted, hk], vsum[b, omitted, hk]
                P = np.exp(scale * qr @ kc.T - lse)
                Pb = np.exp(scale * qr @ kb.T - lse)
                dS = P * (g @ vc.T - Dr)
                dSb = Pb * (g @ vb.T - mass[omitted][None, :] * Dr)
                dq[b, rows, h] = scale * (dS @ kc + dSb @ kb)
                dk[b, cols, hk] += scale * dS.T @ qr
                dv[b, cols, hk] += P.T @ g
                dkbar[b, omitted, hk] += scale * dSb.T @ qr
                dvsum[b, omitted, hk] += Pb.T @ g
    return dq, dk, dv, dkbar, dvsum
