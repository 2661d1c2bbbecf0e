"""Closed form of the unrolled recurrence, for tiny lengths (numpy, float64).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

Unrolling h_t = a_t h_{t-1} + x_t (x) B_t of [分块推理 §2] (page
"分块推理：解锁循环模型并行计算，实现长序列高效处理") from h_{-1} = h0 gives

    h_t = sum_{s<=t} (prod_{r=s+1..t} a_r) x_s (x) B_s  +  (prod_{r=0..t} a_r) h0,

so  y_t = sum_{s<=t} (C_t . B_s)(prod_{r=s+1..t} a_r) x_s + (prod_{r=0..t} a_r) h0 C_t + D x_t.

Every product is formed with np.prod over the slice of a, with no log/exp shortcut and no
sharing of partial products between (s, t) pairs.  Cost is O(L^2 (P + N) + L^3) per head,
so keep L small (tens of tokens).
"""
import numpy as np


def closed_form(x, dt, A, B, C, D=None, init=None):
    x, dt, A, B, C = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    h0 = np.zeros((batch, H, P, N)) if init is None else np.asarray(init, dtype=np.float64)
    y = np.zeros((batch, L, H, P))
    fin = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dt[b, :, h] * A[h])
            for t in range(L):
                acc = np.zeros(P)
                for s in range(t + 1):
                    w = np.prod(a[s + 1:t + 1])               # empty product = 1
                    acc += np.dot(C[b, t, g], B[b, s, g]) * w * x[b, s, h]
                acc += np.prod(a[0:t + 1]) * (h0[b, h] @ C[b, t, g])
                y[b, t, h] = acc + D[h] * x[b, t, h]
            f = np.prod(a) * h0[b, h]
            for s in range(L):
                f = f + np.prod(a[s + 1:L]) * np.outer(x[b, s, h], B[b, s, g])
            fin[b, h] = f
    return y, fin
