"""A model of the fused forward kernel's bf16 roundings, for one sequence and
one v-head, used to decide where precision matters (test infrastructure: it
is neither the oracle nor the product).

It follows the kernel's arithmetic for a 64-token chunk (gated delta rule
chunk form; bf16 MFMA operands, fp32 accumulation, fp32 state):

  hb = bf16(H);  R = v - e^G (k hb);  Ao = bf16(-strict_lower(e^{G_i-G_j} k_i.k_j))
  per 16-token diagonal block: L = strict_lower(b_i e^{G_i-G_j} k_i.k_j),
      D = (I + L)^-1 by the product ladder (I+X)(I+X^2)(I+X^4)(I+X^8), X = -L,
      with bf16-rounded factors and fp32 partial products,
      Di = bf16(D diag(b)),  Dd = bf16(diag(e^{G_L-G}) D diag(b))
  block substitution: Xb_a = bf16(Di_a bf16(R_a + sum_{c<a} Ao_ac Xb_c)),
                      Vt_a = bf16(Dd_a (same))
  o = bf16(scale e^G (q hb) + bf16(P) Xb),  P = scale e^{G_i-G_j} q_i.k_j (j <= i)
  H = e^{G_L} H + k^T Vt

and can switch each rounding off.  The fp64 reference is the per-token
recurrence S_t = e^{g_t} S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = scale S_t q_t, written out again here.
"""
from __future__ import annotations

import numpy as np

import gdr_inputs as gi


def _bf(x):
    return gi.round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _inverse(L, exact: bool):
    """(I + L)^-1 of a strictly lower 16x16 block: exactly, or by the
    kernel's ladder on transposed factors with bf16-rounded multiplicands."""
    if exact:
        return np.linalg.inv(np.eye(16) + L)
    X = -L
    x, xt = _bf(X), _bf(X.T)
    x2, x2t = _f32(x @ x), _f32(xt @ xt)
    p1t = _f32(np.eye(16) + X.T)
    p2t = _f32(_bf(x2).T @ _bf(p1t) + p1t)
    x4, x4t = _f32(_bf(x2t).T @ _bf(x2)), _f32(_bf(x2).T @ _bf(x2t))
    p3t = _f32(_bf(x4).T @ _bf(p2t) + p2t)
    x8 = _f32(_bf(x4t).T @ _bf(x4))
    return _f32(_bf(x8).T @ _bf(p3t) + p3t).T


def kernel_model(q, k, v, g, b, h0, scale, exact_inverse=False, round_vnew=True, round_o=True):
    """Outputs and final state of one (sequence, v-head) under the kernel's
    roundings.  exact_inverse: the diagonal-block inverses exact (fp64);
    round_vnew=False: Vnew's bf16 roundings (the substitution operand and its
    two products Xb, Vt) left out; round_o=False: o not rounded to bf16."""
    T, d = k.shape
    H = h0.copy()
    O = np.zeros((T, d))
    for c0 in range(0, T, 64):
        sl = slice(c0, c0 + 64)
        qc, kc, vc, gc, bc = q[sl], k[sl], v[sl], g[sl], b[sl]
        n = len(gc)
        G = _f32(np.cumsum(gc))
        eg, GL = _f32(np.exp(G)), G[-1]
        lam = _f32(np.exp(GL - G))
        hb = _bf(H)
        R = _f32(vc - eg[:, None] * _f32(kc @ hb))
        S = _f32(kc @ kc.T)
        E = np.exp(np.minimum(G[:, None] - G[None, :], 0.0))
        Ao = _bf(-np.tril(E * S, -1))
        rnd = _bf if round_vnew else (lambda a: a)
        Xb, Vt = np.zeros((n, d)), np.zeros((n, d))
        for a0 in range(0, n, 16):
            ia = slice(a0, min(a0 + 16, n))
            m = ia.stop - ia.start
            L = np.zeros((16, 16))
            L[:m, :m] = np.tril(bc[ia, None] * E[ia, ia] * S[ia, ia], -1)
            D = _inverse(_f32(L), exact_inverse)[:m, :m]
            Di, Dd = _bf(D * bc[ia][None, :]), _bf(lam[ia][:, None] * D * bc[ia][None, :])
            Ra = R[ia] + sum(Ao[ia, c:c + 16] @ Xb[c:c + 16] for c in range(0, a0, 16))
            rb = rnd(_f32(Ra))   # the substitution's operand and its two results: Vnew's roundings
            Xb[ia], Vt[ia] = rnd(_f32(Di @ rb)), rnd(_f32(Dd @ rb))
        P = _bf(np.tril(scale * E * _f32(qc @ kc.T)))
        o = _f32(_f32(scale * eg)[:, None] * _f32(qc @ hb) + P @ Xb)
        O[sl] = _bf(o) if round_o else o
        H = _f32(np.exp(GL) * H + kc.T @ Vt)
    return O, H


def reference(q, k, v, g, b, h0, scale):
    """The per-token recurrence in fp64."""
    H = h0.copy()
    O = np.zeros_like(v)
    for t in range(len(k)):
        H = np.exp(g[t]) * H
        H = H + np.outer(k[t], b[t] * (v[t] - H.T @ k[t]))
        O[t] = scale * H.T @ q[t]
    return O, H


def case(T: int, g_mode: str, seed: int = 77):
    """One sequence, one head, d = 128, bf16 inputs of the benchmark's distributions."""
    d = gi.generate(gi.Workload("model", 1, T, 1, 1, 128, 128, "bf16", seed=seed), g_mode=g_mode)
    q, k, v, g, b = (d[n][0, :, 0].astype(np.float64) for n in ("q", "k", "v", "g", "beta"))
    return q, k, v, g, b, d["h0"][0, 0].astype(np.float64), d["scale"]
