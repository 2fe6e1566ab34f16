"""Pins for the per-channel-gate (KDA-style) oracle ``oracle.gdr_kda_fwd``.

The variant of "feat(cake_kda): add paired recurrent training for SM100a and
SM103a" carries one log-gate per key channel: the decay of the gated delta rule
becomes ``diag(exp(g_t))``, g_t in R^dk, applied on the key side:
``S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``,
``o_t = scale S_t q_t``; the returned state is ``H = S^T`` ``[dk, dv]``.  The
transform that makes g from a raw gate is not defined on the pages and is not
part of this (g is the log-decay itself).

Each ``pin_kda_*`` takes a callable with the signature of ``oracle.gdr_kda_fwd``.
"""
from __future__ import annotations

import numpy as np


def _case(seed, lengths, T, Hk, Hv, dk, dv, with_h0=True, beta_zero=False, g_scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = rng.standard_normal((1, T, Hk, dk))
    k = rng.standard_normal((1, T, Hk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, Hv, dv))
    g = -g_scale * np.log1p(np.exp(-rng.standard_normal((1, T, Hv, dk))))
    beta = np.zeros((1, T, Hv)) if beta_zero else 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, Hv))))
    h0 = 0.3 * rng.standard_normal((len(lengths), Hv, dk, dv)) if with_h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, h0=h0, scale=0.6)


def _call(fwd, c, **kw):
    return fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], c["h0"], scale=c["scale"], **kw)


def _close(name, got, ref, tol):
    err = float(np.abs(np.asarray(got) - np.asarray(ref)).max())
    assert err <= tol, "%s: max err %.3e > %.1e" % (name, err, tol)


def literal(c):
    """The matrix form written literally (S is dv x dk)."""
    q, k, v, g, beta, cu, h0, sc = (c[n] for n in ("q", "k", "v", "g", "beta", "cu", "h0", "scale"))
    Hk, Hv, dk, dv = q.shape[2], v.shape[2], q.shape[3], v.shape[3]
    o = np.zeros(v.shape)
    ht = np.zeros((len(cu) - 1, Hv, dk, dv))
    for n in range(len(cu) - 1):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            S = np.zeros((dv, dk)) if h0 is None else h0[n, h].T.copy()
            for t in range(cu[n], cu[n + 1]):
                kt = k[0, t, hk]
                S = S @ np.diag(np.exp(g[0, t, h])) @ (np.eye(dk) - beta[0, t, h] * np.outer(kt, kt)) \
                    + beta[0, t, h] * np.outer(v[0, t, h], kt)
                o[0, t, h] = sc * S @ q[0, t, hk]
            if cu[n + 1] > cu[n]:
                ht[n, h] = S.T
    return o, ht


def chunked(c, C):
    """Chunk form with a per-channel reference row m inside each chunk:
    q~ = q e^{G - G_m}, k~ = k e^{G - G_m}, k^ = k e^{G_m - G} (per channel),
    A = tril(diag(b) k~ k^T, -1), P = tril(q~ k^T), S_m = diag(e^{G_m}) H,
    U = (I + A)^-1 diag(b) (V - k~ S_m), O = scale (q~ S_m + P U),
    H <- diag(e^{G_L}) H + diag(e^{G_L - G_m}) k^^T U."""
    q, k, v, g, beta, cu, h0, sc = (c[n] for n in ("q", "k", "v", "g", "beta", "cu", "h0", "scale"))
    Hk, Hv, dk, dv = q.shape[2], v.shape[2], q.shape[3], v.shape[3]
    o = np.zeros(v.shape)
    ht = np.zeros((len(cu) - 1, Hv, dk, dv))
    m = (C - 1) // 2
    for n in range(len(cu) - 1):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            H = np.zeros((dk, dv)) if h0 is None else h0[n, h].copy()
            for a0 in range(cu[n], cu[n + 1], C):
                L = min(C, cu[n + 1] - a0)
                Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
                gg = np.zeros((C, dk)); bb = np.zeros(C)
                Q[:L], K[:L], V[:L] = q[0, a0:a0 + L, hk], k[0, a0:a0 + L, hk], v[0, a0:a0 + L, h]
                gg[:L], bb[:L] = g[0, a0:a0 + L, h], beta[0, a0:a0 + L, h]
                G = np.cumsum(gg, axis=0)
                Gm, GL = G[m], G[-1]
                Qt, Kt, Kh = Q * np.exp(G - Gm), K * np.exp(G - Gm), K * np.exp(Gm - G)
                A = np.tril(bb[:, None] * (Kt @ Kh.T), -1)
                P = np.tril(Qt @ Kh.T)
                Sm = np.exp(Gm)[:, None] * H
                U = np.linalg.solve(np.eye(C) + A, bb[:, None] * (V - Kt @ Sm))
                o[0, a0:a0 + L, h] = (sc * (Qt @ Sm + P @ U))[:L]
                H = np.exp(GL)[:, None] * H + np.exp(GL - Gm)[:, None] * (Kh.T @ U)
            if cu[n + 1] > cu[n]:
                ht[n, h] = H
    return o, ht


def chunked_blocks(c, C, B=16, stats=None):
    """Chunk form with one reference per block of B rows (per channel), so that
    no factor exceeds e^{(decay of one block)}: with R_b = G at the row before
    block b (R_0 = 0) and b(i) the block of row i,
      row operands   q~_i = q_i e^{G_i - R_b(i)},  k~_i = k_i e^{G_i - R_b(i)}      (<= 1)
      column copies  k^(b)_j = k_j e^{R_b - G_j},  j < B (b + 1)                  (<= 1 for j < B b)
      A_ij = b_i k~_i . k^(b(i))_j (j < i),  P_ij = q~_i . k^(b(i))_j (j <= i)
      state terms    q_i e^{G_i} H and k_i e^{G_i} H (reference: the chunk start)
      U = (I + A)^-1 diag(b) (V - (k e^G) H),  O = scale ((q e^G) H + P U)
      H <- diag(e^{G_L}) H + (k e^{G_L - G})^T U.
    ``stats`` (a dict) receives the largest exponent any factor takes."""
    q, k, v, g, beta, cu, h0, sc = (c[n] for n in ("q", "k", "v", "g", "beta", "cu", "h0", "scale"))
    Hk, Hv, dk, dv = q.shape[2], v.shape[2], q.shape[3], v.shape[3]
    o = np.zeros(v.shape)
    ht = np.zeros((len(cu) - 1, Hv, dk, dv))
    top = -np.inf
    for n in range(len(cu) - 1):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            H = np.zeros((dk, dv)) if h0 is None else h0[n, h].copy()
            for a0 in range(cu[n], cu[n + 1], C):
                L = min(C, cu[n + 1] - a0)
                Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
                gg = np.zeros((C, dk)); bb = np.zeros(C)
                Q[:L], K[:L], V[:L] = q[0, a0:a0 + L, hk], k[0, a0:a0 + L, hk], v[0, a0:a0 + L, h]
                gg[:L], bb[:L] = g[0, a0:a0 + L, h], beta[0, a0:a0 + L, h]
                G = np.cumsum(gg, axis=0)
                GL = G[-1]
                blk = np.arange(C) // B
                R = np.stack([np.zeros(dk) if b == 0 else G[B * b - 1] for b in range(C // B)])
                Qt, Kt = Q * np.exp(G - R[blk]), K * np.exp(G - R[blk])
                A = np.zeros((C, C)); P = np.zeros((C, C))
                for i in range(C):
                    b = blk[i]
                    Kc = K[:B * (b + 1)] * np.exp(R[b] - G[:B * (b + 1)])
                    top = max(top, float((R[b] - G[:B * (b + 1)]).max()), float((G[i] - R[b]).max()))
                    A[i, :i] = bb[i] * (Kc[:i] @ Kt[i])
                    P[i, :i + 1] = Kc[:i + 1] @ Qt[i]
                Qs, Ks = Q * np.exp(G), K * np.exp(G)
                U = np.linalg.solve(np.eye(C) + A, bb[:, None] * (V - Ks @ H))
                o[0, a0:a0 + L, h] = (sc * (Qs @ H + P @ U))[:L]
                H = np.exp(GL)[:, None] * H + (K * np.exp(GL - G)).T @ U
            if cu[n + 1] > cu[n]:
                ht[n, h] = H
    if stats is not None:
        stats["max_exponent"] = top
    return o, ht


def pin_kda_block_references(fwd, _scalar=None):
    """Against the chunk form with one reference per 16-row block (the form the
    GPU kernel evaluates), chunks of 64 and 16 and blocks of 16 and 4; with
    every gate at -5 per token and channel (the pages' safe-gate lower bound)
    no factor of that form exceeds e^{80} (inside fp32), while the form with
    one reference row per 64-token chunk needs e^{160}."""
    c = _case(76, [150, 1, 64, 65], 280, 1, 2, 8, 8)
    o, ht = _call(fwd, c)
    for C, B in ((64, 16), (16, 16), (64, 4)):
        o2, ht2 = chunked_blocks(c, C, B)
        _close("blocks(%d, %d) o" % (C, B), o, o2, 1e-10)
        _close("blocks(%d, %d) ht" % (C, B), ht, ht2, 1e-10)
    c5 = _case(77, [100, 37], 137, 1, 1, 8, 8)
    c5["g"][:] = -5.0
    o, ht = _call(fwd, c5)
    st = {}
    o2, ht2 = chunked_blocks(c5, 64, 16, st)
    _close("g = -5 o", o, o2, 1e-10)
    _close("g = -5 ht", ht, ht2, 1e-10)
    assert st["max_exponent"] <= 80.0 + 1e-9, st
    assert 5.0 * 32 > 88.0   # the reference-row form: e^{G_m - G} over half a chunk


def pin_kda_scalar_reduction(fwd, _scalar=None):
    """Gates equal over the channels give the scalar recurrence: against the
    (separately pinned) scalar oracle."""
    import oracle
    c = _case(71, [9, 0, 70], 85, 1, 2, 6, 5)
    gs = c["g"][..., 0]
    c["g"] = np.repeat(gs[..., None], 6, axis=-1)
    o, ht = _call(fwd, c)
    o2, ht2 = oracle.gdr_fwd(c["q"], c["k"], c["v"], gs, c["beta"], c["cu"], c["h0"], scale=c["scale"])
    _close("scalar reduction o", o, o2, 1e-12)
    _close("scalar reduction ht", ht, ht2, 1e-12)


def pin_kda_literal(fwd, _scalar=None):
    """Against the literal matrix form (GQA, dk != dv, a ghost, tokens outside
    every segment, different gates per channel)."""
    c = _case(72, [13, 0, 40], 60, 2, 4, 5, 3)
    o, ht = _call(fwd, c)
    o2, ht2 = literal(c)
    _close("literal o", o, o2, 1e-12)
    _close("literal ht", ht, ht2, 1e-12)
    assert np.all(o[0, 53:] == 0.0), "o written outside the segments"


def pin_kda_chunked(fwd, _scalar=None):
    """Against the chunk form with a reference row inside each chunk, for chunk
    sizes 1, 4, 16 and 64 (the chunk form the GPU kernel evaluates)."""
    c = _case(73, [150, 1, 64, 65], 280, 1, 2, 8, 8)
    o, ht = _call(fwd, c)
    for C in (1, 4, 16, 64):
        o2, ht2 = chunked(c, C)
        _close("chunked(%d) o" % C, o, o2, 1e-10)
        _close("chunked(%d) ht" % C, ht, ht2, 1e-10)


def pin_kda_pure_decay(fwd, _scalar=None):
    """beta = 0: H_t = diag(exp(G_t)) H_0 with G_t the running sum of g per
    channel, so o_t = scale H_0^T (exp(G_t) o q_t) and ht = diag(exp(G_T)) H_0."""
    c = _case(74, [30], 30, 1, 1, 7, 4, beta_zero=True)
    o, ht = _call(fwd, c)
    G = np.cumsum(c["g"][0, :, 0], axis=0)
    H0 = c["h0"][0, 0]
    o_ref = np.stack([c["scale"] * H0.T @ (np.exp(G[t]) * c["q"][0, t, 0]) for t in range(30)])
    _close("pure decay o", o[0, :, 0], o_ref, 1e-12)
    _close("pure decay ht", ht[0, 0], np.exp(G[-1])[:, None] * H0, 1e-12)


def pin_kda_channel_selective(fwd, _scalar=None):
    """A channel whose gate is -inf-like (very negative) is forgotten at once:
    with beta = 0 its state row is zero after the first token while the other
    rows keep h0 (exp(0) = 1)."""
    c = _case(75, [5], 5, 1, 1, 4, 3, beta_zero=True)
    c["g"][:] = 0.0
    c["g"][0, 0, 0, 2] = -800.0
    _, ht = _call(fwd, c)
    H0 = c["h0"][0, 0]
    assert np.all(ht[0, 0, 2] == 0.0), "channel 2 not forgotten"
    _close("kept channels", np.delete(ht[0, 0], 2, axis=0), np.delete(H0, 2, axis=0), 0.0)


ALL_KDA_PINS = [pin_kda_scalar_reduction, pin_kda_literal, pin_kda_chunked, pin_kda_block_references,
                pin_kda_pure_decay, pin_kda_channel_selective]
