"""Pins for the fp64 backward oracle: checks that do not trust its own formulas.

Each ``pin_bwd_*`` function takes a backward callable with the signature of
``oracle.gdr_bwd`` (and, for the finite-difference pin, the forward
``oracle.gdr_fwd``, itself pinned by ``oracle_pins.py``) and raises
``AssertionError`` on a disagreement.  ``test_oracle_bwd_pins.py`` runs them on
the oracle; ``test_oracle_mutants.py`` runs them on broken copies of it.

The derivative being pinned is that of the gated delta rule forward pass
(``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``,
``o_t = scale S_t q_t``, state returned as ``H = S^T``), the op whose backward
"Findings from integrating FlashQLA's Blackwell GDN kernels into a JAX trainer"
discusses (opening summary, items 3-4), for the scalar loss
``L = sum(o * do) + sum(ht * dht)``.
"""
from __future__ import annotations

import numpy as np

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _case(seed, lengths, T, Hk, Hv, dk, dv, with_h0=True, beta_zero=False):
    """Small fp64 inputs: q, k unit-norm, v ~ N(0,1), g = logsigmoid, beta = sigmoid."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    assert cu[-1] <= T
    q = rng.standard_normal((1, T, Hk, dk))
    k = rng.standard_normal((1, T, Hk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, Hv, dv))
    x = rng.standard_normal((1, T, Hv))
    g = -np.log1p(np.exp(-x))
    beta = np.zeros((1, T, Hv)) if beta_zero else 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, Hv))))
    n = len(lengths)
    h0 = 0.5 * rng.standard_normal((n, Hv, dk, dv)) if with_h0 else None
    do = rng.standard_normal((1, T, Hv, dv))
    dht = rng.standard_normal((n, Hv, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, h0=h0, do=do, dht=dht, scale=0.7)


def _call(bwd, c, **kw):
    return bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], cu_seqlens=c["cu"], h0=c["h0"],
               dht=c["dht"], scale=c["scale"], **kw)


def _close(name, got, ref, rtol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, "%s: shape %s vs %s" % (name, got.shape, ref.shape)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    mag = max(1.0, float(np.abs(ref).max())) if ref.size else 1.0
    assert err <= rtol * mag, "%s: max err %.3e (ref max %.3e)" % (name, err, mag)


def _torch_grads(c):
    """Reverse-mode derivative by torch.autograd of the matrix recurrence,
    written here in its literal form (S is dv x dk, S <- a S (I - b k k^T) + b v k^T)."""
    import torch
    t = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True)
         for n in ("q", "k", "v", "g", "beta")}
    h0 = None if c["h0"] is None else torch.tensor(c["h0"], dtype=torch.float64, requires_grad=True)
    do = torch.tensor(c["do"], dtype=torch.float64)
    dht = torch.tensor(c["dht"], dtype=torch.float64)
    cu = c["cu"]
    Hk, Hv = c["q"].shape[2], c["v"].shape[2]
    dk, dv = c["q"].shape[3], c["v"].shape[3]
    loss = torch.zeros((), dtype=torch.float64)
    eye = torch.eye(dk, dtype=torch.float64)
    for n in range(len(cu) - 1):
        if cu[n + 1] == cu[n]:
            continue
        for h in range(Hv):
            hk = h // (Hv // Hk)
            S = torch.zeros(dv, dk, dtype=torch.float64) if h0 is None else h0[n, h].T
            for s in range(cu[n], cu[n + 1]):
                kt, qt, vt = t["k"][0, s, hk], t["q"][0, s, hk], t["v"][0, s, h]
                a, b = torch.exp(t["g"][0, s, h]), t["beta"][0, s, h]
                S = a * S @ (eye - b * torch.outer(kt, kt)) + b * torch.outer(vt, kt)
                loss = loss + c["scale"] * torch.dot(S @ qt, do[0, s, h])
            loss = loss + torch.sum(S.T * dht[n, h])
    loss.backward()
    out = {("d" + n): (t[n].grad.numpy() if t[n].grad is not None else np.zeros(c[n].shape))
           for n in ("q", "k", "v", "g", "beta")}
    out["dh0"] = h0.grad.numpy() if h0 is not None and h0.grad is not None else None
    return out


def pin_bwd_autograd(bwd, fwd=None):
    """Every gradient element against torch.autograd of the literal recurrence:
    GQA (2 v-heads per q/k head), dk != dv, a segment longer than one 64-token
    chunk, a ghost segment, tokens outside every segment, an initial state."""
    c = _case(11, [70, 0, 45], 120, 1, 2, 5, 3)
    got = _call(bwd, c)
    ref = _torch_grads(c)
    for n in GRADS:
        _close("autograd " + n, got[n], ref[n], 1e-9)
    # tokens 115..119 belong to no segment
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(got[n][0, 115:] == 0.0), "%s written outside the segments" % n


def pin_bwd_autograd_zero_state(bwd, fwd=None):
    """As above with no initial state and fixed-length rows (B = 2)."""
    c = _case(12, [40], 40, 2, 2, 4, 4, with_h0=False)
    got = _call(bwd, c)
    ref = _torch_grads(c)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        _close("autograd(h0=None) " + n, got[n], ref[n], 1e-9)
    # the gradient of the zero initial state is still the adjoint of the state
    assert got["dh0"].shape == (1, 2, 4, 4) and np.abs(got["dh0"]).max() > 0


def pin_bwd_finite_differences(bwd, fwd):
    """Directional derivatives against central differences of the forward
    oracle: L(x + e u) - L(x - e u) over 2e for a random direction u per input."""
    c = _case(13, [9, 66], 80, 1, 2, 4, 3)
    got = _call(bwd, c)
    rng = np.random.Generator(np.random.PCG64(99))

    def loss(cc):
        o, ht = fwd(cc["q"], cc["k"], cc["v"], cc["g"], cc["beta"], cc["cu"], cc["h0"],
                    scale=cc["scale"])
        return float(np.sum(o * cc["do"]) + np.sum(ht * cc["dht"]))

    eps = 1e-5
    for name in ("q", "k", "v", "g", "beta", "h0"):
        u = rng.standard_normal(c[name].shape)
        cp = dict(c); cp[name] = c[name] + eps * u
        cm = dict(c); cm[name] = c[name] - eps * u
        fd = (loss(cp) - loss(cm)) / (2 * eps)
        an = float(np.sum(got["d" + name] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
            "finite differences d%s: %.10f vs %.10f" % (name, fd, an)


def pin_bwd_no_write_closed_form(bwd, fwd=None):
    """beta = 0: the state only decays, H_t = exp(G_t) H0 with G_t the running
    sum of g.  Then, with A_t = exp(G_T - G_t) dht + scale sum_{s>=t} exp(G_s - G_t) q_s do_s^T
    the adjoint of H_t:  dq_t = scale exp(G_t) H0 do_t,  dk = dv = 0,
    dbeta_t = k_t^T A_t (v_t - exp(G_t) H0^T k_t),
    dg_t = sum_{s>=t} scale exp(G_s) q_s^T H0 do_s + exp(G_T) <H0, dht>,
    dh0 = sum_t scale exp(G_t) q_t do_t^T + exp(G_T) dht."""
    c = _case(14, [23], 23, 1, 1, 3, 4, beta_zero=True)
    got = _call(bwd, c)
    q, k, v, g, do = c["q"][0, :, 0], c["k"][0, :, 0], c["v"][0, :, 0], c["g"][0, :, 0], c["do"][0, :, 0]
    H0, dht, sc = c["h0"][0, 0], c["dht"][0, 0], c["scale"]
    T = q.shape[0]
    G = np.cumsum(g)
    dq = np.stack([sc * np.exp(G[t]) * H0 @ do[t] for t in range(T)])
    _close("closed dq", got["dq"][0, :, 0], dq, 1e-12)
    _close("closed dk", got["dk"], np.zeros_like(got["dk"]), 1e-12)
    _close("closed dv", got["dv"], np.zeros_like(got["dv"]), 1e-12)
    contrib = np.array([sc * np.exp(G[s]) * q[s] @ H0 @ do[s] for s in range(T)])
    tail = np.exp(G[-1]) * np.sum(H0 * dht)
    dg = np.array([contrib[t:].sum() + tail for t in range(T)])
    _close("closed dg", got["dg"][0, :, 0], dg, 1e-12)
    db = []
    for t in range(T):
        A = np.exp(G[-1] - G[t]) * dht + sum(sc * np.exp(G[s] - G[t]) * np.outer(q[s], do[s])
                                             for s in range(t, T))
        Hprev = np.exp(G[t - 1]) * H0 if t > 0 else H0
        db.append(k[t] @ A @ (v[t] - np.exp(g[t]) * Hprev.T @ k[t]))
    _close("closed dbeta", got["dbeta"][0, :, 0], np.array(db), 1e-12)
    dh0 = sum(sc * np.exp(G[t]) * np.outer(q[t], do[t]) for t in range(T)) + np.exp(G[-1]) * dht
    _close("closed dh0", got["dh0"][0, 0], dh0, 1e-12)


def pin_bwd_packing(bwd, fwd=None):
    """Packing invariance: the gradients of a packed batch (with ghosts in the
    middle and at the end) equal those of each segment run alone; ghost rows
    of dh0 keep the caller's bytes."""
    lengths = [5, 0, 67, 30, 0]
    c = _case(15, lengths, 102, 1, 2, 4, 4)
    sentinel = np.full(c["dht"].shape, 7.25)
    got = _call(bwd, c, dh0_init=sentinel)
    cu = c["cu"]
    for n, L in enumerate(lengths):
        if L == 0:
            assert np.all(got["dh0"][n] == 7.25), "ghost %d: dh0 written" % n
            continue
        a, b = cu[n], cu[n + 1]
        one = dict(q=c["q"][:, a:b], k=c["k"][:, a:b], v=c["v"][:, a:b], g=c["g"][:, a:b],
                   beta=c["beta"][:, a:b], do=c["do"][:, a:b], cu=np.array([0, L]),
                   h0=c["h0"][n:n + 1], dht=c["dht"][n:n + 1], scale=c["scale"])
        r = _call(bwd, one)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            _close("packed %s seg %d" % (name, n), got[name][:, a:b], r[name], 1e-12)
        _close("packed dh0 seg %d" % n, got["dh0"][n:n + 1], r["dh0"], 1e-12)


ALL_BWD_PINS = [pin_bwd_autograd, pin_bwd_autograd_zero_state, pin_bwd_finite_differences,
                pin_bwd_no_write_closed_form, pin_bwd_packing]
