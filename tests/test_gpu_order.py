"""GPU: the dispatch order of the forward pass (gdr_dispatch_order) against a
plain CPU model of the same schedule, bit for bit.

Model: `groups` identical machines; sequence n keeps one busy for
w_n = ceil(L_n / 64) + 1 units (length 0: w = 0, scheduled last); work-groups
start in list order on the machine that frees first (ties: lowest index).
Longest first (ties by index) is the baseline; first-fit-decreasing packing
at the smallest fitting capacity among up to 64 evenly spaced candidates
below the baseline makespan, replayed as a list (the machine that frees
first takes the next item of its bin, else the largest item left), replaces
it only when its makespan is smaller.
"""
import numpy as np
import pytest

import gdr_inputs as gi
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _weights(lens):
    return [((L + 63) // 64 + 1) if L > 0 else 0 for L in lens]


def _list_makespan(ws, m):
    fin = [0] * m
    for x in ws:
        b = min(range(m), key=lambda i: (fin[i], i))
        fin[b] += x
    return max(fin) if ws else 0


def _first_fit(ws, m, cap):
    load, bins = [0] * m, []
    for x in ws:
        b = next((i for i in range(m) if load[i] + x <= cap), -1)
        if b < 0:
            return None
        load[b] += x
        bins.append(b)
    return bins


def model_order(lens, m):
    n = len(lens)
    w = _weights(lens)
    idx = sorted(range(n), key=lambda i: (-w[i], i))
    sw = [w[i] for i in idx]
    k = sum(1 for x in sw if x > 0)
    mk_lpt = _list_makespan(sw[:k], m)
    lo = max(-(-sum(sw[:k]) // m), sw[0] if k else 0)
    hi = mk_lpt - 1
    if k > m and hi >= lo:
        step = (hi - lo + 64) // 64
        caps = [lo + j * step for j in range(64) if lo + j * step <= hi]
        best = next((c for c in caps if _first_fit(sw[:k], m, c) is not None), None)
        if best is not None:
            bins = _first_fit(sw[:k], m, best)
            fin, left, out = [0] * m, set(range(k)), []
            for _ in range(k):
                bm = min(range(m), key=lambda i: (fin[i], i))
                own = [i for i in sorted(left) if bins[i] == bm]
                pick = own[0] if own else min(left)
                left.discard(pick)
                fin[bm] += sw[pick]
                out.append(pick)
            if max(fin) < mk_lpt:
                return [idx[i] for i in out] + idx[k:]
    return idx


def _gpu_order(lens, m):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    order = gdr.dispatch_order(torch.from_numpy(cu).cuda(), m)
    torch.cuda.synchronize()
    return order.cpu().numpy().tolist()


def test_dispatch_order_matches_model():
    rng = np.random.default_rng(7)
    say("dispatch order: 300 random cases against the model")
    improved = 0
    for case in range(300):
        m = int(rng.integers(1, 17))
        n = int(rng.integers(1, 65))
        top = int(rng.choice([200, 4000, 9000]))
        lens = rng.integers(1, top, size=n)
        lens[rng.random(n) < 0.1] = 0
        lens = [int(x) for x in lens]
        got = _gpu_order(lens, m)
        want = model_order(lens, m)
        assert sorted(got) == list(range(n)), (case, got)
        assert got == want, (case, m, lens, got, want)
        w = _weights(lens)
        lpt = sorted(range(n), key=lambda i: (-w[i], i))
        mk = _list_makespan([w[i] for i in got if w[i] > 0], m)
        mk_lpt = _list_makespan([w[i] for i in lpt if w[i] > 0], m)
        assert mk <= mk_lpt
        improved += mk < mk_lpt
    say("  packed order better than longest first in %d of 300" % improved)
    assert improved > 0


def test_dispatch_order_packed64k_segments():
    w = gi.WORKLOADS["packed64k_gqa_Hk16_Hv32_d128"]
    lens = gi.draw_lengths(np.random.Generator(np.random.PCG64(w.seed)), w)
    got = _gpu_order(lens, 8)
    assert got == model_order(lens, 8)
    ws = _weights(lens)
    lpt = sorted(range(len(lens)), key=lambda i: (-ws[i], i))
    mk, mk_lpt = _list_makespan([ws[i] for i in got], 8), _list_makespan([ws[i] for i in lpt], 8)
    say("packed 64k segments, 8 machines: model makespan %d (longest first %d)" % (mk, mk_lpt))
    assert mk < mk_lpt
