"""The no-allocation forward entry point (gdr_chunk_fwd_noalloc) against
gdr_chunk_fwd, through the C ABI: two calls in a row, the second on a smaller
input, each bit-identical to the allocating entry point and within the
forward tolerances of the oracle; no device memory is taken; too many
sequences are rejected with a message."""
import numpy as np
import pytest

import gdr_inputs as gi
from gpu_helpers import compare, np64, run_oracle, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    assert torch.cuda.is_available()
    gdr.library()


def _both(d):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    t = to_device(d)
    B, T = t["q"].shape[:2]
    N = (t["cu"].shape[0] - 1) if t["cu"] is not None else B
    hv, dv = t["v"].shape[2], t["v"].shape[3]
    dk = t["q"].shape[3]
    o_a = torch.full((B, T, hv, dv), 7.0, dtype=t["q"].dtype, device="cuda")
    ht_a = torch.full((N, hv, dk, dv), -5.0, device="cuda")
    o_b, ht_b = o_a.clone(), ht_a.clone()
    gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"], o=o_a, ht=ht_a)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    gdr.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"],
                          o=o_b, ht=ht_b)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the no-allocation entry point took device memory"
    return o_a, ht_a, o_b, ht_b


def test_noalloc_two_calls_second_smaller():
    import torch
    w = gi.WORKLOADS["varlen8_ghost8_H32_d128"]
    first = gi.generate(w)
    small = gi.random_lengths_case(seed=31, n_real=3, lo=1, hi=150, ghost_slots=2, hk=2, hv=4, d=128)
    for name, d in (("varlen 8 + 8 ghosts, H=32", first), ("smaller: 3 segments + 2 ghosts, Hk=2, Hv=4", small)):
        say("no-alloc:", name)
        o_a, ht_a, o_b, ht_b = _both(d)
        assert torch.equal(o_a, o_b), "%s: o differs from gdr_chunk_fwd" % name
        assert torch.equal(ht_a, ht_b), "%s: ht differs from gdr_chunk_fwd" % name
        cu = d["cu_seqlens"]
        real = [i for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
        o_ref, ht_ref = run_oracle(d)
        compare(np64(o_b), np64(ht_b[real]), o_ref, ht_ref[real], "no-alloc " + name)


def test_noalloc_fixed_length_rows():
    import torch
    d = gi.generate(gi.WORKLOADS["tiny_fp32_T128_H2_d64"])
    say("no-alloc: fixed-length rows, fp32, d=64")
    o_a, ht_a, o_b, ht_b = _both(d)
    assert torch.equal(o_a, o_b) and torch.equal(ht_a, ht_b)


def test_noalloc_rejects_too_many_sequences():
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    say("no-alloc: 16381 sequences rejected")
    n = 16381
    cu = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    q = torch.zeros((1, 0, 1, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, 0, 1), dtype=torch.bfloat16, device="cuda")
    ht = torch.zeros((n, 1, 64, 64), device="cuda")
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_fwd_noalloc(q, q, q, g, g, cu, None, ht=ht)
    assert e.value.status == -2 and "at most 16380 sequences" in e.value.message
