"""The library's reusable workspaces: calls interleaved on two streams (more
calls than workspace buffers, different segment layouts so the dispatch orders
differ) give bit-identical results to the same calls made one at a time."""
import numpy as np
import pytest

from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


def test_workspace_ring_two_streams():
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    import gdr_inputs
    cases = [gdr_inputs.random_lengths_case(200 + i, n_real=5, lo=1, hi=400, ghost_slots=2, hk=2, hv=8, d=128)
             for i in range(2)]
    ts = [to_device(d) for d in cases]

    def call(t, d, stream=None):
        o = torch.zeros_like(t["v"])
        ht = torch.zeros((t["cu"].shape[0] - 1, t["v"].shape[2], 128, 128), device="cuda")
        if stream is None:
            gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"], o=o, ht=ht)
        else:
            with torch.cuda.stream(stream):
                gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"],
                              o=o, ht=ht)
        return o, ht

    ref = [call(t, d) for t, d in zip(ts, cases)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(12):   # 24 calls over 8 workspace buffers
        for i in range(2):
            outs.append((i, call(ts[i], cases[i], streams[i])))
    torch.cuda.synchronize()
    for i, (o, ht) in outs:
        assert torch.equal(o, ref[i][0]) and torch.equal(ht, ref[i][1]), "stream %d result differs" % i
    say("24 interleaved calls on two streams: bit-identical")
