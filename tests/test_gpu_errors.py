"""GPU tests of the failure paths: a forced launch failure, the opt-in
device-side check of cu_seqlens, a hand-off wait that gives up (forced from
the host with a tiny poll limit, so every kernel still ends normally), and
calls that allocate nothing once the workspace ring exists.

Every condition here is forced from the host; no kernel faults or hangs."""
import numpy as np
import pytest

import gdr_inputs as gi
from gpu_helpers import compare, dev, np64, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    assert torch.cuda.is_available()
    gdr.library()
    yield
    gdr.debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 0)
    gdr.debug_set(gdr.GDR_DEBUG_CHECK_CU, 0)
    gdr.debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, -1)
    gdr.device_status(clear=True)


def small_case(seed=21):
    w = gi.Workload("errors", 1, 0, 2, 4, 128, 128, "bf16", seg_range=(1, 2), n_segments=4, seed=seed)
    return gi.generate(w, lengths=[70, 0, 200, 33])


def test_forced_launch_failure_leaves_outputs_untouched():
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    say("forced launch failure: forward, cumsum, decode")
    d = small_case()
    t = to_device(d)
    o = torch.full((1, 303, 4, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    ht = torch.full((4, 4, 128, 128), -2.0, device="cuda")
    gdr.debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 1)
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"], o=o, ht=ht)
    assert e.value.status == -7 and "forward kernel" in e.value.message
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(ht == -2.0), "a failed launch touched an output"
    # the hook is consumed: the next call runs and is correct
    o2, ht2 = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"],
                            o=o, ht=ht)
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(d)
    real = [0, 2, 3]
    compare(np64(o2), np64(ht2[real]), o_ref, ht_ref[real], "after a forced failure")
    # other entry points report the same way
    gdr.debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 1)
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_local_cumsum(t["g"], t["cu"])
    assert e.value.status == -7 and "cumsum" in e.value.message
    gdr.debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 1)
    h = torch.zeros((2, 4, 128, 128), device="cuda")
    with pytest.raises(gdr.GdrError) as e:
        gdr.decode_step(t["q"][0, :2], t["k"][0, :2], t["v"][0, :2], t["g"][0, :2], t["beta"][0, :2], h)
    assert e.value.status == -7 and "decode kernel" in e.value.message
    gdr.debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 0)


@pytest.mark.parametrize("bad,msg", [
    ([5, 70, 70, 270, 303], "cu[0] must be 0"),
    ([0, 70, 60, 270, 303], "must not decrease (cu[1] = 70 > cu[2] = 60)"),
    ([0, 70, 70, 270, 300], "must equal the 303 tokens"),
])
def test_cu_content_check(bad, msg):
    """With the check on, invalid cu_seqlens content is reported before any
    work is enqueued; valid content gives the same results as without it."""
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    say("cu content check:", bad)
    d = small_case()
    t = to_device(d)
    o = torch.full((1, 303, 4, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    ht = torch.full((4, 4, 128, 128), -2.0, device="cuda")
    cu_bad = dev(np.array(bad, dtype=np.int32), "i32")
    gdr.debug_set(gdr.GDR_DEBUG_CHECK_CU, 1)
    try:
        with pytest.raises(gdr.GdrError) as e:
            gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_bad, t["h0"], scale=d["scale"], o=o, ht=ht)
        assert e.value.status == -1 and msg in e.value.message, e.value.message
        torch.cuda.synchronize()
        assert torch.all(o == 3.0) and torch.all(ht == -2.0)
        with pytest.raises(gdr.GdrError) as e:
            gdr.chunk_local_cumsum(t["g"], cu_bad)
        assert e.value.status == -1 and msg in e.value.message
        o1, ht1 = run_gpu(t, d["scale"])
    finally:
        gdr.debug_set(gdr.GDR_DEBUG_CHECK_CU, 0)
    o2, ht2 = run_gpu(t, d["scale"])
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_wait_give_up_is_reported():
    """A poll limit of 0 makes the kernel's hand-off waits give up at once:
    the call still ends, the device status word says so, and ht is NaN.
    With the default limit the same call is clean again."""
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    say("forced wait give-up")
    d = small_case(seed=23)
    t = to_device(d)
    assert gdr.device_status(clear=True) == 0, "status word set by an earlier test"
    gdr.debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, 0)
    try:
        o, ht = run_gpu(t, d["scale"])
        bits = gdr.device_status(clear=True)
    finally:
        gdr.debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, -1)
    say("status bits after forced give-up:", bits)
    assert bits & gdr.GDR_DEVSTAT_WAIT_TIMEOUT
    real = [0, 2, 3]
    assert bool(torch.isnan(ht[real]).any()), "a give-up must poison ht"
    o, ht = run_gpu(t, d["scale"])
    assert gdr.device_status() == 0
    o_ref, ht_ref = run_oracle(d)
    compare(np64(o), np64(ht[real]), o_ref, ht_ref[real], "default poll limit")


def test_no_allocation_after_first_call():
    """Once the first call has created the workspace ring, further calls (varlen
    forward, checkpoints, cumsum) take no device memory: free memory is unchanged
    over 40 calls."""
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    say("no allocation after the first call")
    d = gi.generate(gi.WORKLOADS["varlen8_ghost8_H32_d128"])
    t = to_device(d)
    N = len(d["cu_seqlens"]) - 1
    o = torch.empty((1, t["q"].shape[1], 32, 128), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((N, 32, 128, 128), device="cuda")
    G = torch.empty(t["g"].shape, device="cuda")
    gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"], o=o, ht=ht)
    gdr.chunk_local_cumsum(t["g"], t["cu"], out=G)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(20):
        gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], scale=d["scale"], o=o, ht=ht)
        gdr.chunk_local_cumsum(t["g"], t["cu"], out=G)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    say("free device memory before / after: %d / %d" % (free0, free1))
    assert free1 == free0
