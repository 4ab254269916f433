"""The step's launches (store_kv, extend, plan-driven decode + merge) captured in a HIP graph and
replayed: none of the entry points allocates, clears memory or synchronises, so the step
records as plain kernel nodes.  Every replay, with eager work and synchronisations between
replays, must equal the eager step bit for bit (the kernels are deterministic)."""
import sys

import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def test_step_replays_from_a_graph():
    import torch
    import bench
    _say("graph capture of a scaled-down mixed step")
    st = bench.setup(5, n_requests=48, n_history=96, pool_slots=1 << 18, n_segments=96, max_ctx=6144,
                     min_ctx=512)
    assert st.ext and st.dec
    bench.step(st)
    torch.cuda.synchronize()
    want_ext, want_dec, want_lse = st.out_ext.clone(), st.out_dec.clone(), st.lse_dec.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream, as torch asks
        bench.step(st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bench.step(st)
    torch.cuda.synchronize()

    scratch = torch.empty_like(st.out_ext)
    for i in range(4):
        st.out_ext.zero_()
        st.out_dec.zero_()
        st.lse_dec.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out_ext.view(torch.int16), want_ext.view(torch.int16)), f"replay {i}: extend"
        assert torch.equal(st.out_dec.view(torch.int16), want_dec.view(torch.int16)), f"replay {i}: decode"
        assert torch.equal(st.lse_dec, want_lse), f"replay {i}: lse"
        scratch.copy_(st.out_ext).mul_(2)  # the program's own eager work between replays
        bench.run_decode(st, flat=True)     # an eager launch of another path into the same buffers
        torch.cuda.synchronize()
    del g
