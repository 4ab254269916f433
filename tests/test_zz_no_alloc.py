"""The allocation-free decode entry point (rs_decode_attention_noalloc) against the
workspace entry point (rs_decode_attention) it shares its kernels with: bit-identical
outputs and lse, plan mode and flat mode, on two calls in a row with the smaller batch
second (the static scratch keeps the first call's contents), and a batch whose workspace
exceeds the scratch refused before anything runs."""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def test_noalloc_decode_matches_the_workspace_entry_point():
    import torch
    import bench
    import radix_tree_prefix_amd as rs
    assert torch.cuda.is_available()
    for cfg in (4, 2):                       # the second call has the smaller batch
        _say(f"noalloc decode, config {cfg}")
        st = bench.setup(cfg)
        bench.run_store(st)
        for flat in (False, True):
            bench.run_decode(st, flat=flat)
            out = torch.full_like(st.out_dec, float("nan"))
            lse = torch.full_like(st.lse_dec, float("nan"))
            rs.decode_attention_noalloc(st.q_dec, st.k_pool, st.v_pool, st.table_dec, st.dec_seq_lens, st.max_seq,
                                        st.wl.sm_scale, out, plan=None if flat else st.plan,
                                        plan_dev=None if flat else st.plan_dev, lse=lse)
            torch.cuda.synchronize()
            assert torch.equal(out, st.out_dec), (cfg, flat)
            assert torch.equal(lse, st.lse_dec), (cfg, flat)
            # and, as every decode path, against the oracle (first and last request)
            got = out.float().cpu().numpy()
            for i in (0, len(st.dec) - 1):
                r = st.dec[i]
                k, v = st.vals.kv_rows(r.tokens, 0, r.seq_len)
                q = st.vals.q_rows(r.tokens, r.seq_len - 1, r.seq_len)
                o, _ = oracle.attend(q, k, v, [r.seq_len - 1], st.wl.sm_scale)
                assert np.abs(got[i] - o[0]).max() <= 2e-2, (cfg, flat, i)
        del st
        torch.cuda.empty_cache()


def test_noalloc_decode_refuses_a_batch_beyond_the_scratch():
    import torch
    import radix_tree_prefix_amd as rs
    _say("noalloc decode: oversize batch refused")
    B, Hq, Hkv, D, L = 64, 64, 8, 128, 65536         # flat workspace: 512 MiB
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((B, L), dtype=torch.int32, device="cuda")
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(rs.RsError) as e:
        rs.decode_attention_noalloc(q, pool, pool, table, seq, L, 0.1, out)
    assert "static scratch" in str(e.value)
