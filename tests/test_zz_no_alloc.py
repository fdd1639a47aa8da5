"""The allocation-free paged decode (fa_decode_paged_gqa_static, through the C
ABI) against the workspace entry point (fa_decode_paged_gqa) on the same
inputs: two calls in a row, the second with a smaller problem, for grouped
and ungrouped heads.  Both run the same kernels, so the outputs must be
identical bit for bit; the oracle bounds them as well."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import BF16_MAX, BF16_MEAN, LSE_MAX, check, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _lib():
    import exact_attention_fwd_amd as fa
    return fa.lib()


def _run_both(p):
    L = _lib()
    q, pool, bt, sl = (t.to(DEV) for t in (p.q, p.kv_pool, p.block_table, p.seq_lens))
    S, H, d = q.shape
    P, _, page, Hkv, _ = pool.shape
    mb = bt.shape[1]
    scale = 1 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    o_ws, o_st = torch.empty_like(q), torch.empty_like(q)
    l_ws = torch.empty(S, H, dtype=torch.float32, device=DEV)
    l_st = torch.empty(S, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(int(L.fa_decode_workspace_bytes(S, H, d, mb)), dtype=torch.uint8, device=DEV)
    print(f"[static decode] S={S} H={H} Hkv={Hkv} d={d} max_blocks={mb}", flush=True)
    rc = L.fa_decode_paged_gqa(S, H, Hkv, d, page, P, mb, q.data_ptr(), pool.data_ptr(), bt.data_ptr(),
                               sl.data_ptr(), o_ws.data_ptr(), l_ws.data_ptr(), scale, ws.data_ptr(),
                               ws.numel(), stream)
    assert rc == 0
    rc = L.fa_decode_paged_gqa_static(S, H, Hkv, d, page, P, mb, q.data_ptr(), pool.data_ptr(), bt.data_ptr(),
                                      sl.data_ptr(), o_st.data_ptr(), l_st.data_ptr(), scale, stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(o_st, o_ws), "static-scratch O differs from the workspace entry point"
    assert torch.equal(l_st, l_ws), "static-scratch LSE differs from the workspace entry point"
    ro, rl = oracle.decode_paged(p.q, p.kv_pool, p.block_table, p.seq_lens, scale=scale, page_size=page)
    check("static decode O", to64(o_st), ro, BF16_MAX, BF16_MEAN)
    check("static decode LSE", to64(l_st), rl, LSE_MAX)


@pytest.mark.parametrize("Hkv", [32, 8])
def test_static_decode_matches_workspace_decode_twice(Hkv):
    # first the full decode configuration (8 sequences, 32 query heads, d = 128,
    # lengths 1024..8192), then a smaller problem that reuses less of the scratch
    w = workloads.CONFIGS["c4"]
    _run_both(workloads.workload_inputs(w, Hkv=Hkv, poison=True, spare_pages=4))
    _run_both(workloads.paged_inputs(num_seqs=3, H=16, Hkv=Hkv // 2, d=128, max_blocks=5, seed=71 + Hkv,
                                     seq_lens=[1, 300, 1200], poison=True, spare_pages=2))


def test_static_decode_refuses_oversized_problem():
    L = _lib()
    fake = 0x1000  # never dereferenced: refused before any launch
    rc = L.fa_decode_paged_gqa_static(8, 32, 8, 128, 256, 4, 64, fake, fake, fake, fake, fake, fake, 0.1, None)
    assert rc == 6
