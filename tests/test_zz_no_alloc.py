"""dsa_sparse_mla_decode_noalloc (static per-GPU scratch, no workspace) against
dsa_sparse_mla_decode (caller workspace), through the C ABI: the same kernels, so the outputs
must agree bit for bit.  Two calls in a row, the second with fewer requests and shorter
contexts, so it reuses scratch that still holds the first call's partials."""
import numpy as np
import pytest
import torch

from synth import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def one_case(d, ctx, seed, k=2048, heads=12):
    print(f"[noalloc] ctx={ctx} k={k} heads={heads} seed={seed}", flush=True)
    cache = W.build_cache(ctx, seed=seed, device="cuda", spare_rows=2)
    dq = W.decode_queries(len(ctx), heads, seed=seed, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    step.run()                               # indices from the real chain, outputs via the workspace
    out2 = torch.full_like(step.out, 7.0)
    lse2 = torch.full_like(step.lse, 7.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d.dsa_sparse_mla_decode_noalloc(step.layout, cache.pool, step.lat_off, cache.ctx_len, step.idx, k, dq.q_mla,
                                    dq.sm_scale, cache.kv_scale, out2, lse2, err)
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0 and int(err.item()) == 0
    assert d.dsa_sparse_mla_decode_workspace_size(len(ctx), heads, k) > 0   # the split path really ran
    assert torch.equal(out2.view(torch.int16), step.out.view(torch.int16))
    assert np.array_equal(lse2.cpu().numpy().view(np.uint32), step.lse.cpu().numpy().view(np.uint32))


def test_noalloc_matches_workspace_call_twice(d):
    one_case(d, [9000, 4096, 2500, 131, 7000, 3000, 6000, 5000], seed=91)
    one_case(d, [3000, 700, 2049], seed=92)


def test_noalloc_limit(d):
    """A call needing more scratch than the static array is refused before any launch."""
    cache = W.build_cache([3000], seed=93, device="cuda", spare_rows=1)
    dq = W.decode_queries(1, 12, seed=93, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=2048)
    q = torch.zeros(1000, 128, 576, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1000, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1000, 128, dtype=torch.float32, device="cuda")
    idx = torch.full((1000, 2048), -1, dtype=torch.int32, device="cuda")
    ctx = torch.full((1000,), 3000, dtype=torch.int32, device="cuda")
    lat_off = torch.full((1000, 47), -1, dtype=torch.int64, device="cuda")  # every buffer sized for the call
    with pytest.raises(d.DsaError) as e:
        d.dsa_sparse_mla_decode_noalloc(step.layout, cache.pool, lat_off, ctx, idx, 2048, q, 0.1, 1.0, out, lse)
    assert e.value.status == d.DSA_ERR_SCRATCH_LIMIT
