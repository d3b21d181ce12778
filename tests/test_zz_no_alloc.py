"""segpaged_decode_noalloc (the decode entry point that allocates nothing: its
workspace is a library-owned device array) against segpaged_decode, through the
C ABI: identical bits when segpaged_decode gets a workspace of the array's size,
the oracle's bar in any case; two calls in a row, the second smaller (the array
keeps the first call's partials); and ENOSPACE, before any work, for a call whose
partials do not fit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.gpu_util import lse_parity, parity, to_bits, to_dev, to_f64

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(spec, layers):
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    kvs = [W.kv_bits(spec, l) for l in range(spec.num_layers)]
    for l in range(spec.num_layers):
        sp.build(plan, l, to_dev(kvs[l][0]), to_dev(kvs[l][1]), bufs["table"], bufs["k_pool"],
                 bufs["v_pool"])
    qs = [W.q_bits(spec, l) for l in range(spec.num_layers)]
    scale = 1 / np.sqrt(spec.head_dim)
    ws = torch.empty(sp.NOALLOC_SCRATCH_BYTES // 4, dtype=torch.float32, device=DEV)
    for layer in layers:
        q = to_dev(np.stack(qs) if layer < 0 else qs[layer])
        o_ref, o_na = torch.empty_like(q), torch.full_like(q, float("nan"))
        shape = q.shape[:-1]
        l_ref = torch.empty(shape, dtype=torch.float32, device=DEV)
        l_na = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
        sp.decode(plan, layer, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o_ref,
                  l_ref, workspace=ws)
        sp.decode_noalloc(plan, layer, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale,
                          o_na, l_na)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o_na), to_bits(o_ref)), (spec.name, layer)
        assert np.array_equal(l_na.cpu().numpy(), l_ref.cpu().numpy()), (spec.name, layer)
        of, lf = to_f64(o_na), l_na.cpu().numpy()
        for l in (range(spec.num_layers) if layer < 0 else [layer]):
            ref, ref_lse = OA.attention(spec, l, qs[l], *kvs[l], scale=scale)
            got = of[l] if layer < 0 else of
            gl = lf[l] if layer < 0 else lf
            parity(got, ref, f"decode_noalloc {spec.name} L{l} (call layer {layer})")
            lse_parity(gl, ref_lse, f"decode_noalloc {spec.name} L{l}")


def test_decode_noalloc_matches_decode_then_a_smaller_call():
    big = W.llama70b_decode(num_layers=2, seqs=3, n=6000, window=700)
    _run(big, [0, 1, -1])
    small = W.mixed_varlen_decode(seqs=2, num_layers=2, lo=100, hi=900, window=64)
    _run(small, [1, -1])


def test_decode_noalloc_rejects_partials_beyond_its_array():
    spec = W.llama70b_decode(num_layers=4, seqs=8, n=32768, window=8192)
    plan = sp.Plan(spec, decode_split_tokens=64)
    need = plan.sizes.decode_workspace_bytes
    assert need > sp.NOALLOC_SCRATCH_BYTES
    # The call is refused before any launch, so the pools are never read.
    pool = torch.empty(plan.sizes.pool_bytes // 2, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((4, 8, 64, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    table = torch.zeros(plan.sizes.table_int32s, dtype=torch.int32, device=DEV)
    with pytest.raises(sp.SegPagedError) as e:
        sp.decode_noalloc(plan, -1, q, table, pool, pool, 0.1, o)
    assert e.value.status == -3
    torch.cuda.synchronize()
