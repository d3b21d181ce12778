"""Parity at the full workload sizes, in the launch configuration bench.py times
(per-layer build + prefill; all-layer decode with the automatic split), on
outputs the oracle can compute one row at a time: sampled query rows of sampled
layers (window, sink, page and last-row edges plus seeded random rows)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.gpu_util import lse_parity, parity, to_bits

sp = pytest.importorskip("sparse_attention_segmentpagetable_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _edge_rows(n, sink, window, page, rng, extra=12):
    cand = {0, 1, sink - 1, sink, sink + 1, window - 1, window, window + 1, sink + window - 1,
            sink + window, sink + window + 1, page - 1, page, page + 1, 2 * page, n // 2,
            n - page - 1, n - page, n - 2, n - 1}
    cand |= set(int(x) for x in rng.integers(0, n, size=extra))
    return np.array(sorted(x for x in cand if 0 <= x < n), dtype=np.int64)


def _check_prefill_rows(spec, layer, b, rows, q, o, lse, k, v, what):
    """q, o: device [T_q, Hq, D] of this layer; k, v: device [T_total, Hkv, D]."""
    kvo, qo = spec.kv_row_offsets()[b], spec.q_row_offsets()[b]
    nb, q0 = spec.seq_len[b], spec.first_query_pos[b]
    idx = torch.as_tensor(qo + rows - q0, device=q.device)
    qb = to_bits(q[idx])
    ob = to_bits(o[idx])
    kb = to_bits(k[kvo:kvo + nb])
    vb = to_bits(v[kvo:kvo + nb])
    ref, ref_lse = OA.attention_rows(spec, layer, b, rows, qb, kb, vb)
    parity(OA.bf16_bits_to_f64(ob), ref, what)
    lse_parity(lse[idx].cpu().numpy(), ref_lse, what)


def test_mistral_layer_prefill_and_decode_fullsize():
    """4 sequences x 8192 tokens, 32 Q / 8 KV heads, D 128, page 64, KV head 0 global,
    1-7 local (sink 4, window 1024); causal prefill plus one decode step."""
    spec = W.mistral_layer("prefill")
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV, workspace=False)
    T, Hq, Hkv, D = spec.total_tokens, 32, 8, 128
    k = W.randn_bf16_device((T + 4, Hkv, D), 2, W.TAG_K, 0, DEV)  # + one decode token per seq
    v = W.randn_bf16_device((T + 4, Hkv, D), 2, W.TAG_V, 0, DEV)
    q = W.randn_bf16_device((T, Hq, D), 2, W.TAG_Q, 0, DEV)
    # prefill reads the first 8192 tokens of each sequence
    kp = torch.cat([k[b * 8193:b * 8193 + 8192] for b in range(4)])
    vpre = torch.cat([v[b * 8193:b * 8193 + 8192] for b in range(4)])
    sp.build(plan, 0, kp, vpre, bufs["table"], bufs["k_pool"], bufs["v_pool"])
    o = torch.empty_like(q)
    lse = torch.empty(T, Hq, dtype=torch.float32, device=DEV)
    sp.prefill(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(D), o, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(201)
    for b in range(4):
        rows = _edge_rows(8192, 4, 1024, 64, rng)
        _check_prefill_rows(spec, 0, b, rows, q, o, lse, kp, vpre, f"mistral prefill seq {b}")
    # decode at position 8192 over the 8193-token cache, decode form
    dspec = W.mistral_layer("decode")
    dplan = sp.Plan(dspec)
    db = dplan.allocate(DEV)
    sp.build(dplan, 0, k, v, db["table"], db["k_pool"], db["v_pool"])
    qd = W.randn_bf16_device((4, Hq, D), 2, W.TAG_Q, 1, DEV)
    od = torch.empty_like(qd)
    lsed = torch.empty(4, Hq, dtype=torch.float32, device=DEV)
    sp.decode(dplan, 0, qd, db["table"], db["k_pool"], db["v_pool"], 1 / np.sqrt(D), od, lsed,
              workspace=db["workspace"])
    torch.cuda.synchronize()
    ref, ref_lse = OA.attention(dspec, 0, to_bits(qd), to_bits(k), to_bits(v))
    parity(OA.bf16_bits_to_f64(to_bits(od)), ref, "mistral decode")
    lse_parity(lsed.cpu().numpy(), ref_lse, "mistral decode")


def test_llama70b_decode_fullsize():
    """80 layers x 8 KV heads (64 Q heads), 15% global, local sink 4 / window 8192,
    page 64; 8 sequences x 32768 tokens; one all-layer decode call. Four layers are
    checked against the oracle (the first two holding global heads among them)."""
    spec = W.llama70b_decode()
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    L, B, N, Hq, Hkv, D = 80, 8, 32768, 64, 8, 128
    glob_layers = [l for l in range(L) if any(spec.kind[l * Hkv + h] == W.GLOBAL for h in range(Hkv))]
    check = sorted({glob_layers[0], glob_layers[1], 37, 79})
    kept = {}
    for l in range(L):
        kd = W.randn_bf16_device((B * N, Hkv, D), 3, W.TAG_K, l, DEV)
        vd = W.randn_bf16_device((B * N, Hkv, D), 3, W.TAG_V, l, DEV)
        sp.build(plan, l, kd, vd, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        if l in check:
            kept[l] = (to_bits(kd), to_bits(vd))
        del kd, vd
    q = W.randn_bf16_device((L, B, Hq, D), 3, W.TAG_Q, 0, DEV)
    o = torch.empty_like(q)
    lse = torch.empty(L, B, Hq, dtype=torch.float32, device=DEV)
    sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(D), o, lse,
              workspace=bufs["workspace"])
    torch.cuda.synchronize()
    for l in check:
        ref, ref_lse = OA.attention(spec, l, to_bits(q[l]), *kept[l])
        parity(OA.bf16_bits_to_f64(to_bits(o[l])), ref, f"llama70b decode layer {l}")
        lse_parity(lse[l].cpu().numpy(), ref_lse, f"llama70b decode layer {l}")


def test_long_prefill_fullsize_sampled_rows():
    """One 131072-token sequence, 64 Q / 8 KV heads, D 128, page 64, 15% global,
    local sink 4 / window 8192; build + prefill per layer as bench.py runs it.
    Two layers (the one with the most global heads and layer 0) are run and
    checked on edge and seeded rows."""
    spec = W.long_prefill()
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV, workspace=False)
    N, Hq, Hkv, D = 131072, 64, 8, 128
    nglob = [sum(spec.kind[l * Hkv + h] == W.GLOBAL for h in range(Hkv)) for l in range(64)]
    layers = sorted({0, int(np.argmax(nglob))})
    rng = np.random.default_rng(401)
    for l in layers:
        q = W.randn_bf16_device((N, Hq, D), 4, W.TAG_Q, l, DEV)
        k = W.randn_bf16_device((N, Hkv, D), 4, W.TAG_K, l, DEV)
        v = W.randn_bf16_device((N, Hkv, D), 4, W.TAG_V, l, DEV)
        o = torch.empty_like(q)
        lse = torch.empty(N, Hq, dtype=torch.float32, device=DEV)
        sp.build(plan, l, k, v, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        sp.prefill(plan, l, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(D), o, lse)
        torch.cuda.synchronize()
        rows = _edge_rows(N, 4, 8192, 64, rng, extra=10)
        _check_prefill_rows(spec, l, 0, rows, q, o, lse, k, v,
                            f"long prefill layer {l} ({nglob[l]} global heads)")
        del q, k, v, o, lse


def test_mixed_varlen_decode_fullsize():
    """32 sequences, log-uniform 2K-128K, 48 layers x 8 KV heads (64 Q heads): 12%
    global, 8% retrieval (seeded 5% index sets, gathered pages), 80% local (sink 4,
    window 4096); one all-layer decode call; three layers checked (all sequences)."""
    spec = W.mixed_varlen_decode()
    plan = sp.Plan(spec)
    bufs = plan.allocate(DEV)
    L, Hq, Hkv, D = 48, 64, 8, 128
    T = spec.total_tokens
    retr_layers = [l for l in range(L) if any(spec.kind[l * Hkv + h] == W.RETRIEVAL for h in range(Hkv))]
    check = sorted({retr_layers[0], 0, 47})
    kept = {}
    for l in range(L):
        kd = W.randn_bf16_device((T, Hkv, D), 5, W.TAG_K, l, DEV)
        vd = W.randn_bf16_device((T, Hkv, D), 5, W.TAG_V, l, DEV)
        sp.build(plan, l, kd, vd, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        if l in check:
            kept[l] = (to_bits(kd), to_bits(vd))
        del kd, vd
    q = W.randn_bf16_device((L, spec.num_seqs, Hq, D), 5, W.TAG_Q, 0, DEV)
    o = torch.empty_like(q)
    lse = torch.empty(L, spec.num_seqs, Hq, dtype=torch.float32, device=DEV)
    sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], 1 / np.sqrt(D), o, lse,
              workspace=bufs["workspace"])
    torch.cuda.synchronize()
    for l in check:
        ref, ref_lse = OA.attention(spec, l, to_bits(q[l]), *kept[l])
        parity(OA.bf16_bits_to_f64(to_bits(o[l])), ref, f"mixed varlen decode layer {l}")
        lse_parity(lse[l].cpu().numpy(), ref_lse, f"mixed varlen decode layer {l}")
