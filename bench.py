"""SegPagedAttention throughput on one MI355X.

One step is one pass of the whole hot path:
  prefill leg  long-prefill workload: one 131072-token sequence, 64 layers x
               (64 Q / 8 KV heads, D 128, page 64, 15% global heads, local
               sink 4 / window 8192); per layer segpaged_build (prefill form,
               dense K/V -> pages) then segpaged_prefill
  decode leg   Llama-3.3-70B-shaped decode: 8 sequences x 32768 tokens, 80
               layers (64 Q / 8 KV heads, 15% global, local sink 4 / window
               8192, page 64); one segpaged_decode over all 80 layers
               (split-K partials + combine). The decode-form cache is built
               once before timing (KV-write time).
Inputs are seeded N(0,1) bf16, resident in HBM before timing.

Prints one JSON line: value = prefill tokens per second of the whole step;
decode KV GB/s, rooflines of the prefill and decode kernels (HIP events on the
launch stream), the oracle's CPU rate on a bounded sample, and the dense-mask
torch SDPA comparison on the same GPU.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SegPaged prefill tok/s & decode KV GB/s (% of peak) at 32K/128K vs dense-mask"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFS = 2500.0         # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--prefill-layers", type=int, default=64)
    ap.add_argument("--prefill-n", type=int, default=131072)
    ap.add_argument("--decode-layers", type=int, default=80)
    ap.add_argument("--decode-n", type=int, default=32768)
    ap.add_argument("--decode-reps", type=int, default=20)
    ap.add_argument("--distinct", type=int, default=8,
                    help="distinct Q and dense K/V tensors the prefill layers cycle through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the mixed-length decode and Mistral-layer figures")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise pass (the FETCH/WRITE_SIZE scale reference)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script into the traffic file")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc run with the MFMA counters into its summary")
    return ap.parse_args()


KERNELS_SRC = os.path.join(ROOT, "sparse_attention_segmentpagetable_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_decode.json")
COPY_BYTES = 1 << 30


def _to_f64(t):
    """A device tensor as float64 on the host (bf16 widens exactly)."""
    return t.double().cpu().numpy()


def _cos(a, b):
    nrm = float(np.linalg.norm(a) * np.linalg.norm(b))
    return float(np.dot(a.ravel(), b.ravel()) / nrm) if nrm > 0 else float(np.array_equal(a, b))


def _acc(got, ref, **extra):
    """Agreement of two outputs [..., heads, D]: max |difference|, cosine over all
    elements and the smallest cosine of a single query head (axis -2)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g2 = np.moveaxis(got, -2, 0).reshape(got.shape[-2], -1)
    r2 = np.moveaxis(ref, -2, 0).reshape(ref.shape[-2], -1)
    out = {"max_abs_err": float(np.max(np.abs(got - ref))) if got.size else 0.0,
           "cos": round(_cos(got, ref), 8),
           "min_head_cos": round(min(_cos(g2[h], r2[h]) for h in range(len(g2))), 8),
           "elements": int(got.size)}
    out.update(extra)
    return out


def _merge_acc(parts):
    """One record from several _acc records: worst error and smallest cosines."""
    if not parts:
        return None
    return {"max_abs_err": max(p["max_abs_err"] for p in parts),
            "min_cos": min(p["cos"] for p in parts),
            "min_head_cos": min(p["min_head_cos"] for p in parts),
            "elements": sum(p["elements"] for p in parts), "checks": len(parts)}


def _kv_tokens(plan, spec, layer=-1):
    """Keys the cache stores against a dense cache of the same tokens: every layer
    and KV head keeping all N_b (what the dense-mask path holds)."""
    st = plan.stats(layer)
    nl = spec.num_layers if layer < 0 else 1
    dense = nl * spec.num_kv_heads * sum(spec.seq_len)
    return {"dense_tokens": int(dense), "stored_tokens": int(st["retained_tokens"]),
            "stored_frac": round(st["retained_tokens"] / dense, 4),
            "saving": round(1 - st["retained_tokens"] / dense, 4),
            "page_slots_frac": round(st["pages"] * spec.page_size / dense, 4),
            "decode_row_keys_frac": round(st["decode_tokens"] / dense, 4)}


def kernels_hash():
    import hashlib
    return hashlib.sha256(open(KERNELS_SRC, "rb").read()).hexdigest()[:16]


def summarize_pmc(fetch_dir, write_dir):
    """HBM bytes per launch of the prefill and decode kernels from rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), each scaled by the ratio of
    the plain copy's known bytes to what the same counter read for it."""
    import csv
    import glob
    import re

    def load(d, counter):
        per, grids = {}, {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                nm = r["Kernel_Name"]
                m = re.search(r"\b(prefill_kernel|decode_partial_kernel|decode_combine_kernel|"
                              r"build_kernel)<\d+[,>]", nm)
                key = m.group(1) if m else ("copy" if "neg_kernel" in nm else None)
                if key:
                    per.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
                    grids.setdefault(key, []).append(int(r["Grid_Size"]))
        # decode: the all-layer call (the largest grid), not the one-layer launches
        for key in ("decode_partial_kernel", "decode_combine_kernel"):
            if key in per:
                g = max(grids[key])
                per[key] = [v for v, gg in zip(per[key], grids[key]) if gg == g]
        return per
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / (sum(fetch["copy"]) / len(fetch["copy"]))
    w_scale = COPY_BYTES / (sum(write["copy"]) / len(write["copy"]))
    out = {"kernels_sha256_16": kernels_hash(), "copy_bytes": COPY_BYTES,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "per_launch": {}}
    for k in ("prefill_kernel", "decode_partial_kernel", "decode_combine_kernel", "build_kernel"):
        if k in fetch and k in write:
            fb = sum(fetch[k]) / len(fetch[k]) * f_scale
            wb = sum(write[k]) / len(write[k]) * w_scale
            out["per_launch"][k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                    "bytes": round(fb + wb), "launches": len(fetch[k])}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_prefill.json")


def summarize_mfma(pmc_dir):
    """Matrix-core busy fraction and effective clock of the prefill kernel from a
    rocprofv3 run with --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
    SQ_BUSY_CYCLES GRBM_GUI_ACTIVE: busy = MFMA-busy cycles / (GPU-active cycles x
    SIMDs); clock = GPU-active cycles / dispatch duration (the GRBM counter comes
    summed over the XCDs: divided by their number); bf16 MFMA flops = MOPS x 512."""
    import csv
    import glob
    import re
    simds, xcc = 1024, 8
    for f in glob.glob(os.path.join(pmc_dir, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if int(r.get("Simd_Count", 0) or 0) > 0:
                simds, xcc = int(r["Simd_Count"]), int(r["Num_Xcc"])
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            m = re.search(r"\b(prefill_kernel|decode_partial_kernel)<\d+[,>]", r["Kernel_Name"])
            if not m:
                continue
            d = per.setdefault((m.group(1), r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            d["grid"] = int(r["Grid_Size"])
    out = {"kernels_sha256_16": kernels_hash(), "per_kernel": {}}
    for k in ("prefill_kernel", "decode_partial_kernel"):
        rows = [v for (kk, _), v in per.items() if kk == k and "GRBM_GUI_ACTIVE" in v]
        if rows and k == "decode_partial_kernel":  # the all-layer call: the largest grid
            g = max(v["grid"] for v in rows)
            rows = [v for v in rows if v["grid"] == g]
        if not rows:
            continue
        busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in rows)
        act = sum(v["GRBM_GUI_ACTIVE"] for v in rows) / xcc
        ns = sum(v["ns"] for v in rows)
        flops = sum(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for v in rows) * 512
        out["per_kernel"][k] = {"launches": len(rows),
                                "mfma_busy_frac": round(busy / (act * simds), 4),
                                "effective_clock_ghz": round(act / ns, 3),
                                "mfma_bf16_flops_per_launch": round(flops / len(rows))}
    json.dump(out, open(MFMA_FILE, "w"), indent=1)
    print(json.dumps(out))


def measured_mfma(kernel):
    """Matrix-core busy fraction and effective clock from the committed counter
    run, or None when the kernel source changed since it was taken."""
    try:
        t = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernels_sha256_16") != kernels_hash():
        return None
    return t.get("per_kernel", {}).get(kernel)


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernels_sha256_16") != kernels_hash():
        return None
    k = t.get("per_launch", {}).get(kernel)
    return None if k is None else k["bytes"]


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path (the units would "
              "shard by KV head with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_attention_segmentpagetable_amd as sp
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ prefill setup
    pspec = W.long_prefill(num_layers=args.prefill_layers, n=args.prefill_n)
    pplan = sp.Plan(pspec)
    pz = pplan.sizes
    pb = pplan.allocate(dev, workspace=False)
    N, Hq, Hkv, D = args.prefill_n, pspec.num_q_heads, pspec.num_kv_heads, pspec.head_dim
    nd = min(args.distinct, args.prefill_layers)
    log(f"prefill: {args.prefill_layers} layers x {N} tokens, pool {2 * pz.pool_bytes / 1e9:.1f} GB,"
        f" items {pz.prefill_items}")
    qs = [W.randn_bf16_device((N, Hq, D), pspec.seed, W.TAG_Q, l, dev) for l in range(nd)]
    ks = [W.randn_bf16_device((N, Hkv, D), pspec.seed, W.TAG_K, l, dev) for l in range(nd)]
    vs = [W.randn_bf16_device((N, Hkv, D), pspec.seed, W.TAG_V, l, dev) for l in range(nd)]
    o_pre = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    lse_pre = torch.empty((N, Hq), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    pstats = [pplan.stats(l) for l in range(args.prefill_layers)]
    prefill_flops = sum(4 * D * pspec.group * s["prefill_pairs"] for s in pstats)
    build_bytes = sum(2 * 2 * D * 2 * s["retained_tokens"] for s in pstats)  # K+V, read + write

    # ------------------------------------------------------------------ decode setup
    dspec = W.llama70b_decode(num_layers=args.decode_layers, n=args.decode_n)
    dplan = sp.Plan(dspec)
    dz = dplan.sizes
    db = dplan.allocate(dev)
    B = dspec.num_seqs
    log(f"decode: {args.decode_layers} layers x {B} x {args.decode_n}, pool "
        f"{2 * dz.pool_bytes / 1e9:.1f} GB, items {dz.decode_items}, ws {dz.decode_workspace_bytes / 1e6:.0f} MB")
    for l in range(args.decode_layers):
        kd = W.randn_bf16_device((B * args.decode_n, Hkv, D), dspec.seed, W.TAG_K, l, dev)
        vd = W.randn_bf16_device((B * args.decode_n, Hkv, D), dspec.seed, W.TAG_V, l, dev)
        sp.build(dplan, l, kd, vd, db["table"], db["k_pool"], db["v_pool"])
        del kd, vd
    q_dec = W.randn_bf16_device((args.decode_layers, B, Hq, D), dspec.seed, W.TAG_Q, 0, dev)
    o_dec = torch.empty_like(q_dec)
    lse_dec = torch.empty((args.decode_layers, B, Hq), dtype=torch.float32, device=dev)
    dstats = dplan.stats(-1)
    decode_bytes = dstats["decode_tokens"] * 2 * D * 2  # K and V, bf16, each visible key once
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):  # an elementwise kernel with a distinctive name: reads and writes 1 GiB
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ev = lambda: torch.cuda.Event(enable_timing=True)
    rec = {"build": [], "prefill": [], "decode": []}

    def step(record):
        for l in range(args.prefill_layers):
            e0, e1, e2 = ev(), ev(), ev()
            e0.record(stream)
            sp.build(pplan, l, ks[l % nd], vs[l % nd], pb["table"], pb["k_pool"], pb["v_pool"])
            e1.record(stream)
            sp.prefill(pplan, l, qs[l % nd], pb["table"], pb["k_pool"], pb["v_pool"], scale,
                       o_pre, lse_pre)
            e2.record(stream)
            if record:
                rec["build"].append((e0, e1))
                rec["prefill"].append((e1, e2))
        e0, e1 = ev(), ev()
        e0.record(stream)
        sp.decode(dplan, -1, q_dec, db["table"], db["k_pool"], db["v_pool"], scale, o_dec,
                  lse_dec, workspace=db["workspace"])
        e1.record(stream)
        if record:
            rec["decode"].append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dur = {k: [a.elapsed_time(b) for a, b in v] for k, v in rec.items()}

    # extra decode-only repetitions for a stable bandwidth figure
    reps = []
    for _ in range(args.decode_reps):
        e0, e1 = ev(), ev()
        e0.record(stream)
        sp.decode(dplan, -1, q_dec, db["table"], db["k_pool"], db["v_pool"], scale, o_dec,
                  lse_dec, workspace=db["workspace"])
        e1.record(stream)
        reps.append((e0, e1))
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in reps]
    dec_med = float(np.median(dec_ms))

    # the same decode as one launch per layer (each reads its own layer's pages,
    # about 1/80 of the K/V, so nothing carries over from one launch to the next)
    layer_reps = []
    for _ in range(4):
        e0, e1 = ev(), ev()
        e0.record(stream)
        for l in range(args.decode_layers):
            sp.decode(dplan, l, q_dec[l], db["table"], db["k_pool"], db["v_pool"], scale,
                      o_dec[l], lse_dec[l], workspace=db["workspace"])
        e1.record(stream)
        layer_reps.append((e0, e1))
    torch.cuda.synchronize()
    dec_layer_ms = float(np.median([a.elapsed_time(b) for a, b in layer_reps[1:]]))

    xfer = page_transfer(torch, sp, dplan, db, dspec, stream, log)
    ceil = measure_ceilings(torch, dev, stream, log)
    # layer 0 once more, untimed: the output the accuracy checks below compare (the
    # timed steps leave the last layer's in o_pre)
    sp.prefill(pplan, 0, qs[0], pb["table"], pb["k_pool"], pb["v_pool"], scale, o_pre, lse_pre)
    torch.cuda.synchronize()

    pre_ms_layer = float(np.mean(dur["prefill"]))
    pre_ms_step = float(np.sum(dur["prefill"])) / args.steps
    bld_ms_step = float(np.sum(dur["build"])) / args.steps
    pre_tflops = prefill_flops / (pre_ms_step * 1e-3) / 1e12
    dec_gbs = decode_bytes / (dec_med * 1e-3) / 1e9
    value = N / (ms_step * 1e-3)
    log(f"step {ms_step:.1f} ms: build {bld_ms_step:.1f} ms, prefill {pre_ms_step:.1f} ms "
        f"({pre_tflops:.0f} TF/s), decode {dec_med:.3f} ms ({dec_gbs:.0f} GB/s)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V, seeded head classes",
        "config": {
            "workload": (f"long-prefill {N} tokens x {args.prefill_layers} layers (64 Q / 8 KV "
                         f"heads, D 128, page 64, 15% global, local sink 4 window 8192; build + "
                         f"prefill per layer) + llama70b-shaped decode {B} x {args.decode_n} x "
                         f"{args.decode_layers} layers (one all-layer decode call)"),
            "prefill_tokens_per_step": N,
            "prefill_layers": args.prefill_layers,
            "decode_batch": B,
            "decode_context": args.decode_n,
            "decode_layers": args.decode_layers,
            "distinct_input_layers": nd,
        },
        "prefill": {
            "tok_per_s_kernels": round(N / ((pre_ms_step + bld_ms_step) * 1e-3), 2),
            "ms_prefill_per_step": round(pre_ms_step, 3),
            "ms_build_per_step": round(bld_ms_step, 3),
            "ms_prefill_per_layer": round(pre_ms_layer, 4),
            "algorithmic_flops_per_step": prefill_flops,
            "tflops": round(pre_tflops, 1),
            "build_gbs": round(build_bytes / (bld_ms_step * 1e-3) / 1e9, 1),
            # the prefill-form cache keeps every key (rows from 0 read it); what the
            # layout saves here is attention work: visible pairs against causal
            "kv_tokens": _kv_tokens(pplan, pspec),
            "attention_pairs_frac_of_causal": round(
                sum(pspec.group * s["prefill_pairs"] for s in pstats) /
                (args.prefill_layers * Hq * N * (N + 1) / 2), 4),
        },
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "frac_of_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
            "ms_median": round(dec_med, 4),
            "ms_min": round(float(np.min(dec_ms)), 4),
            "reps": args.decode_reps,
            "kv_bytes": decode_bytes,
            "kv_tokens": _kv_tokens(dplan, dspec),
            "ms_in_steps": [round(x, 4) for x in dur["decode"]],
            "per_layer_launches": {
                "launches": args.decode_layers,
                "ms_all_layers": round(dec_layer_ms, 4),
                "ms_per_layer": round(dec_layer_ms / args.decode_layers, 4),
                "gbs": round(decode_bytes / (dec_layer_ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(decode_bytes / (dec_layer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            },
            "page_transfer": xfer,
        },
        "roofline": {
            "kernel": "prefill_kernel",
            "bound": "mfma",
            "achieved": round(pre_tflops, 1),
            "peak": BF16_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / BF16_PEAK_TFS, 4),
            "frac_of_measured_ceiling": round(pre_tflops / ceil["mfma_bf16_tflops"], 4),
            "mfma_counters": measured_mfma("prefill_kernel"),
            "traffic": measured_traffic("prefill_kernel"),
            "traffic_unit": "bytes per launch (one layer)",
        },
        "roofline_decode": {
            "kernel": "decode_partial_kernel + decode_combine_kernel",
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "frac_of_measured_ceiling": round(dec_gbs / ceil["hbm_read_gbs"], 4),
            "traffic": measured_traffic("decode_partial_kernel"),
            "traffic_unit": "bytes per launch (all layers)",
            "algorithmic_bytes_per_launch": decode_bytes,
        },
    }

    out["measured_ceilings"] = ceil
    if not args.no_dense:
        try:
            out["dense_mask"] = dense_mask_baseline(torch, W, pspec, dspec, ks[0], vs[0], qs[0],
                                                    dev, pre_ms_layer, dec_med, args, log,
                                                    o_pre, q_dec, o_dec)
        except Exception as e:  # the comparison path is optional context
            out["dense_mask"] = {"error": f"{type(e).__name__}: {e}"[:300]}
    if not args.no_cpu_baseline:
        # the oracle rows timed for the baseline double as the accuracy check of the
        # timed outputs (prefill: layer 0 rows; decode: the all-layer call's rows)
        out["cpu_baseline"] = cpu_baseline(torch, W, pspec, qs[0], ks[0], vs[0], args, log,
                                           o_pre)
        out["prefill"]["accuracy_vs_oracle"] = out["cpu_baseline"].pop("accuracy")
        out["cpu_baseline"]["decode"] = cpu_baseline_decode(torch, W, dspec, dplan, q_dec, dev,
                                                            args, log, o_dec)
        out["decode"]["accuracy_vs_oracle"] = out["cpu_baseline"]["decode"].pop("accuracy")
    if not args.no_extra:
        del pb, db, qs, ks, vs, o_pre, lse_pre, q_dec, o_dec, lse_dec
        torch.cuda.empty_cache()
        samples = {}
        out.update(extra_configs(torch, W, sp, dev, stream, log, samples))
        if not args.no_cpu_baseline:
            cpu_baseline_extra(W, samples, out, log)
    print(json.dumps(out), flush=True)


def page_transfer(torch, sp, plan, bufs, spec, stream, log):
    """The decode cache moved as page streams (all layers in one call each way):
    what a prefill machine would send a decode machine, against the dense K/V of
    the same tokens. Export and import each read and write the stream's bytes."""
    n = sp.stream_elems(plan, -1)
    ks = torch.empty(n, dtype=torch.bfloat16, device=bufs["k_pool"].device)
    vs = torch.empty_like(ks)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts]))

    ex_ms = timed(lambda: sp.export_pages(plan, -1, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                          ks, vs))
    im_ms = timed(lambda: sp.import_pages(plan, -1, ks, vs, bufs["table"], bufs["k_pool"],
                                          bufs["v_pool"]))
    stream_bytes = 2 * n * 2
    st = plan.stats(-1)
    retained = st["retained_tokens"] * 2 * spec.head_dim * 2
    dense = 2 * spec.num_layers * spec.num_kv_heads * spec.head_dim * 2 * sum(spec.seq_len)
    del ks, vs
    torch.cuda.empty_cache()
    log(f"page transfer: {stream_bytes / 1e9:.2f} GB stream (dense {dense / 1e9:.1f} GB, "
        f"{dense / stream_bytes:.2f}x less), export {ex_ms:.2f} ms, import {im_ms:.2f} ms")
    return {
        "workload": "the llama70b-shaped decode cache (all layers) as K and V page streams",
        "stream_bytes": stream_bytes,
        "retained_kv_bytes": retained,
        "dense_kv_bytes": dense,
        "dense_over_stream": round(dense / stream_bytes, 3),
        "export_ms": round(ex_ms, 3),
        "import_ms": round(im_ms, 3),
        "export_hbm_gbs": round(2 * stream_bytes / (ex_ms * 1e-3) / 1e9, 1),
        "import_hbm_gbs": round(2 * stream_bytes / (im_ms * 1e-3) / 1e9, 1),
    }


def measure_ceilings(torch, dev, stream, log):
    """What the chip sustains on this machine, from the probes of libsegpaged_probe.so:
    dense bf16 MFMA issue with N(0,1) operands (one and two 8-wave workgroups per
    CU; the better is kept) and a streaming read of 4 GiB (16 times the 256 MB
    Infinity Cache; the best of 1-32 workgroups per CU x 4, 8, 16 loads in flight
    per thread). Operands that change every MFMA hold the clock lower than constant
    ones (~1.6 vs ~2.0 PFLOP/s here), so the probe rotates them as the attention
    kernels' operands do. Timed with HIP events, median of 5."""
    from sparse_attention_segmentpagetable_amd import probe
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device="cpu").manual_seed(2024)
    seed = torch.randn(probe.SEED_ELEMS, generator=g).to(torch.bfloat16).to(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def med(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts]))

    iters = 200
    best = 0.0
    for per_cu in (1, 2):
        wgs = cus * per_cu
        out = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
        ms = med(lambda: probe.mfma_bf16(seed, iters, wgs, out))
        best = max(best, wgs * 8 * iters * 8 * 32768 / (ms * 1e-3) / 1e12)
    src = torch.ones((4 << 30) // 4, dtype=torch.float32, device=dev)
    ms = float("inf")
    for per_cu in (1, 2, 4, 8, 16, 32):
        for depth in (4, 8, 16):
            wgs = cus * per_cu
            out = torch.empty(wgs, dtype=torch.float32, device=dev)
            ms = min(ms, med(lambda: probe.hbm_read(src, wgs, out, depth=depth)))
    hbm = src.numel() * 4 / (ms * 1e-3) / 1e9
    del src
    torch.cuda.empty_cache()
    log(f"measured ceilings: bf16 MFMA {best:.0f} TF/s, HBM read {hbm:.0f} GB/s")
    return {"mfma_bf16_tflops": round(best, 1), "hbm_read_gbs": round(hbm, 1),
            "mfma_frac_of_peak": round(best / BF16_PEAK_TFS, 4),
            "hbm_frac_of_peak": round(hbm / HBM_PEAK_GBS, 4),
            "probes": "include/segpaged_probe.h (bf16 MFMA loop, N(0,1) operands; 4 GiB "
                      "streaming read)"}


def _bits(t):
    """bf16 bits of a device tensor as host uint16."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _sample(samples, key, spec, layer, b, pos, q_rows, k_seq, v_seq, got):
    """Keep what the oracle needs to check rows `pos` of sequence b: host bits of
    their queries and of the sequence's K/V (uint16), and the GPU's output rows."""
    samples.setdefault(key, []).append((spec, layer, b, np.asarray(pos), q_rows, k_seq, v_seq,
                                        got))


def extra_configs(torch, W, sp, dev, stream, log, samples):
    """The other configurations of the scope table, timed outside the step (not part
    of `value`): the mixed-length decode with retrieval heads (32 sequences of 2K-128K
    tokens, 48 layers, one all-layer call; working set far beyond the caches) and the
    Mistral-7B-shaped layer (4 x 8K prefill and one decode step; the decode working
    set of 31 MB is cache-resident, so its GB/s is context, not an HBM figure)."""
    res = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(reps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in pairs]
        return float(np.median(ms)), float(np.min(ms))

    # mixed-length decode
    spec = W.mixed_varlen_decode()
    plan = sp.Plan(spec)
    bufs = plan.allocate(dev)
    L, Hq, Hkv, D = spec.num_layers, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    T = spec.total_tokens
    for l in range(L):
        kd = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_K, l, dev)
        vd = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_V, l, dev)
        sp.build(plan, l, kd, vd, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        del kd, vd
    q = W.randn_bf16_device((L, spec.num_seqs, Hq, D), spec.seed, W.TAG_Q, 0, dev)
    o = torch.empty_like(q)
    lse = torch.empty((L, spec.num_seqs, Hq), dtype=torch.float32, device=dev)
    st = plan.stats(-1)
    kv_bytes = st["decode_tokens"] * 2 * D * 2
    med, mn = timed(lambda: sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                      1.0 / math.sqrt(D), o, lse, workspace=bufs["workspace"]), 10)
    gbs = kv_bytes / (med * 1e-3) / 1e9
    # oracle check rows: the longest and the shortest sequence, and two seeded ones,
    # each at a seeded layer (retrieval heads included where the layer has them)
    rng = np.random.default_rng([spec.seed, 79])
    kvo = spec.kv_row_offsets()
    pick = [int(np.argmax(spec.seq_len)), int(np.argmin(spec.seq_len))]
    pick += [int(x) for x in rng.choice(spec.num_seqs, size=2, replace=False)]
    for b in pick:
        l = int(rng.integers(0, L))
        kd = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_K, l, dev)
        vd = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_V, l, dev)
        sl = slice(kvo[b], kvo[b] + spec.seq_len[b])
        _sample(samples, "decode_mixed", spec, l, b, [spec.seq_len[b] - 1], _bits(q[l, b:b + 1]),
                _bits(kd[sl]), _bits(vd[sl]), _to_f64(o[l, b:b + 1]))
        del kd, vd
    res["decode_mixed"] = {
        "workload": (f"{spec.num_seqs} sequences of {min(spec.seq_len)}-{max(spec.seq_len)} tokens, "
                     f"{L} layers x {Hkv} KV heads (12% global, 8% retrieval with 5% index sets, "
                     f"local sink 4 window 4096), one all-layer decode call"),
        "value": round(gbs, 1), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_median": round(med, 4), "ms_min": round(mn, 4), "kv_bytes": kv_bytes,
        "decode_items": plan.sizes.decode_items,
        "kv_tokens": _kv_tokens(plan, spec),
    }
    log(f"mixed decode: {med:.3f} ms, {gbs:.0f} GB/s")
    del plan, bufs, q, o, lse
    torch.cuda.empty_cache()

    # Mistral-7B-shaped layer
    spec = W.mistral_layer("prefill")
    plan = sp.Plan(spec)
    bufs = plan.allocate(dev, workspace=False)
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    T = spec.total_tokens
    k = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_K, 0, dev)
    v = W.randn_bf16_device((T, Hkv, D), spec.seed, W.TAG_V, 0, dev)
    q = W.randn_bf16_device((T, Hq, D), spec.seed, W.TAG_Q, 0, dev)
    o = torch.empty_like(q)
    sp.build(plan, 0, k, v, bufs["table"], bufs["k_pool"], bufs["v_pool"])
    flops = 4 * D * spec.group * plan.stats(0)["prefill_pairs"]
    pmed, pmn = timed(lambda: sp.prefill(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                         1.0 / math.sqrt(D), o), 20)
    bmed, _ = timed(lambda: sp.build(plan, 0, k, v, bufs["table"], bufs["k_pool"], bufs["v_pool"]), 20)
    dspec = W.mistral_layer("decode")
    dplan = sp.Plan(dspec)
    db = dplan.allocate(dev)
    kd = W.randn_bf16_device((dspec.total_tokens, Hkv, D), dspec.seed, W.TAG_K, 0, dev)
    vd = W.randn_bf16_device((dspec.total_tokens, Hkv, D), dspec.seed, W.TAG_V, 0, dev)
    sp.build(dplan, 0, kd, vd, db["table"], db["k_pool"], db["v_pool"])
    qd = W.randn_bf16_device((dspec.num_seqs, Hq, D), dspec.seed, W.TAG_Q, 1, dev)
    od = torch.empty_like(qd)
    dmed, dmn = timed(lambda: sp.decode(dplan, 0, qd, db["table"], db["k_pool"], db["v_pool"],
                                        1.0 / math.sqrt(D), od, workspace=db["workspace"]), 50)
    dbytes = dplan.stats(0)["decode_tokens"] * 2 * D * 2
    # oracle check rows: per sequence the sink, window and page edges, the last row
    # and 22 seeded rows of the prefill; every decode row
    rng = np.random.default_rng([spec.seed, 80])
    n = spec.seq_len[0]
    for b in range(spec.num_seqs):
        pos = sorted(set([0, 3, 4, 63, 64, 1023, 1024, 1027, 1028, n - 1] +
                         [int(x) for x in rng.choice(n, size=22, replace=False)]))
        rows = torch.as_tensor([b * n + p for p in pos], device=dev)
        _sample(samples, "mistral_prefill", spec, 0, b, pos, _bits(q[rows]),
                _bits(k[b * n:(b + 1) * n]), _bits(v[b * n:(b + 1) * n]), _to_f64(o[rows]))
        nd, kv0 = dspec.seq_len[b], dspec.kv_row_offsets()[b]
        kvd = slice(kv0, kv0 + nd)
        _sample(samples, "mistral_decode", dspec, 0, b, [nd - 1], _bits(qd[b:b + 1]),
                _bits(kd[kvd]), _bits(vd[kvd]), _to_f64(od[b:b + 1]))
    res["mistral_layer"] = {
        "workload": "4 x 8192 tokens, 32 Q / 8 KV heads, D 128, page 64, KV head 0 global, 1-7 local (sink 4, window 1024)",
        "prefill_tflops": round(flops / (pmed * 1e-3) / 1e12, 1),
        "prefill_frac_of_bf16_peak": round(flops / (pmed * 1e-3) / 1e12 / BF16_PEAK_TFS, 4),
        "prefill_ms": round(pmed, 4), "prefill_flops": flops,
        "prefill_tok_per_s_with_build": round(T / ((pmed + bmed) * 1e-3), 1),
        "build_ms": round(bmed, 4),
        "decode_ms": round(dmed, 4), "decode_kv_bytes": dbytes,
        "decode_gbs_cache_resident": round(dbytes / (dmed * 1e-3) / 1e9, 1),
        "prefill_kv_tokens": _kv_tokens(plan, spec),
        "decode_kv_tokens": _kv_tokens(dplan, dspec),
    }
    log(f"mistral layer: prefill {pmed:.3f} ms ({flops / (pmed * 1e-3) / 1e12:.0f} TF/s), "
        f"decode {dmed * 1e3:.1f} us")
    del plan, bufs, k, v, q, o, dplan, db
    torch.cuda.empty_cache()
    res["tiny"] = tiny_config(torch, W, sp, dev, timed, log, samples)
    res["long_prefill_decode_form_build"] = decode_form_build(torch, W, sp, dev, timed, log)
    res["decode_context_sweep"] = decode_context_sweep(torch, W, sp, dev, timed, log)
    res["decode_loop_append"] = decode_loop_append(torch, W, sp, dev, stream, log)
    res["chunked_prefill"] = chunked_prefill(torch, W, sp, dev, stream, log)
    res["retrieval_selection"] = retrieval_selection(torch, W, sp, dev, timed, log)
    res["shared_document"] = shared_document(torch, W, sp, dev, timed, log)
    return res


def shared_document(torch, W, sp, dev, timed, log):
    """Sequences that begin with one shared document (the same tokens at the same
    positions): the Llama-shaped decode, 8 layers x 8 sequences x 32768 tokens, all 8
    sequences sharing their first 16384 tokens. The pool stores each page inside the
    document once per (layer, KV head); decode reads every unit's pages as before.
    Pool bytes against the same cache without sharing, build and decode time."""
    from dataclasses import replace as _replace
    n, c, L = 32768, 16384, 8
    base = W.llama70b_decode(num_layers=L, n=n)
    B, Hq, Hkv, D = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_dim
    spec = _replace(base, doc_group=[0] * B, doc_len=[c] * B)
    plan = sp.Plan(spec)
    own_pool = sp.Plan(base).sizes.pool_bytes
    bufs = plan.allocate(dev)
    k = W.randn_bf16_device((B * n, Hkv, D), spec.seed, W.TAG_K, 0, dev)
    v = W.randn_bf16_device((B * n, Hkv, D), spec.seed, W.TAG_V, 0, dev)
    kv = k.view(B, n, Hkv, D)
    vv = v.view(B, n, Hkv, D)
    kv[1:, :c] = kv[0, :c]  # the shared document: the same rows in every sequence
    vv[1:, :c] = vv[0, :c]
    bms = []
    for l in range(L):
        ms, _ = timed(lambda: sp.build(plan, l, k, v, bufs["table"], bufs["k_pool"],
                                       bufs["v_pool"]), 3)
        bms.append(ms)
    q = W.randn_bf16_device((L, B, Hq, D), spec.seed, W.TAG_Q, 0, dev)
    o = torch.empty_like(q)
    med, _ = timed(lambda: sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                     1.0 / math.sqrt(D), o, workspace=bufs["workspace"]), 10)
    kv_bytes = plan.stats(-1)["decode_tokens"] * 2 * D * 2
    pool = plan.sizes.pool_bytes
    log(f"shared document: pool {pool / 1e6:.0f} MB vs {own_pool / 1e6:.0f} MB unshared, "
        f"decode {med:.3f} ms ({kv_bytes / (med * 1e-3) / 1e9:.0f} GB/s of K/V the rows see)")
    del plan, bufs, k, v, q, o
    torch.cuda.empty_cache()
    return {"workload": f"llama70b-shaped decode {B} x {n} x {L} layers, every sequence "
                        f"beginning with the same {c}-token document",
            "pool_bytes_per_tensor": pool, "unshared_pool_bytes_per_tensor": own_pool,
            "pool_saving": round(1 - pool / own_pool, 4),
            "build_ms_per_layer": round(float(np.mean(bms)), 4),
            "decode_ms": round(med, 4), "decode_kv_bytes_seen": kv_bytes,
            "decode_gbs_of_keys_seen": round(kv_bytes / (med * 1e-3) / 1e9, 1)}


def tiny_config(torch, W, sp, dev, timed, log, samples):
    """The tiny workload (1 layer, 8 Q / 4 KV heads, D 64, page 16, 512 tokens):
    causal prefill of all rows and the decode step at 513 tokens; launch-bound,
    timed for context and kept whole for the oracle check."""
    res = {}
    for form in ("prefill", "decode"):
        spec = W.tiny(form)
        plan = sp.Plan(spec)
        bufs = plan.allocate(dev)
        kb, vb = W.kv_bits(spec, 0)
        qb = W.q_bits(spec, 0)
        dv = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        sp.build(plan, 0, dv(kb), dv(vb), bufs["table"], bufs["k_pool"], bufs["v_pool"])
        q = dv(qb)
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(spec.head_dim)
        if form == "prefill":
            fn = lambda: sp.prefill(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                    scale, o)
        else:
            fn = lambda: sp.decode(plan, 0, q, bufs["table"], bufs["k_pool"], bufs["v_pool"],
                                   scale, o, workspace=bufs["workspace"])
        med, mn = timed(fn, 50)
        n = spec.seq_len[0]
        _sample(samples, f"tiny_{form}", spec, 0, 0, list(range(spec.first_query_pos[0], n)), qb,
                kb, vb, _to_f64(o))
        res[form] = {"ms_median": round(med, 4), "ms_min": round(mn, 4),
                     "kv_tokens": _kv_tokens(plan, spec)}
        del plan, bufs, q, o
    log(f"tiny: prefill {res['prefill']['ms_median'] * 1e3:.1f} us, decode "
        f"{res['decode']['ms_median'] * 1e3:.1f} us")
    return res


def cpu_baseline_extra(W, samples, out, log):
    """The oracle on the rows kept from the other workloads' timed outputs: the
    equivalence check of the runtime explainer (cosine, and max |O - O_ref|)
    against the fp64 definition, per workload."""
    from oracle import attention as OA
    where = {"tiny_prefill": ("tiny", "prefill"), "tiny_decode": ("tiny", "decode"),
             "mistral_prefill": ("mistral_layer", "prefill_accuracy_vs_oracle"),
             "mistral_decode": ("mistral_layer", "decode_accuracy_vs_oracle"),
             "decode_mixed": ("decode_mixed", "accuracy_vs_oracle")}
    for key, rows in samples.items():
        t0 = time.perf_counter()
        acc = []
        for spec, layer, b, pos, qb, kb, vb, got in rows:
            ref, _ = OA.attention_rows(spec, layer, b, pos, qb, kb, vb)
            acc.append(_acc(got, ref))
        rec = dict(_merge_acc(acc), rows=int(sum(len(r[3]) for r in rows)),
                   oracle_seconds=round(time.perf_counter() - t0, 2))
        top, field = where[key]
        if key.startswith("tiny_"):
            out[top][field]["accuracy_vs_oracle"] = rec
        else:
            out[top][field] = rec
        log(f"oracle check {key}: max|err| {rec['max_abs_err']:.3e} min cos {rec['min_cos']:.8f}")


def retrieval_selection(torch, W, sp, dev, timed, log):
    """Top-p retrieval-set selection (segpaged_select_topp) on one Llama-shaped
    layer, 8 sequences x 32768 keys, KV heads 0-1 retrieval (16 (sequence, head)
    pairs): the decode row's attention over the dense history, then top-p = 0.9.
    The scoring pass reads each pair's dense K once (the algorithmic bytes)."""
    from dataclasses import replace as _replace
    n = 32768
    base = W.llama70b_decode(num_layers=1, n=n)
    kind = [W.RETRIEVAL, W.RETRIEVAL] + [W.LOCAL] * 6
    retr = {(b, 0, h): np.zeros(0, np.int32) for b in range(base.num_seqs) for h in (0, 1)}
    spec = _replace(base, kind=kind, retrieval=retr)
    B, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    plan = sp.Plan(spec)
    bufs = plan.allocate(dev, workspace=False)
    k = W.randn_bf16_device((B * n, Hkv, D), spec.seed, W.TAG_K, 0, dev)
    sp.build(plan, 0, k, k, bufs["table"], bufs["k_pool"], bufs["v_pool"])
    q = W.randn_bf16_device((B, Hq, D), spec.seed, W.TAG_Q, 0, dev) * 4
    T = plan.sizes.kv_rows
    out_pos = torch.empty(Hkv * T, dtype=torch.int32, device=dev)
    out_cnt = torch.empty(B * Hkv, dtype=torch.int32, device=dev)
    ws = torch.empty(plan.sizes.select_workspace_bytes // 4, dtype=torch.float32, device=dev)
    ms, _ = timed(lambda: sp.select_topp(plan, 0, q, k, bufs["table"], 1 / math.sqrt(D), 0.9,
                                         out_pos, out_cnt, ws), 10)
    kept = float(out_cnt.view(B, Hkv)[:, :2].float().mean())
    kbytes = 2 * B * n * D * 2
    log(f"retrieval selection: {ms:.3f} ms for {2 * B} pairs x {n} keys "
        f"({kbytes / (ms * 1e-3) / 1e9:.0f} GB/s of dense K), {kept:.0f} keys kept per pair at p 0.9")
    del plan, bufs, k, q, out_pos, out_cnt, ws
    torch.cuda.empty_cache()
    return {"workload": f"llama-shaped layer, {B} seqs x {n} keys, 2 retrieval KV heads, top-p 0.9",
            "ms": round(ms, 4), "dense_k_gbs": round(kbytes / (ms * 1e-3) / 1e9, 1),
            "keys_kept_per_pair": round(kept, 1)}


def chunked_prefill(torch, W, sp, dev, stream, log):
    """The long-prefill workload (131072 tokens, 2 layers) taken in 8 chunks of
    16384 over a cache planned for growth: local heads hold their sink and a ring
    of ceil((8192 + 16384 - 1)/64) + 1 pages instead of the whole prompt. Per
    chunk: segpaged_plan_append, segpaged_append of the chunk's K/V, then the
    chunk's prefill rows per layer. Reports prefill TFLOP/s over all chunks, the
    append time, and the pool bytes against the one-shot (prefill-form) plan."""
    from dataclasses import replace as _replace
    N, chunk, L = 131072, 16384, 2
    full = W.long_prefill(num_layers=L, n=N)
    Hq, Hkv, D = full.num_q_heads, full.num_kv_heads, full.head_dim
    spec = _replace(full, seq_len=[chunk], first_query_pos=[0])
    plan = sp.Plan(spec, append_capacity=N - chunk, append_chunk=chunk)
    one_shot_pool = sp.Plan(full).sizes.pool_bytes
    bufs = plan.allocate(dev, workspace=False)
    k = W.randn_bf16_device((N, Hkv, D), full.seed, W.TAG_K, 0, dev)
    v = W.randn_bf16_device((N, Hkv, D), full.seed, W.TAG_V, 0, dev)
    q = W.randn_bf16_device((N, Hq, D), full.seed, W.TAG_Q, 0, dev)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for l in range(L):
        sp.build(plan, l, k[:chunk], v[:chunk], bufs["table"], bufs["k_pool"], bufs["v_pool"])
    pre, app, flops = [], [], 0
    n = chunk
    for c in range(N // chunk):
        if c > 0:
            plan.append([chunk])
            e0, e1 = ev(), ev()
            e0.record(stream)
            for l in range(L):
                sp.append(plan, l, k[n:n + chunk], v[n:n + chunk], bufs["table"], bufs["k_pool"],
                          bufs["v_pool"])
            e1.record(stream)
            app.append((e0, e1))
            n += chunk
        for l in range(L):
            flops += 4 * D * full.group * plan.stats(l)["prefill_pairs"]
            e0, e1 = ev(), ev()
            e0.record(stream)
            sp.prefill(plan, l, q[n - chunk:n], bufs["table"], bufs["k_pool"], bufs["v_pool"], scale,
                       o[n - chunk:n])
            e1.record(stream)
            pre.append((e0, e1))
    torch.cuda.synchronize()
    pre_ms = sum(a.elapsed_time(b) for a, b in pre)
    app_ms = sum(a.elapsed_time(b) for a, b in app)
    tf = flops / (pre_ms * 1e-3) / 1e12
    log(f"chunked prefill: {pre_ms / L:.1f} ms/layer over {N // chunk} chunks ({tf:.0f} TF/s), "
        f"append {app_ms / L:.3f} ms/layer, pool {plan.sizes.pool_bytes / 1e6:.0f} MB vs "
        f"{one_shot_pool / 1e6:.0f} MB one-shot")
    pool = plan.sizes.pool_bytes
    dense_bytes = L * N * Hkv * D * 2
    del plan, bufs, k, v, q, o
    torch.cuda.empty_cache()
    return {"workload": f"long-prefill {N} tokens x {L} layers in {N // chunk} chunks of {chunk}",
            "prefill_ms_per_layer": round(pre_ms / L, 3), "prefill_tflops": round(tf, 1),
            "append_ms_per_layer": round(app_ms / L, 4),
            "pool_bytes_per_tensor": pool, "one_shot_pool_bytes_per_tensor": one_shot_pool,
            "pool_frac_of_dense_kv": round(pool / dense_bytes, 4),
            "kv_saving_vs_dense": round(1 - pool / dense_bytes, 4)}


def decode_loop_append(torch, W, sp, dev, stream, log):
    """The Llama-shaped decode (8 x 32K x 80 layers) as a decode loop: a cache
    planned once with room to grow, then per step each sequence gains a token
    (segpaged_plan_append on the host, segpaged_append writing its K/V for all 80
    layers) and the all-layer decode runs. Host plan time, device append time and
    decode time per step; the step is what a serving loop pays per token."""
    import time as _time
    steps, cap = 32, 64
    spec = W.llama70b_decode(num_layers=80, n=32768)
    B, Hkv, D, L = spec.num_seqs, spec.num_kv_heads, spec.head_dim, spec.num_layers
    plan = sp.Plan(spec, append_capacity=cap)
    bufs = plan.allocate(dev)
    for l in range(L):
        kd = W.randn_bf16_device((B * 32768, Hkv, D), spec.seed, W.TAG_K, l, dev)
        vd = W.randn_bf16_device((B * 32768, Hkv, D), spec.seed, W.TAG_V, l, dev)
        sp.build(plan, l, kd, vd, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        del kd, vd
    q = W.randn_bf16_device((L, B, spec.num_q_heads, D), spec.seed, W.TAG_Q, 0, dev)
    o = torch.empty_like(q)
    kn = W.randn_bf16_device((L, B, Hkv, D), spec.seed, 77, 0, dev)
    vn = W.randn_bf16_device((L, B, Hkv, D), spec.seed, 78, 0, dev)
    scale = 1.0 / math.sqrt(D)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    host_ms, app_ev, dec_ev, kv_bytes = [], [], [], []
    torch.cuda.synchronize()
    t0 = _time.perf_counter()
    for _ in range(steps):
        h0 = _time.perf_counter()
        plan.append([1] * B)
        host_ms.append((_time.perf_counter() - h0) * 1e3)
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        sp.append(plan, -1, kn, vn, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        e1.record(stream)
        sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"], bufs["v_pool"], scale, o,
                  workspace=bufs["workspace"])
        e2.record(stream)
        app_ev.append((e0, e1))
        dec_ev.append((e1, e2))
        kv_bytes.append(plan.stats(-1)["decode_tokens"] * 2 * D * 2)
    torch.cuda.synchronize()
    wall = (_time.perf_counter() - t0) * 1e3 / steps
    app_ms = float(np.median([a.elapsed_time(b) for a, b in app_ev]))
    dec_ms = float(np.median([a.elapsed_time(b) for a, b in dec_ev]))
    gbs = float(np.median(kv_bytes)) / (dec_ms * 1e-3) / 1e9
    log(f"decode loop: step {wall:.3f} ms wall (host plan {np.median(host_ms):.3f} ms, "
        f"append {app_ms:.3f} ms, decode {dec_ms:.3f} ms = {gbs:.0f} GB/s)")
    del plan, bufs, q, o, kn, vn
    torch.cuda.empty_cache()
    return {"workload": "llama70b-shaped decode 8 x 32768 x 80 layers, one token per sequence "
                        "per step, 32 steps, cache planned once with append capacity 64",
            "steps": steps, "ms_per_step_wall": round(wall, 4),
            "host_plan_append_ms": round(float(np.median(host_ms)), 4),
            "append_kernel_ms": round(app_ms, 4), "decode_ms": round(dec_ms, 4),
            "decode_kv_gbs": round(gbs, 1),
            "tokens_per_s": round(B / (wall * 1e-3), 1)}


def decode_form_build(torch, W, sp, dev, timed, log):
    """The long-prefill workload's cache in decode form (what decoding after the
    prefill keeps: local heads only their sink and last 8192 keys), built per layer
    from the same dense K/V and reported apart from the prefill-form build."""
    pspec = W.long_prefill(num_layers=4)
    dspec = W.decode_form(pspec)
    plan = sp.Plan(dspec)
    bufs = plan.allocate(dev, workspace=False)
    n, Hkv, D = pspec.seq_len[0], pspec.num_kv_heads, pspec.head_dim
    k = W.randn_bf16_device((n, Hkv, D), pspec.seed, W.TAG_K, 0, dev)
    v = W.randn_bf16_device((n, Hkv, D), pspec.seed, W.TAG_V, 0, dev)
    per = []
    for l in range(4):
        ms, _ = timed(lambda: sp.build(plan, l, k, v, bufs["table"], bufs["k_pool"],
                                       bufs["v_pool"]), 10)
        tok = plan.stats(l)["retained_tokens"]
        per.append((ms, tok))
    ms = float(np.mean([p[0] for p in per]))
    tok = float(np.mean([p[1] for p in per]))
    gbs = 2 * 2 * D * 2 * tok / (ms * 1e-3) / 1e9
    log(f"long-prefill decode-form build: {ms:.3f} ms/layer, {2 * D * 2 * tok / 1e6:.0f} MB of "
        f"K/V kept, {gbs:.0f} GB/s")
    kvt = _kv_tokens(plan, dspec)
    del plan, bufs, k, v
    torch.cuda.empty_cache()
    return {"workload": f"layers 0-3 of the long-prefill workload ({n} tokens) in decode form",
            "ms_per_layer": round(ms, 4), "kv_bytes_kept_per_layer": int(2 * D * 2 * tok),
            "gbs_read_plus_write": round(gbs, 1), "kv_tokens": kvt}


def decode_context_sweep(torch, W, sp, dev, timed, log):
    """Decode speedup over the dense-mask path as the context grows: the
    Llama-shaped decode (8 sequences, 8 layers, 15% global, local sink 4 window
    8192) at N = 8K .. 128K; SegPaged one all-layer call, dense-mask torch SDPA
    with boolean masks per layer on dense K/V, both on the same K/V values."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    rows = []
    for n in (8192, 16384, 32768, 65536, 131072):
        spec = W.llama70b_decode(num_layers=8, n=n)
        B, Hq, Hkv, D, G, L = (spec.num_seqs, spec.num_q_heads, spec.num_kv_heads,
                               spec.head_dim, spec.group, spec.num_layers)
        plan = sp.Plan(spec)
        bufs = plan.allocate(dev)
        k = W.randn_bf16_device((B * n, Hkv, D), spec.seed, W.TAG_K, 0, dev)
        v = W.randn_bf16_device((B * n, Hkv, D), spec.seed, W.TAG_V, 0, dev)
        for l in range(L):
            sp.build(plan, l, k, v, bufs["table"], bufs["k_pool"], bufs["v_pool"])
        q = W.randn_bf16_device((L, B, Hq, D), spec.seed, W.TAG_Q, 0, dev)
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(D)
        seg_ms, _ = timed(lambda: sp.decode(plan, -1, q, bufs["table"], bufs["k_pool"],
                                            bufs["v_pool"], scale, o, workspace=bufs["workspace"]),
                          10)
        kv_bytes = plan.stats(-1)["decode_tokens"] * 2 * D * 2
        del bufs, plan
        # dense: [B, Hkv, n, D], the G query heads of a KV head folded into the query axis
        kd = k.view(B, n, Hkv, D).permute(0, 2, 1, 3).contiguous()
        vd = v.view(B, n, Hkv, D).permute(0, 2, 1, 3).contiguous()
        del k, v
        qd = q[0].view(B, Hkv, G, D).contiguous()
        jj = torch.arange(n, device=dev)
        masks = []
        for l in range(L):
            mm = []
            for h in range(Hkv):
                kind, s_, w_ = spec.head_class(l, h)
                m = jj <= n - 1
                if kind == W.LOCAL:
                    m = m & ((jj < s_) | (jj > n - 1 - w_))
                mm.append(m)
            masks.append(torch.stack(mm)[None, :, None, :].expand(B, Hkv, G, n).contiguous())
        with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
            def dense_all():
                for l in range(L):
                    F.scaled_dot_product_attention(qd, kd, vd, attn_mask=masks[l])
            dense_ms, _ = timed(dense_all, 3)
        del kd, vd, qd, masks, q, o
        torch.cuda.empty_cache()
        rows.append({"n": n, "segpaged_ms": round(seg_ms, 4),
                     "segpaged_kv_gbs": round(kv_bytes / (seg_ms * 1e-3) / 1e9, 1),
                     "dense_mask_ms": round(dense_ms, 4),
                     "speedup_vs_dense_mask": round(dense_ms / seg_ms, 2)})
        log(f"decode sweep N={n}: segpaged {seg_ms:.3f} ms, dense-mask {dense_ms:.3f} ms, "
            f"x{dense_ms / seg_ms:.1f}")
    return {"workload": "llama70b-shaped decode, 8 seqs x 8 layers, one all-layer call",
            "rows": rows}


def _sdpa_choice(torch, q, k, v, mask):
    """The backend torch SDPA picks on its own for these arguments."""
    try:
        from torch.nn.attention import SDPBackend
        return SDPBackend(int(torch._fused_sdp_choice(q, k, v, attn_mask=mask, dropout_p=0.0,
                                                        is_causal=False))).name
    except Exception as e:  # private API: report, do not fail
        return f"unknown ({type(e).__name__})"


def dense_mask_baseline(torch, W, pspec, dspec, k0, v0, q0, dev, pre_ms_layer, dec_ms, args, log,
                        o_pre0, q_dec, o_dec):
    """The pages' comparison path: dense K/V plus a boolean attention mask through
    torch SDPA on the same GPU. The G query heads of a KV head share its mask, so
    they are folded into the query-length axis: SDPA reads each KV head once (no
    K/V repetition). Timed on a slice and scaled linearly: a dense-mask row costs
    the same at every position. Its outputs are compared with SegPaged's on the
    same inputs (o_pre0: layer 0 of the prefill workload; o_dec: the decode
    workload's all-layer call), the equivalence check of the runtime explainer."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    res = {}
    N, Hq, Hkv, D, G = args.prefill_n, pspec.num_q_heads, pspec.num_kv_heads, pspec.head_dim, pspec.group
    R = 256
    rows = torch.arange(N - R, N, device=dev)
    j = torch.arange(N, device=dev)
    masks = []
    for h in range(Hkv):
        kind, s, w = pspec.head_class(0, h)
        m = j[None, :] <= rows[:, None]
        if kind == W.LOCAL:
            m = m & ((j[None, :] < s) | (j[None, :] > rows[:, None] - w))
        masks.append(m.repeat_interleave(G, dim=0))      # rows (position, head-in-group)
    mask = torch.stack(masks)[None]                     # [1, Hkv, R*G, N]
    q = q0[N - R:].reshape(R, Hkv, G, D).permute(1, 0, 2, 3).reshape(1, Hkv, R * G, D).contiguous()
    k = k0.permute(1, 0, 2)[None].contiguous()          # [1, Hkv, N, D]
    v = v0.permute(1, 0, 2)[None].contiguous()
    backend = "EFFICIENT_ATTENTION"
    default = _sdpa_choice(torch, q, k, v, mask)
    with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
        for _ in range(2):
            od = F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        e1.record()
        torch.cuda.synchronize()
    t_slice = e0.elapsed_time(e1) / 3
    t_layer = t_slice * N / R
    # SDPA rows (KV head, position, head in group) -> [position, Q head, D]
    od = od[0].view(Hkv, R, G, D).permute(1, 0, 2, 3).reshape(R, Hq, D)
    agree = _acc(_to_f64(o_pre0[N - R:]), _to_f64(od), rows=f"{N - R}..{N - 1} of layer 0")
    # the backend SDPA picks unforced, timed on the same slice
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    e1.record()
    torch.cuda.synchronize()
    t_default = e0.elapsed_time(e1) / 3
    res["prefill"] = {"backend": f"torch SDPA {backend}, bool mask, GQA group folded into rows",
                      "default_backend": default,
                      "default_backend_ms_slice": round(t_default, 3),
                      "rows_timed": R, "ms_slice": round(t_slice, 3),
                      "ms_per_layer_extrapolated": round(t_layer, 2),
                      "speedup_vs_dense_mask": round(t_layer / pre_ms_layer, 2),
                      "segpaged_vs_dense_mask": agree}
    log(f"dense-mask prefill agreement: cos {agree['cos']:.8f}, max|diff| "
        f"{agree['max_abs_err']:.3e}; SDPA picks {default} unforced")
    del od
    del q, k, v, mask
    log(f"dense-mask prefill: {t_layer:.1f} ms/layer (extrapolated) vs {pre_ms_layer:.1f}")
    # the same layer through our own kernel with every head global: causal
    # attention over the whole context, no block skipping -- separates the gain of
    # the kernel (dense-mask SDPA vs this) from that of the layout (this vs SegPaged)
    from dataclasses import replace as _replace
    import sparse_attention_segmentpagetable_amd as sp
    gspec = _replace(pspec, num_layers=1, kind=[W.GLOBAL] * Hkv, sink=[0] * Hkv, window=[1] * Hkv)
    gplan = sp.Plan(gspec)
    gb = gplan.allocate(dev, workspace=False)
    sp.build(gplan, 0, k0, v0, gb["table"], gb["k_pool"], gb["v_pool"])
    go = torch.empty_like(q0)
    sp.prefill(gplan, 0, q0, gb["table"], gb["k_pool"], gb["v_pool"], 1 / math.sqrt(D), go)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    sp.prefill(gplan, 0, q0, gb["table"], gb["k_pool"], gb["v_pool"], 1 / math.sqrt(D), go)
    e1.record()
    torch.cuda.synchronize()
    t_glob = e0.elapsed_time(e1)
    gflops = 4 * D * G * gplan.stats(0)["prefill_pairs"]
    res["prefill_all_global_own_kernel"] = {
        "ms_per_layer": round(t_glob, 2), "tflops": round(gflops / (t_glob * 1e-3) / 1e12, 1),
        "kernel_gain_vs_dense_mask": round(t_layer / t_glob, 2),
        "layout_gain_vs_all_global": round(t_glob / pre_ms_layer, 2)}
    log(f"all-global prefill with our kernel: {t_glob:.1f} ms/layer "
        f"({gflops / (t_glob * 1e-3) / 1e12:.0f} TF/s)")
    del gplan, gb, go
    torch.cuda.empty_cache()
    # decode: a few layers of the decode workload on dense K/V [B, Hkv, n, D]
    # decode: layers 0-3 of the decode workload, the same K/V the pages hold, as
    # dense [B, Hkv, n, D], and the same queries
    B, n = dspec.num_seqs, args.decode_n
    nl = 4
    kd = [W.randn_bf16_device((B * n, Hkv, D), dspec.seed, W.TAG_K, l, dev)
          .view(B, n, Hkv, D).permute(0, 2, 1, 3).contiguous() for l in range(nl)]
    vd = [W.randn_bf16_device((B * n, Hkv, D), dspec.seed, W.TAG_V, l, dev)
          .view(B, n, Hkv, D).permute(0, 2, 1, 3).contiguous() for l in range(nl)]
    qd = [q_dec[l].view(B, Hkv, G, D).contiguous() for l in range(nl)]
    jj = torch.arange(n, device=dev)
    dmasks = []
    for l in range(nl):
        mm = []
        for h in range(Hkv):
            kind, s, w = dspec.head_class(l, h)
            m = jj <= n - 1
            if kind == W.LOCAL:
                m = m & ((jj < s) | (jj > n - 1 - w))
            mm.append(m)
        dmasks.append(torch.stack(mm)[None, :, None, :].expand(B, Hkv, G, n).contiguous())
    ddefault = _sdpa_choice(torch, qd[0], kd[0], vd[0], dmasks[0])
    agree = []
    with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
        for l in range(nl):
            od = F.scaled_dot_product_attention(qd[l], kd[l], vd[l], attn_mask=dmasks[l])
            agree.append(_acc(_to_f64(o_dec[l]), _to_f64(od.reshape(B, Hq, D))))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for l in range(nl):
            F.scaled_dot_product_attention(qd[l], kd[l], vd[l], attn_mask=dmasks[l])
        e1.record()
        torch.cuda.synchronize()
    t_all = e0.elapsed_time(e1) / nl * args.decode_layers
    dense_bytes = 2 * B * Hkv * n * D * 2 * args.decode_layers
    res["decode"] = {"backend": f"torch SDPA {backend}, bool mask, GQA group folded into rows",
                     "default_backend": ddefault,
                     "layers_timed": nl, "ms_all_layers_extrapolated": round(t_all, 3),
                     "dense_kv_gbs": round(dense_bytes / (t_all * 1e-3) / 1e9, 1),
                     "speedup_vs_dense_mask": round(t_all / dec_ms, 2),
                     "segpaged_vs_dense_mask": dict(_merge_acc(agree), layers="0-3")}
    log(f"dense-mask decode: {t_all:.2f} ms (80 layers, extrapolated) vs {dec_ms:.3f}")
    return res


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return {d["internal_api"]: d["num_threads"] for d in threadpool_info()}
    except Exception as e:
        return f"unknown ({type(e).__name__})"


def cpu_baseline(torch, W, pspec, q0, k0, v0, args, log, o_layer0):
    """The oracle as it stands (numpy fp64, dense scores + explicit mask), timed on
    the host cores on a bounded sample: rows of layer 0 at seeded positions, all
    64 Q heads, against the full 131072-token context. The same oracle rows check
    the GPU's layer-0 output at those positions (returned under "accuracy")."""
    from oracle import attention as OA
    N = args.prefill_n
    kb = k0.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = v0.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng([pspec.seed, 77])
    cores = len(os.sched_getaffinity(0))
    done_rows, spent = 0, 0.0
    chunk = 2
    acc = []
    # edges first (sink, window and page boundaries, the last row), then seeded rows
    edges = [0, 3, 4, 63, 64, 8191, 8192, 8195, 8196, N - 1]
    while spent < args.cpu_seconds:
        if done_rows < len(edges):
            pos = np.array(edges[done_rows:done_rows + chunk])
        else:
            pos = np.sort(rng.choice(N, size=chunk, replace=False))
        idx = torch.as_tensor(pos, device=q0.device)
        qr = q0[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        ref, _ = OA.attention_rows(pspec, 0, 0, pos, qr, kb, vb)
        spent += time.perf_counter() - t0
        done_rows += chunk
        acc.append(_acc(_to_f64(o_layer0[idx]), ref))
    head_rows_per_s = done_rows * pspec.num_q_heads / spent
    tok_s = head_rows_per_s / (pspec.num_q_heads * args.prefill_layers)
    log(f"oracle: {done_rows} rows x 64 heads in {spent:.1f} s -> {tok_s:.4f} tok/s")
    return {"value": round(tok_s, 5), "unit": "tok/s", "cores": cores,
            "blas_threads": _blas_threads(), "kind": "oracle",
            "sample": (f"{done_rows} query rows of layer 0 (sink, window, page and last-row "
                       f"edges, then seeded positions), all {pspec.num_q_heads} Q heads, full "
                       f"{N}-token context; scaled to {args.prefill_layers} layers x "
                       f"{pspec.num_q_heads} heads per token"),
            "seconds": round(spent, 2),
            "accuracy": dict(_merge_acc(acc), rows=done_rows, layer=0)}


def cpu_baseline_decode(torch, W, dspec, dplan, q_dec, dev, args, log, o_dec):
    """The oracle on the decode workload: the decode row of one (sequence, layer) at a
    time, against that sequence's whole dense K/V, until about a third of the
    prefill baseline's time has passed. Rate = K/V bytes of the keys the row sees
    (bf16) per second."""
    from oracle import attention as OA
    B, n, L = dspec.num_seqs, dspec.seq_len[0], dspec.num_layers
    Hkv, D = dspec.num_kv_heads, dspec.head_dim
    rng = np.random.default_rng([dspec.seed, 78])
    done, spent, nbytes = 0, 0.0, 0
    acc = []
    while spent < args.cpu_seconds / 3:
        l, b = int(rng.integers(0, L)), int(rng.integers(0, B))
        kd = W.randn_bf16_device((B * n, Hkv, D), dspec.seed, W.TAG_K, l, dev)
        vd = W.randn_bf16_device((B * n, Hkv, D), dspec.seed, W.TAG_V, l, dev)
        kb = kd[b * n:(b + 1) * n].view(torch.int16).cpu().numpy().view(np.uint16)
        vb = vd[b * n:(b + 1) * n].view(torch.int16).cpu().numpy().view(np.uint16)
        qr = q_dec[l, b:b + 1].view(torch.int16).cpu().numpy().view(np.uint16)
        del kd, vd
        t0 = time.perf_counter()
        ref, _ = OA.attention_rows(dspec, l, b, [n - 1], qr, kb, vb)
        spent += time.perf_counter() - t0
        acc.append(_acc(_to_f64(o_dec[l, b:b + 1]), ref))
        nbytes += dplan.stats(l)["decode_tokens"] // B * 2 * D * 2
        done += 1
    gbs = nbytes / spent / 1e9
    log(f"oracle decode: {done} (sequence, layer) rows in {spent:.1f} s -> {gbs:.3f} GB/s")
    return {"value": round(gbs, 4), "unit": "GB/s", "kind": "oracle",
            "sample": (f"the decode row of {done} seeded (sequence, layer) pairs of the "
                       f"{L}-layer decode workload, each against its {n}-token dense K/V"),
            "seconds": round(spent, 2),
            "accuracy": dict(_merge_acc(acc), rows=done)}


if __name__ == "__main__":
    main()
