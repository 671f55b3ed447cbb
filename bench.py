"""Benchmark of the CSA2 decode step on one MI355X.

A step is one Full layer of the 128K-context decode workload: for 16
sequences with one query token each, the lightning indexer scores all 32,768
compressed entries (64 heads x 128, bf16), the certified top-2048 is
selected, the 2048 rows are gathered and 64 heads x 512 attend to them.  The
inputs are seeded synthetic tensors drawn on the GPU (N(0,1) keys, queries
and KV, U(0,1) head weights); several independent input sets are rotated so
that no step finds its 640 MiB of inputs in the 256 MB Infinity Cache.

Prints one JSON line: query-tokens/s of the whole step, the indexer
kernel's HBM roofline fraction (live HIP-event timing of the same launch
configuration), the attention (gather) kernel's rate, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
COPY_BYTES = 1 << 30  # counter calibration: bytes read and written by one plain copy
WORKLOAD = dict(B=16, Q=1, N=32768, HI=64, dI=128, H=64, D=512, k=2048, m=4, ctx_tokens=131072)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="independent input sets rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=["decode-128k", "decode-128k-fp4idx", "v41-decoder-1m"],
                    default="decode-128k",
                    help="decode-128k: one Full layer of the 128K-context decode (the default line); "
                         "decode-128k-fp4idx: the same with the indexer keys quantized to FP4 on the device; "
                         "v41-decoder-1m: the 20-layer V4.1 decoder schedule at a 1M-token context")
    ap.add_argument("--only", choices=["indexer", "attention", "layer", "copy"], default=None,
                    help="launch only this part, for counter collection (prints no JSON); 'copy' is a plain "
                         "1 GiB device-to-device copy that calibrates the byte counters")
    return ap.parse_args()


def make_sets(torch, n_sets, seed=1):
    W = WORKLOAD
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sets = []
    for _ in range(n_sets):
        s = {
            "kI": torch.randn(W["B"], W["N"], W["dI"], generator=g, device="cuda").to(torch.bfloat16),
            "kv": torch.randn(W["B"], W["N"], W["D"], generator=g, device="cuda").to(torch.bfloat16),
            "qI": torch.randn(W["B"], W["Q"], W["HI"], W["dI"], generator=g, device="cuda").to(torch.bfloat16),
            "w": torch.rand(W["B"], W["Q"], W["HI"], generator=g, device="cuda"),
            "q": torch.randn(W["B"], W["Q"], W["H"], W["D"], generator=g, device="cuda").to(torch.bfloat16),
        }
        sets.append(s)
    torch.cuda.synchronize()
    return sets


def event_time(torch, fn, reps):
    """Mean duration (ms) of fn() bracketed by HIP events on the current stream."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / reps


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "sparse_long_context_csa2_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_src):
    """HBM bytes per indexer launch from the committed counter summary, or None
    when it is missing or was taken on a different kernel source."""
    path = os.path.join(HERE, "profiles", "indexer_decode128k_pmc.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_src_sha") != kernel_src:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(torch, oracle, s0, budget_s):
    """Time the oracle's Full layer on the whole batch of one input set, repeated
    until about budget_s of CPU time has been spent (at least once)."""
    W = WORKLOAD
    cpu = {k: v.cpu() for k, v in s0.items()}

    def once():
        oracle.layer("FULL", k=W["k"], scale=W["D"] ** -0.5, q=cpu["q"], kv=cpu["kv"], qI=cpu["qI"], w=cpu["w"],
                     kI=cpu["kI"])

    reps, total = 0, 0.0
    while reps == 0 or total < budget_s:
        t0 = time.perf_counter()
        once()
        total += time.perf_counter() - t0
        reps += 1
    return {"value": reps * W["B"] * W["Q"] / total, "unit": "query-tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{reps} x the full batch ({W['B']} seqs x 1 query token, 32,768 entries each): Full layer "
                      f"(indexer, top-2048, attention) in binary64; {total:.1f} s total"}


E2M1_BOUNDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # the synthetic generator's midpoints between E2M1 magnitudes


def fp4_rows_gpu(torch, g, B, N, D):
    """FP4 rows [B, N, D/2 + D/16] drawn on the GPU as the synthetic generator
    does: N(0,1) values to their E2M1 codes, E4M3 scales log-uniform in
    [2^-4, 2^4]; one sequence at a time to bound the temporaries."""
    bounds = torch.tensor(E2M1_BOUNDS, device="cuda")
    out = torch.empty(B, N, D // 2 + D // 16, dtype=torch.uint8, device="cuda")
    for bb in range(B):
        x = torch.randn(N, D, generator=g, device="cuda")
        code = torch.bucketize(x.abs(), bounds, right=True).to(torch.uint8) | ((x < 0).to(torch.uint8) << 3)
        del x
        out[bb, :, : D // 2] = code[:, 0::2] | (code[:, 1::2] << 4)
        del code
        u = torch.rand(N, D // 16, generator=g, device="cuda") * 8.0 - 4.0
        ex = torch.floor(u)
        mant = torch.floor((torch.exp2(u - ex) - 1.0) * 8.0).clamp(0, 7)
        out[bb, :, D // 2:] = ((ex + 7).to(torch.uint8) << 3) | mant.to(torch.uint8)
    return out


def run_v41_decoder(a, torch, b):
    """V4.1's decoder schedule as one step: 1 Full + 3 Reuse, then 4 x (1 Reindex
    + 3 Reuse), around one persistent 16,384-position pool; every token kept
    (m = 1), so a 1M-token context is 1,048,576 entries per sequence; Full
    top-2048, Reindex top-512; FP4 main KV (64 heads x 512), bf16 indexer 64 x 128."""
    B, N, HI, dI, H, D, k, kr, P = 16, 1 << 20, 64, 128, 64, 512, 2048, 512, 16384
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    kI = torch.randn(B, N, dI, generator=g, device="cuda").to(torch.bfloat16)
    kv = fp4_rows_gpu(torch, g, B, N, D)
    scale = D ** -0.5
    modes = ["FULL"] + ["REUSE"] * 3 + (["REINDEX"] + ["REUSE"] * 3) * 4

    def qI_w():
        return (torch.randn(B, 1, HI, dI, generator=g, device="cuda").to(torch.bfloat16),
                torch.rand(B, 1, HI, generator=g, device="cuda"))

    layers, pool, idx = [], None, None
    for mode in modes:
        q = torch.randn(B, 1, H, D, generator=g, device="cuda").to(torch.bfloat16)
        if mode == "FULL":
            qi, w = qI_w()
            L = b.Layer("FULL", q=q, kv=kv, k=k, scale=scale, qI=qi, w=w, kI=kI, m=1, P=P)
            pool, idx = L.pool, L.idx
        elif mode == "REINDEX":
            qi, w = qI_w()
            L = b.Layer("REINDEX", q=q, kv=kv, k=kr, scale=scale, qI=qi, w=w, kI=kI, m=1, pool=pool)
            idx = L.idx
        else:
            L = b.Layer("REUSE", q=q, kv=kv, k=idx.shape[-1], scale=scale, idx=idx)
        layers.append(L)
    torch.cuda.synchronize()

    def step():
        for L in layers:
            L.run()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / a.steps

    full = layers[0]
    sc = torch.empty(B, 1, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, b._index_ws(b.BF16, B, 1, HI, dI, N, 0)), dtype=torch.uint8, device="cuda")
    qi0, w0 = full.tensors["qI"], full.tensors["w"]
    run_idx = lambda i: b.index_score(qi0, w0, kI, want_err=False, scores=sc, ws=ws)
    run_idx(0)
    t_idx_ms = event_time(torch, run_idx, max(10, a.steps))
    idx_bytes = B * N * dI * 2 + B * HI * (dI * 2 + 4) + B * N * 4
    gbs = idx_bytes / (t_idx_ms * 1e-3) / 1e9
    res = {
        "metric": "decode query-tokens/s through the V4.1 decoder schedule (20 layers) at 1M ctx",
        "value": B / t_step,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "V4.1 decoder schedule: 1 Full (pool 16,384, top-2048) + 3 Reuse, then 4 x "
                               "(1 Reindex top-512 + 3 Reuse); 16 seqs x 1 query, 1,048,576 entries (1M tokens, "
                               "m = 1), indexer 64x128 bf16, FP4 KV 64 heads x 512",
                   "global_batch": B, "seq_len": N},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "kernel": "indexer score of the Full layer (1,048,576 entries)",
                     "algorithmic_bytes": idx_bytes, "launch_ms": t_idx_ms},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the CSA2 step here is a single-GPU "
              f"kernel path and there is no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_long_context_csa2_amd import binding as b

    if a.workload == "v41-decoder-1m":
        run_v41_decoder(a, torch, b)
        return
    if a.only == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(a.warmup + a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {COPY_BYTES} bytes {a.warmup + a.steps} times", flush=True)
        return

    W = WORKLOAD
    scale = W["D"] ** -0.5
    sets = make_sets(torch, max(1, a.sets))
    fp4idx = a.workload == "decode-128k-fp4idx"
    if fp4idx:
        # FP4 indexer keys: the bf16 keys quantized on the device (E2M1 + E4M3 per 16 channels)
        for s in sets:
            kI = s["kI"]
            s["kI"] = b.quantize_fp4(kI.reshape(-1, W["dI"])).reshape(W["B"], W["N"], -1)
            del kI
        torch.cuda.synchronize()
    layers = [b.Layer("FULL", q=s["q"], kv=s["kv"], k=W["k"], scale=scale, qI=s["qI"], w=s["w"], kI=s["kI"])
              for s in sets]
    idx_scores = [torch.empty(W["B"], W["Q"], W["N"], dtype=torch.float32, device="cuda") for _ in sets]
    idx_ws = torch.empty(max(1, b._index_ws(b.BF16, W["B"], W["Q"], W["HI"], W["dI"], W["N"], 0)),
                         dtype=torch.uint8, device="cuda")

    def run_indexer(i):
        s = sets[i % len(sets)]
        b.index_score(s["qI"], s["w"], s["kI"], want_err=False, scores=idx_scores[i % len(sets)], ws=idx_ws)

    def run_attention(i):
        L = layers[i % len(layers)]
        b.sparse_attn(L.tensors["q"], L.tensors["kv"], L.idx, scale, out=L.out)

    if a.only:
        fn = {"indexer": run_indexer, "attention": run_attention,
              "layer": lambda i: layers[i % len(layers)].run()}[a.only]
        for L in layers:
            L.run()
        for i in range(a.warmup + a.steps):
            fn(i)
        torch.cuda.synchronize()
        print(f"ran {a.only} {a.warmup + a.steps} times", flush=True)
        return

    for i in range(a.warmup):
        layers[i % len(layers)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        layers[i % len(layers)].run()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / a.steps

    # live per-launch timing of the dominant kernel and of the gather/attention kernel
    reps = max(10, a.steps)
    for i in range(3):
        run_indexer(i)
    t_idx_ms = event_time(torch, run_indexer, reps)
    t_att_ms = event_time(torch, run_attention, reps)

    key_row = (W["dI"] // 2 + W["dI"] // 16) if fp4idx else W["dI"] * 2
    idx_bytes = (W["B"] * W["N"] * key_row              # keys
                 + W["B"] * W["Q"] * W["HI"] * (W["dI"] * 2 + 4)  # queries, weights
                 + W["B"] * W["Q"] * W["N"] * 4)        # fp32 scores written
    att_bytes = (W["B"] * W["Q"] * W["k"] * (W["D"] * 2 + 4)     # gathered rows + indices
                 + 2 * W["B"] * W["Q"] * W["H"] * W["D"] * 2)   # queries in, outputs out
    idx_gbs = idx_bytes / (t_idx_ms * 1e-3) / 1e9
    att_gbs = att_bytes / (t_att_ms * 1e-3) / 1e9
    ksrc = src_hash("indexer.hip", "common.h")
    traffic = None if fp4idx else traffic_from_profile(ksrc)

    res = {
        "metric": "decode query-tokens/s at 128K ctx + indexer/gather HBM GB/s as % of peak",
        "value": W["B"] * W["Q"] / t_step,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "CSA2 Full-layer decode, 128K tokens/seq compressed at m=4 to 32,768 entries, "
                               "16 seqs x 1 query, indexer 64x128 " + ("FP4 keys (bf16 queries)" if fp4idx else "bf16")
                               + ", top-2048, 64 heads x 512 bf16 shared KV",
                   "global_batch": W["B"] * W["Q"], "seq_len": W["ctx_tokens"], "input_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": idx_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": idx_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "indexer score (" + ("k_index_stream<64,128,FP4 keys>" if fp4idx else "k_index_stream<64,128>")
                               + ")", "algorithmic_bytes": idx_bytes,
                     "launch_ms": t_idx_ms},
        "gather": {"kernel": "attention (k_attn_mfma<512,bf16> + combine)", "achieved": att_gbs,
                   "frac": att_gbs / HBM_PEAK_GBS, "algorithmic_bytes": att_bytes, "launch_ms": t_att_ms},
        "kernel_src_sha": ksrc,
    }
    if fp4idx:
        res["metric"] = "decode query-tokens/s at 128K ctx with FP4 indexer keys + indexer HBM GB/s as % of peak"
    if not a.no_cpu_baseline and not fp4idx:
        import oracle
        res["cpu_baseline"] = cpu_baseline(torch, oracle, sets[0], a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
