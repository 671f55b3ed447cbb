"""Benchmarks of the CSA2 hot path on one MI355X.

Default line (``--workload decode-128k``): one Full layer of the 128K-context
decode -- for 16 sequences with one query token each, the lightning indexer
scores all 32,768 compressed entries (64 heads x 128, bf16), the certified
top-2048 is selected, the 2048 rows are gathered and 64 heads x 512 attend
to them.  Inputs are seeded synthetic tensors drawn on the GPU (N(0,1) keys,
queries and KV, U(0,1) head weights); nine independent input sets are
rotated so that neither the 1.2 GB of indexer keys nor the 288 MB of rows the
nine layers gather fit the 256 MB Infinity Cache between two uses.

Other workloads (one JSON line each, same fields): ``tiny-c1`` (the tiny
fp32 decode), ``decode-128k-fp4-group`` (FP4 main KV, one group of 1 Full + 5
Reuse layers, with per-layer times), ``hier-1m`` (1M-token context: a Full
layer with a 16,384-entry pool and 3 Reindex layers, batch 4),
``prefill-c5`` (a 4096-token causal chunk at a 65,536-token context,
compression included), ``decode-128k-fp4idx`` and ``v41-decoder-1m``.

Each line carries the dominant kernel's roofline fraction from live
HIP-event timing of the same launch configuration, and the CPU oracle timed
on a bounded sample of the same workload (median of three samples, with the
CPU model, the threads used and, for the decode lines, a one-thread time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix cores, published
SPIN_CYCLES = 2_000_000      # torch.cuda._sleep ahead of a timed batch: about 1 ms at the shader clock
COPY_BYTES = 1 << 30         # counter calibration: bytes read and written by one plain copy
C2 = dict(B=16, Q=1, N=32768, HI=64, dI=128, H=64, D=512, k=2048, m=4, ctx_tokens=131072)
WORKLOADS = ["decode-128k", "tiny-c1", "decode-128k-fp4-group", "hier-1m", "prefill-c5", "decode-128k-fp4idx",
             "v41-decoder-1m"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=9, help="independent input sets rotated across steps (decode-128k)")
    ap.add_argument("--cpu-seconds", type=float, default=5.0, help="target length of each oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=WORKLOADS, default="decode-128k")
    ap.add_argument("--only", choices=["indexer", "attention", "layer", "copy"], default=None,
                    help="decode-128k: launch only this part, for counter collection (prints no JSON); 'copy' is "
                         "a plain 1 GiB device-to-device copy that calibrates the byte counters")
    return ap.parse_args()


# ------------------------------------------------------------------ timing

def event_time(torch, fn, reps):
    """Mean duration (ms) per call of fn(i) over `reps` calls issued back to
    back between two HIP events on the current stream (the gaps between
    launches included).  A spin kernel queued ahead of the first event keeps
    the GPU busy while the host queues the calls, so that host-side call
    overhead does not show up as idle time, and the events' own cost is paid
    once rather than per call."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    start.record()
    for i in range(reps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def wall_time(torch, fn, warmup, steps):
    """Seconds per call of fn(i), timed over `steps` calls after `warmup`."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


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


def line(metric, value, unit, a, t_step, dtype, config, roofline, extra=None):
    res = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic", "config": config, "roofline": roofline}
    if extra:
        res.update(extra)
    return res


def hbm_roofline(kernel, nbytes, launch_ms, traffic=None, **kw):
    gbs = nbytes / (launch_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
         "traffic": traffic, "kernel": kernel, "algorithmic_bytes": nbytes, "launch_ms": launch_ms}
    r.update(kw)
    return r


def mfma_roofline(kernel, flops, launch_ms, **kw):
    tfs = flops / (launch_ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
         "frac": tfs / MFMA_BF16_PEAK_TFS, "traffic": None, "kernel": kernel, "algorithmic_flops": flops,
         "launch_ms": launch_ms}
    r.update(kw)
    return r


# ------------------------------------------------------------ CPU baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_samples(fn, budget_s, n=3):
    """n samples, each repeating fn() until about budget_s (at least once):
    per-call seconds of every sample."""
    out = []
    for _ in range(n):
        reps, total = 0, 0.0
        while reps == 0 or total < budget_s:
            t0 = time.perf_counter()
            fn()
            total += time.perf_counter() - t0
            reps += 1
        out.append(total / reps)
    return out


def one_thread_seconds(workload):
    """Seconds per oracle call of the workload's sample with one OpenMP thread
    (a child process: the oracle's thread count is fixed when it loads)."""
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = (f"import sys; sys.path.insert(0, {HERE!r}); import bench, oracle; "
            f"s = bench.oracle_sample_seconds({workload!r}); print(oracle.threads(), s)")
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
        threads, secs = r.stdout.strip().splitlines()[-1].split()
        return {"threads": int(threads), "seconds": float(secs)}
    except Exception:
        return None


def _oracle_inputs(workload):
    """CPU tensors of the oracle sample of a decode workload (seeded; the workload's shapes)."""
    import torch
    from sparse_long_context_csa2_amd import synth
    if workload == "tiny-c1":
        return synth.make_decode(synth.tiny_full(seed=0))
    if workload == "decode-128k":
        g = torch.Generator().manual_seed(1)
        W = C2
        return {"kI": torch.randn(W["B"], W["N"], W["dI"], generator=g).to(torch.bfloat16),
                "kv": torch.randn(W["B"], W["N"], W["D"], generator=g).to(torch.bfloat16),
                "qI": torch.randn(W["B"], 1, W["HI"], W["dI"], generator=g).to(torch.bfloat16),
                "w": torch.rand(W["B"], 1, W["HI"], generator=g),
                "q": torch.randn(W["B"], 1, W["H"], W["D"], generator=g).to(torch.bfloat16)}
    raise ValueError(workload)


def _oracle_fn(workload, d):
    import oracle
    if workload == "tiny-c1":
        spec, lay = d["spec"], d["layers"][0]
        return lambda: oracle.layer("FULL", k=spec.k, scale=spec.scale, q=lay["q"], kv=d["kv"], qI=lay["qI"],
                                    w=lay["w"], kI=d["kI"])
    if workload == "decode-128k":
        return lambda: oracle.layer("FULL", k=C2["k"], scale=C2["D"] ** -0.5, q=d["q"], kv=d["kv"], qI=d["qI"],
                                    w=d["w"], kI=d["kI"])
    raise ValueError(workload)


def oracle_sample_seconds(workload):
    """One call of the oracle's sample of a decode workload, in seconds (what
    the one-thread child process prints)."""
    fn = _oracle_fn(workload, _oracle_inputs(workload))
    fn()
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline_decode(workload, queries, budget_s, what):
    import oracle
    fn = _oracle_fn(workload, _oracle_inputs(workload))
    secs = timed_samples(fn, budget_s)
    med = statistics.median(secs)
    one = one_thread_seconds(workload)
    return {"value": queries / med, "unit": "query-tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "samples_s": secs, "statistic": "median of 3",
            "one_thread": None if one is None else {"value": queries / one["seconds"], **one},
            "sample": what}


# ----------------------------------------------------------------- inputs

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


def make_sets(torch, n_sets, seed=1):
    W = C2
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sets = []
    for _ in range(n_sets):
        sets.append({
            "kI": torch.randn(W["B"], W["N"], W["dI"], generator=g, device="cuda").to(torch.bfloat16),
            "kv": torch.randn(W["B"], W["N"], W["D"], generator=g, device="cuda").to(torch.bfloat16),
            "qI": torch.randn(W["B"], W["Q"], W["HI"], W["dI"], generator=g, device="cuda").to(torch.bfloat16),
            "w": torch.rand(W["B"], W["Q"], W["HI"], generator=g, device="cuda"),
            "q": torch.randn(W["B"], W["Q"], W["H"], W["D"], generator=g, device="cuda").to(torch.bfloat16),
        })
    torch.cuda.synchronize()
    return sets


def indexer_bytes(B, Q, N, HI, dI, key_row):
    """Algorithmic bytes of an indexer launch: read (keys once, queries,
    weights) and written (fp32 scores), as (read, write)."""
    return B * N * key_row + B * Q * HI * (dI * 2 + 4), B * Q * N * 4


# -------------------------------------------------------------- workloads

def run_decode_128k(a, torch, b, fp4idx=False):
    W = C2
    scale = W["D"] ** -0.5
    sets = make_sets(torch, max(1, a.sets))
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
        if a.only == "copy":
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(a.warmup + a.steps):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(f"copied {COPY_BYTES} bytes {a.warmup + a.steps} times", flush=True)
            return None
        fn = {"indexer": run_indexer, "attention": run_attention,
              "layer": lambda i: layers[i % len(layers)].run()}[a.only]
        for L in layers:
            L.run()
        for i in range(a.warmup + a.steps):
            fn(i)
        torch.cuda.synchronize()
        print(f"ran {a.only} {a.warmup + a.steps} times", flush=True)
        return None

    t_step = wall_time(torch, lambda i: layers[i % len(layers)].run(), a.warmup, a.steps)
    reps = max(2 * len(sets), a.steps)
    for i in range(3):
        run_indexer(i)
    t_idx_ms = event_time(torch, run_indexer, reps)
    t_att_ms = event_time(torch, run_attention, reps)

    key_row = (W["dI"] // 2 + W["dI"] // 16) if fp4idx else W["dI"] * 2
    rd, wr = indexer_bytes(W["B"], W["Q"], W["N"], W["HI"], W["dI"], key_row)
    att_bytes = (W["B"] * W["Q"] * W["k"] * (W["D"] * 2 + 4)     # gathered rows + indices
                 + 2 * W["B"] * W["Q"] * W["H"] * W["D"] * 2)   # queries in, outputs out
    ksrc = src_hash("indexer.hip", "common.h")
    traffic = None if fp4idx else traffic_from_profile(ksrc)
    idx_kernel = "k_index_stream<64,128" + (",FP4 keys>" if fp4idx else ">")
    roof = hbm_roofline(f"indexer score ({idx_kernel})", rd, t_idx_ms, traffic,
                        score_write_bytes=wr, score_write_note="written fp32 scores, not in algorithmic_bytes")
    gather_gbs = att_bytes / (t_att_ms * 1e-3) / 1e9
    both = (rd + att_bytes) / ((t_idx_ms + t_att_ms) * 1e-3) / 1e9
    config = {"workload": "CSA2 Full-layer decode, 128K tokens/seq compressed at m=4 to 32,768 entries, 16 seqs x 1 "
                          "query, indexer 64x128 " + ("FP4 keys (bf16 queries)" if fp4idx else "bf16")
                          + ", top-2048, 64 heads x 512 bf16 shared KV",
              "global_batch": W["B"] * W["Q"], "seq_len": W["ctx_tokens"], "input_sets": len(sets)}
    extra = {"gather": {"kernel": "attention (k_attn_split<512,bf16> + combine, given indices)",
                        "achieved": gather_gbs, "frac": gather_gbs / HBM_PEAK_GBS,
                        "algorithmic_bytes": att_bytes, "launch_ms": t_att_ms},
             "indexer_plus_gather": {"achieved": both, "frac": both / HBM_PEAK_GBS,
                                     "note": "indexer reads + gather bytes over the two launches' time"},
             "kernel_src_sha": ksrc}
    metric = "decode query-tokens/s at 128K ctx + indexer/gather HBM GB/s as % of peak"
    if fp4idx:
        metric = "decode query-tokens/s at 128K ctx with FP4 indexer keys + indexer HBM GB/s as % of peak"
    res = line(metric, W["B"] * W["Q"] / t_step, "query-tokens/s", a, t_step, "bf16", config, roof, extra)
    if not a.no_cpu_baseline and not fp4idx:
        res["cpu_baseline"] = cpu_baseline_decode(
            "decode-128k", W["B"], a.cpu_seconds,
            "the whole batch (16 seqs x 1 query token, 32,768 entries each): Full layer (indexer, top-2048, "
            "attention) in binary64, repeated to ~%gs per sample" % a.cpu_seconds)
    return res


def run_tiny_c1(a, torch, b):
    from sparse_long_context_csa2_amd import synth
    spec = synth.tiny_full(seed=0)
    d = synth.make_decode(spec)
    lay = d["layers"][0]

    def cu(t):
        return t.cuda()

    L = b.Layer("FULL", q=cu(lay["q"]), kv=cu(d["kv"]), k=spec.k, scale=spec.scale, qI=cu(lay["qI"]),
                w=cu(lay["w"]), kI=cu(d["kI"]))
    a.steps = max(a.steps, 200)
    t_step = wall_time(torch, lambda i: L.run(), a.warmup, a.steps)
    qI, w, kI = L.tensors["qI"], L.tensors["w"], L.tensors["kI"]
    sc = torch.empty(1, 1, spec.N, dtype=torch.float32, device="cuda")
    t_idx = event_time(torch, lambda i: b.index_score(qI, w, kI, want_err=False, scores=sc), a.steps)
    rd, wr = spec.N * spec.dI * 4 + spec.HI * (spec.dI * 4 + 4), spec.N * 4
    roof = hbm_roofline("indexer score (k_index_valu, fp32)", rd, t_idx, None, score_write_bytes=wr,
                        note="about 130 KB per launch: launch latency, not HBM, sets the time")
    config = {"workload": "tiny CSA2 Full-layer decode: 2048 tokens at m=4 -> 512 entries, indexer 4x64 fp32, "
                          "top-64, 8 heads x 128 fp32 KV", "global_batch": 1, "seq_len": 2048}
    res = line("decode query-tokens/s, tiny fp32 Full layer", 1 / t_step, "query-tokens/s", a, t_step, "f32",
               config, roof)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode("tiny-c1", 1, a.cpu_seconds,
                                                  "the whole tiny Full layer in binary64, repeated to ~%gs per "
                                                  "sample" % a.cpu_seconds)
    return res


def run_fp4_group(a, torch, b):
    """1 Full + 5 Reuse over FP4 main KV (16 seqs, 32,768 entries)."""
    W = C2
    B, N, HI, dI, H, D, k = W["B"], W["N"], W["HI"], W["dI"], W["H"], W["D"], W["k"]
    scale = D ** -0.5
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    sets = []
    for _ in range(3):
        kI = torch.randn(B, N, dI, generator=g, device="cuda").to(torch.bfloat16)
        kv = fp4_rows_gpu(torch, g, B, N, D)
        qI = torch.randn(B, 1, HI, dI, generator=g, device="cuda").to(torch.bfloat16)
        w = torch.rand(B, 1, HI, generator=g, device="cuda")
        qs = [torch.randn(B, 1, H, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(6)]
        full = b.Layer("FULL", q=qs[0], kv=kv, k=k, scale=scale, qI=qI, w=w, kI=kI)
        reuse = [b.Layer("REUSE", q=qs[i], kv=kv, k=k, scale=scale, idx=full.idx) for i in range(1, 6)]
        sets.append((full, reuse))
    torch.cuda.synchronize()

    def group(i):
        full, reuse = sets[i % len(sets)]
        full.run()
        for L in reuse:
            L.run()

    t_group = wall_time(torch, group, a.warmup, a.steps)
    t_full = event_time(torch, lambda i: sets[i % len(sets)][0].run(), max(12, a.steps))
    t_reuse = event_time(torch, lambda i: sets[i % len(sets)][1][i % 5].run(), max(12, a.steps))
    row = D // 2 + D // 16
    att_bytes = B * k * (row + 4) + 2 * B * H * D * 2
    roof = hbm_roofline("Reuse layer attention (k_attn_split<512,FP4> + combine)", att_bytes, t_reuse, None,
                        note="FP4 rows of 288 B; 9.4 MB gathered per layer, so the three rotated sets can sit in "
                             "the 256 MB Infinity Cache: not an HBM-only figure")
    config = {"workload": "CSA2 6-layer group (1 Full + 5 Reuse) decode at 128K tokens/seq (32,768 entries), "
                          "16 seqs x 1 query, indexer 64x128 bf16, top-2048, FP4 main KV (E2M1 + E4M3 per 16), "
                          "64 heads x 512", "global_batch": B, "seq_len": W["ctx_tokens"], "input_sets": len(sets)}
    extra = {"layers": {"full_layer_ms": t_full, "reuse_layer_ms": t_reuse, "group_ms": t_group * 1e3,
                        "reuse_share_of_group": 5 * t_reuse / (t_group * 1e3)}}
    res = line("decode query-tokens/s through a 1 Full + 5 Reuse group at 128K ctx, FP4 KV", B / t_group,
               "query-tokens/s", a, t_group, "bf16", config, roof, extra)
    if not a.no_cpu_baseline:
        import oracle
        full, reuse = sets[0]
        sl = slice(0, 2)  # two of the 16 sequences
        cpu = {"q": [full.tensors["q"][sl].cpu()] + [L.tensors["q"][sl].cpu() for L in reuse],
               "kv": full.tensors["kv"][sl].cpu(), "qI": full.tensors["qI"][sl].cpu(),
               "w": full.tensors["w"][sl].cpu(), "kI": full.tensors["kI"][sl].cpu()}

        def fn():
            r = oracle.layer("FULL", k=k, scale=scale, q=cpu["q"][0], kv=cpu["kv"], qI=cpu["qI"], w=cpu["w"],
                             kI=cpu["kI"])
            for qq in cpu["q"][1:]:
                oracle.layer("REUSE", k=k, scale=scale, q=qq, kv=cpu["kv"], idx=r["idx"])

        secs = timed_samples(fn, a.cpu_seconds)
        res["cpu_baseline"] = {"value": 2 / statistics.median(secs), "unit": "query-tokens/s",
                               "cores": oracle.threads(), "kind": "oracle", "cpu_model": cpu_model(),
                               "samples_s": secs, "statistic": "median of 3",
                               "sample": "2 of the 16 sequences through the whole group in binary64"}
    return res


def run_hier_1m(a, torch, b):
    """1M tokens at m=4 (262,144 entries), batch 4: Full (pool 16,384, top-2048) + 3 Reindex (top-2048)."""
    B, N, HI, dI, H, D, k, P = 4, 262144, 64, 128, 64, 512, 2048, 16384
    scale = D ** -0.5
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    kI = torch.randn(B, N, dI, generator=g, device="cuda").to(torch.bfloat16)
    kv = fp4_rows_gpu(torch, g, B, N, D)

    def qiw():
        return (torch.randn(B, 1, HI, dI, generator=g, device="cuda").to(torch.bfloat16),
                torch.rand(B, 1, HI, generator=g, device="cuda"),
                torch.randn(B, 1, H, D, generator=g, device="cuda").to(torch.bfloat16))

    qi, w, q = qiw()
    full = b.Layer("FULL", q=q, kv=kv, k=k, scale=scale, qI=qi, w=w, kI=kI, P=P)
    layers = [full]
    for _ in range(3):
        qi, w, q = qiw()
        layers.append(b.Layer("REINDEX", q=q, kv=kv, k=k, scale=scale, qI=qi, w=w, kI=kI, pool=full.pool))
    torch.cuda.synchronize()

    def group(i):
        for L in layers:
            L.run()

    a.steps = min(a.steps, 20)
    t_group = wall_time(torch, group, min(a.warmup, 3), a.steps)
    sc = torch.empty(B, 1, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, b._index_ws(b.BF16, B, 1, HI, dI, N, 0)), dtype=torch.uint8, device="cuda")
    t_idx = event_time(torch, lambda i: b.index_score(full.tensors["qI"], full.tensors["w"], kI, want_err=False,
                                                       scores=sc, ws=ws), 10)
    t_full = event_time(torch, lambda i: full.run(), 10)
    t_rei = event_time(torch, lambda i: layers[1 + i % 3].run(), 12)
    rd, wr = indexer_bytes(B, 1, N, HI, dI, dI * 2)
    roof = hbm_roofline("Full-layer indexer score (k_index_stream<64,128>, 262,144 entries)", rd, t_idx, None,
                        score_write_bytes=wr)
    config = {"workload": "1M-token hierarchical indexer: 4 seqs x 1 query, 1,048,576 tokens at m=4 -> 262,144 "
                          "entries, bf16 indexer 64x128, Full layer top-2048 + 16,384-entry pool, 3 Reindex layers "
                          "top-2048 of the pool, FP4 main KV 64 heads x 512", "global_batch": B, "seq_len": 1 << 20}
    extra = {"layers": {"full_layer_ms": t_full, "reindex_layer_ms": t_rei, "group_ms": t_group * 1e3}}
    res = line("decode query-tokens/s through Full + 3 Reindex at 1M ctx", B / t_group, "query-tokens/s", a,
               t_group, "bf16", config, roof, extra)
    if not a.no_cpu_baseline:
        import oracle
        cpu = {n: full.tensors[n][:1].cpu() for n in ("q", "qI", "w")}
        kI1, kv1 = kI[:1].cpu(), kv[:1].cpu()

        def fn():
            oracle.layer("FULL", k=k, scale=scale, q=cpu["q"], kv=kv1, qI=cpu["qI"], w=cpu["w"], kI=kI1, P=P)

        secs = timed_samples(fn, a.cpu_seconds)
        res["cpu_baseline"] = {"value": 1 / statistics.median(secs), "unit": "query-tokens/s (Full layer only)",
                               "cores": oracle.threads(), "kind": "oracle", "cpu_model": cpu_model(),
                               "samples_s": secs, "statistic": "median of 3",
                               "sample": "1 of the 4 sequences through the Full layer (262,144 entries, pool and "
                                         "top-2048) in binary64; the Reindex layers are not included"}
    return res


def run_prefill_c5(a, torch, b):
    """A 4096-token causal chunk at the end of a 65,536-token context: compress
    the KV and indexer keys (m=4, two-group windows), then one Full layer."""
    from sparse_long_context_csa2_amd import synth
    spec = synth.Prefill(seed=4)
    T, m, Qc, D, dI, HI, H, k = spec.T, spec.m, spec.Qc, spec.D, spec.dI, spec.HI, spec.H, spec.k
    n_ent = T // m
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    x = torch.randn(T, D, generator=g, device="cuda").to(torch.bfloat16)
    xI = torch.randn(T, dI, generator=g, device="cuda").to(torch.bfloat16)
    wz = (torch.randn(D, D, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    wzI = (torch.randn(dI, dI, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    bias = torch.randn(2 * m, D, generator=g, device="cuda") * 0.02
    biasI = torch.randn(2 * m, dI, generator=g, device="cuda") * 0.02
    qI = torch.randn(1, Qc, HI, dI, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(1, Qc, H, D, generator=g, device="cuda").to(torch.bfloat16)
    w = torch.rand(1, Qc, HI, generator=g, device="cuda")
    q_pos = torch.arange(T - Qc, T, dtype=torch.int64, device="cuda").view(1, Qc)
    kv = torch.empty(n_ent, D, dtype=torch.bfloat16, device="cuda")
    kI = torch.empty(n_ent, dI, dtype=torch.bfloat16, device="cuda")
    b.compress(x, n_ent, m, 0, wz, bias, out=kv)
    b.compress(xI, n_ent, m, 0, wzI, biasI, out=kI)
    kv3, kI3 = kv.view(1, n_ent, D), kI.view(1, n_ent, dI)
    L = b.Layer("FULL", q=q, kv=kv3, k=k, scale=spec.scale, qI=qI, w=w, kI=kI3, q_pos=q_pos, m=m)
    torch.cuda.synchronize()

    def step(i):
        b.compress(x, n_ent, m, 0, wz, bias, out=kv)
        b.compress(xI, n_ent, m, 0, wzI, biasI, out=kI)
        L.run()

    a.steps = min(a.steps, 20)
    a.warmup = min(a.warmup, 3)
    t_step = wall_time(torch, step, a.warmup, a.steps)
    sc = torch.empty(1, Qc, n_ent, dtype=torch.float32, device="cuda")
    t_idx = event_time(torch, lambda i: b.index_score(qI, w, kI3, q_pos=q_pos, m=m, want_err=False, scores=sc), 5)
    t_att = event_time(torch, lambda i: b.sparse_attn(q, kv3, L.idx, spec.scale, out=L.out), 5)
    t_cmp = event_time(torch, lambda i: b.compress(x, n_ent, m, 0, wz, bias, out=kv), 5)
    pos = torch.arange(T - Qc, T, dtype=torch.float64)
    vis = torch.clamp(torch.floor((pos + 1) / m), max=n_ent)
    idx_flops = 2.0 * float(vis.sum()) * HI * dI
    att_flops = 4.0 * Qc * k * H * D
    cmp_flops = 2.0 * T * D * D
    roof = mfma_roofline("prefill attention (k_attn_tiles<512,32,2>: S and O on bf16 matrix cores)", att_flops, t_att)
    config = {"workload": "prefill chunk: 4096 causal query tokens at the end of a 65,536-token context; bf16 KV "
                          "(512) and indexer keys (128) compressed at m=4 over two-group windows; indexer 64x128, "
                          "top-2048, 64 heads x 512", "global_batch": Qc, "seq_len": T}
    extra = {"kernels": {
        "indexer": mfma_roofline("k_index_prefill<64,128>", idx_flops, t_idx),
        "attention": mfma_roofline("k_attn_tiles<512,32,2>", att_flops, t_att),
        "compress_kv": mfma_roofline("k_compress_mfma<512> (+ W transpose)", cmp_flops, t_cmp)}}
    res = line("prefill tokens/s (4096-token chunk at 64K ctx, compression included)", Qc / t_step, "tokens/s",
               a, t_step, "bf16", config, roof, extra)
    if not a.no_cpu_baseline:
        import oracle
        nq = 8
        rows = torch.linspace(0, Qc - 1, nq).round().long().cuda()
        kvc, kIc = kv3.cpu(), kI3.cpu()
        cq = {"q": q[:, rows].cpu(), "qI": qI[:, rows].cpu(), "w": w[:, rows].cpu(), "q_pos": q_pos[:, rows].cpu()}
        xs, xIs = x[: 256 * m].cpu(), xI[: 256 * m].cpu()
        wzc, wzIc, bc, bIc = wz.cpu(), wzI.cpu(), bias.cpu(), biasI.cpu()

        def f_layer():
            oracle.layer("FULL", k=k, scale=spec.scale, q=cq["q"], kv=kvc, qI=cq["qI"], w=cq["w"], kI=kIc,
                         q_pos=cq["q_pos"], m=m)

        def f_cmp():
            oracle.compress(xs, 256, m, 0, wzc, bc)
            oracle.compress(xIs, 256, m, 0, wzIc, bIc)

        s_layer = timed_samples(f_layer, a.cpu_seconds / 2)
        s_cmp = timed_samples(f_cmp, a.cpu_seconds / 2)
        est = statistics.median(s_layer) * Qc / nq + statistics.median(s_cmp) * n_ent / 256
        res["cpu_baseline"] = {"value": Qc / est, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
                               "cpu_model": cpu_model(), "statistic": "median of 3 per part",
                               "samples_s": {"layer_8_queries": s_layer, "compress_256_entries": s_cmp},
                               "sample": "Full layer of 8 of the 4096 query tokens and compression of 256 of the "
                                         "16,384 entries (KV and keys) in binary64, scaled to the whole chunk"}
    return res


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

    def step(i):
        for L in layers:
            L.run()

    t_step = wall_time(torch, step, a.warmup, a.steps)
    full = layers[0]
    sc = torch.empty(B, 1, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, b._index_ws(b.BF16, B, 1, HI, dI, N, 0)), dtype=torch.uint8, device="cuda")
    qi0, w0 = full.tensors["qI"], full.tensors["w"]
    t_idx_ms = event_time(torch, lambda i: b.index_score(qi0, w0, kI, want_err=False, scores=sc, ws=ws),
                          max(10, a.steps))
    rd, wr = indexer_bytes(B, 1, N, HI, dI, dI * 2)
    roof = hbm_roofline("indexer score of the Full layer (1,048,576 entries)", rd, t_idx_ms, None,
                        score_write_bytes=wr)
    config = {"workload": "V4.1 decoder schedule: 1 Full (pool 16,384, top-2048) + 3 Reuse, then 4 x "
                          "(1 Reindex top-512 + 3 Reuse); 16 seqs x 1 query, 1,048,576 entries (1M tokens, "
                          "m = 1), indexer 64x128 bf16, FP4 KV 64 heads x 512", "global_batch": B, "seq_len": N}
    res = line("decode query-tokens/s through the V4.1 decoder schedule (20 layers) at 1M ctx", B / t_step,
               "query-tokens/s", a, t_step, "bf16", config, roof)
    res["cpu_baseline"] = None
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the CSA2 step here is a single-GPU "
              f"kernel path and there is no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_long_context_csa2_amd import binding as b

    run = {"decode-128k": lambda: run_decode_128k(a, torch, b),
           "decode-128k-fp4idx": lambda: run_decode_128k(a, torch, b, fp4idx=True),
           "tiny-c1": lambda: run_tiny_c1(a, torch, b),
           "decode-128k-fp4-group": lambda: run_fp4_group(a, torch, b),
           "hier-1m": lambda: run_hier_1m(a, torch, b),
           "prefill-c5": lambda: run_prefill_c5(a, torch, b),
           "v41-decoder-1m": lambda: run_v41_decoder(a, torch, b)}[a.workload]
    res = run()
    if res is not None:
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
