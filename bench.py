"""Benchmark: batch-1 greedy lookahead decoding at the LLaMA-2-7B shape.

Workload (synthetic, seeded): random-init bf16 LLaMA-2-7B-shaped decoder
(32 layers, d 4096, 32 heads, FFN 11008, vocab 32000); 128-token prompt of
Zipf(1.1) ids with 3 repeated 16-token spans; lookahead N=5, W=15, G=15 with
the prompt's n-grams seeded into the pool; 256 new greedy tokens per
generation.

One bench step = one lookahead decoding step (one la_step: candidate gather,
one forward pass over M = 121 rows, verification, KV commit, window slide,
pool insert).  Prefills happen before the timed region.  `value` = emitted
tokens / wall time of the K timed steps.

Also reported: step compression S, the same engine's autoregressive
tokens/s and the speedup over it, per-step HBM bytes / time, the roofline
of the dominant kernel (the projection GEMM) from per-launch HIP events, and
the CPU oracle's greedy AR tokens/s on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batch-1 greedy tokens/sec at 7B shape (N=5,W=15,G=15); step compression; HBM GB/s"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--ar-steps", type=int, default=256)
    ap.add_argument("--shape", default="llama7b")
    ap.add_argument("--N", type=int, default=5)
    ap.add_argument("--W", type=int, default=15)
    ap.add_argument("--G", type=int, default=15)
    ap.add_argument("--prompt-len", type=int, default=128)
    ap.add_argument("--prompt", choices=["auto", "zipf", "code"], default="auto",
                    help="prompt recipe: Zipf(1.1) ids with repeated spans, or code-like lines "
                         "(20 lines of 24 ids from a 2000-id sub-vocabulary, 40%% repeated); "
                         "auto: code for the 13B shape, Zipf otherwise")
    ap.add_argument("--max-new", type=int, default=256)
    ap.add_argument("--profile-steps", type=int, default=32)
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-tokens", type=int, default=48)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: sampling verification (Algorithm 4) at this temperature, "
                         "for lookahead and AR alike; 0: greedy")
    ap.add_argument("--seed", type=int, default=0, help="key of the sampling draws")
    ap.add_argument("--top-k", type=int, default=0, help="sampling: top-K cut (0 = none)")
    ap.add_argument("--top-p", type=float, default=0.0, help="sampling: top-P cut (0 = none)")
    ap.add_argument("--pool-lru", action="store_true",
                    help="evict pool n-grams by recency instead of FIFO (LA_POOL_LRU)")
    ap.add_argument("--adaptive", choices=["on", "off"], default="on",
                    help="also time the configuration with LA_ADAPTIVE_G (the adaptive_G field)")
    ap.add_argument("--pool-cap", type=int, default=0,
                    help="suffixes kept per first token (0 = G)")
    ap.add_argument("--pool-study", action="store_true",
                    help="instead: step compression S against the pool cap, eviction policy "
                         "(FIFO, recency) and selection rule (newest, by context) on the small "
                         "random-init models whose greedy output "
                         "repeats n-grams (micro, tiny), eight motif prompts each")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: step time against the row count "
                         "M over a grid of (N, W = G), one JSON line per configuration")
    ap.add_argument("--sweep-steps", type=int, default=32)
    ap.add_argument("--scaling-fit", action="store_true",
                    help="step compression S of the small random-init models over N and W = G "
                         "through the C-ABI, checked against the oracle's values in "
                         "tests/golden/scaling_points.json, and the Eq. 5/7 fit of (alpha, f)")
    ap.add_argument("--attention", action="store_true",
                    help="instead: time the lookahead attention call alone (32 heads, head_dim 128, "
                         "bf16) at prefixes 512, 2048, 8192 for (N, W, G) = (5, 15, 15) and (7, 7, 7)")
    ap.add_argument("--gemm", action="store_true",
                    help="instead: time the projection GEMM call alone (split-K product and its "
                         "piece reduction) for the shape's four projection weights at the step's "
                         "row count and at one row, cold weights")
    ap.add_argument("--calibrate", choices=["on", "off"], nargs="?", const="on", default="on",
                    help="first run a 1 GiB HBM read (la_probe_read): the achievable read "
                         "bandwidth the fractions are also reported against, and the "
                         "known-size kernel that scales the PMC byte counters")
    ap.add_argument("--seed-sweep", type=int, default=5,
                    help="also report S over this many prompt seeds (0 = off)")
    return ap.parse_args()


def calibrate():
    """Known-size kernels: read 1 GiB with la_probe_read, write 1 GiB with a
    fill.  Returns the measured read bandwidth (GB/s)."""
    import torch
    from exact_decoding_amd import binding as B
    n = 1 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.zeros(B.LA_PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    # the first reads of a process run below the settled rate: 20 untimed
    for _ in range(20):
        B.la_probe_read(buf, n, out, None)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        B.la_probe_read(buf, n, out, None)
    e1.record()
    torch.cuda.synchronize()
    gbps = reps * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return gbps


PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_llama7b_lookahead_pmc.md")
GEMM_SOURCE = os.path.join(ROOT, "exact_decoding_amd", "csrc", "k_gemm.hip")


def gemm_traffic():
    """HBM bytes per k_gemm_bf16 launch from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source has changed since the
    counters were taken (or there is no summary)."""
    import hashlib
    try:
        text = open(PMC_SUMMARY).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l)
    if fields.get("k_gemm.hip sha256", "").strip() != src:
        return None
    return float(fields["traffic bytes per launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_steps(sessions_factory, K, sync):
    """Run exactly K steps over pre-prefilled sessions; returns (seconds,
    tokens, steps_per_session_seen)."""
    sessions = sessions_factory()
    it = iter(sessions)
    ses = next(it)
    sync()
    t0 = time.perf_counter()
    tokens = 0
    for _ in range(K):
        if ses.done:
            ses = next(it)
        tokens += len(ses.step())
    sync()
    dt = time.perf_counter() - t0
    for s in sessions:
        s.close()
    return dt, tokens


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and the cores this process
    may run on (its affinity mask)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return model, len(os.sched_getaffinity(0))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_tiny():
    """The oracle (as it stands) on the tiny fp32 workload: whole greedy AR
    (32 new tokens) and whole lookahead (N=3, W=4, G=4, prompt as reference)
    after the 16-token motif prompt, on one BLAS thread and on all of them."""
    import synth
    from oracle import lookahead as la
    from oracle.model import OracleModel
    from threadpoolctl import threadpool_limits
    s = synth.SHAPES["tiny"]
    om = OracleModel(s, synth.gen_weights(s, 0))
    prompt = synth.prompt_motif(s.vocab, seed=1)
    win = synth.gen_window(3, 4, s.vocab, seed=2)
    out = {}
    for label, nthreads in (("1_thread", 1), ("all_threads", host_cpu()[1])):
        with threadpool_limits(limits=nthreads):
            t0 = time.perf_counter()
            ar = la.greedy_ar(om, prompt, 32)
            t_ar = time.perf_counter() - t0
            t0 = time.perf_counter()
            r = la.lookahead(om, prompt, 3, 4, 4, 32, win, prompt_ref=True)
            t_la = time.perf_counter() - t0
        out[label] = {"threads": nthreads, "ar_tokens_per_s": len(ar.tokens) / t_ar,
                      "lookahead_tokens_per_s": len(r.tokens) / t_la, "lookahead_S": r.S,
                      "lookahead_equals_ar": r.tokens == ar.tokens,
                      "pool": {"inserts": r.pool.inserts, "dup_skips": r.pool.dup_skips,
                               "evictions": r.pool.evictions, "ngrams": r.pool.n_ngrams()}}
    return out


def cpu_baseline(shape, weights, prompt, n_tokens):
    """Oracle greedy AR (as it stands) on a bounded sample: the first
    `n_tokens` decode steps after the prompt, prefill excluded from timing."""
    import numpy as np
    from oracle.model import OracleModel, causal_vis, argmax_lowest
    from oracle import lookahead as la
    cpu_model, host_cores = host_cpu()
    cores = min(blas_threads(), host_cores)
    om = OracleModel(shape, weights)
    # keep decoded float64 weights only when the host has room for them
    try:
        mem_kb = int([l for l in open("/proc/meminfo") if l.startswith("MemAvailable")][0].split()[1])
    except Exception:
        mem_kb = 0
    need = sum(int(np.prod(w.shape)) for w in weights) * 8
    om.keep = mem_kb * 1024 > 2.5 * need
    cache, cur = la.prefill(om, prompt)
    P = cache[0][0].shape[0]
    t0 = time.perf_counter()
    for _ in range(n_tokens):
        logits, kv = om.forward([cur], [P], causal_vis(P, 1), past=cache)
        cache = [(np.concatenate([K, k]), np.concatenate([V, v])) for (K, V), (k, v) in zip(cache, kv)]
        P += 1
        cur = int(argmax_lowest(logits)[0])
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{shape.name} greedy AR, {n_tokens} decode tokens after the "
                      f"{len(prompt)}-token prompt (prefill untimed), float64 numpy, "
                      f"weights {'decoded once' if om.keep else 'decoded per call'}",
            "cpu_model": cpu_model, "host_cores": host_cores,
            "tiny_fp32": cpu_tiny()}


SWEEP_N = (3, 5, 7)
SWEEP_W = (1, 2, 4, 7, 10, 15, 20, 30)
# [LD] Table 3 (LLaMA-2-7B-Chat, MT-Bench, one A100): label, N, W, G, prompt as
# reference, the S and the speedup the pages report
TABLE3 = [("3", 10, 1, 3, True, 1.45, 1.36), ("4", 5, 1, 10, True, 1.51, 1.36),
          ("5", 5, 1, 30, False, 1.12, 1.04), ("6", 5, 1, 30, True, 1.59, 1.46),
          ("7", 5, 30, 1, False, 1.79, 1.61), ("8", 5, 15, 15, False, 1.96, 1.78),
          ("9", 5, 15, 15, True, 2.05, 1.88)]


def sweep(args, model, shape, prompt):
    """Step time of the engine against M = 1 + (W + G)(N - 1) (G = W), next to
    the AR step: the ratio is the compression S a model must reach for the
    lookahead step to pay off at that configuration on this GPU."""
    import synth
    K = args.sweep_steps

    def time_steps(N, W, G, ar, prompt_ref=True):
        ses = model.session(prompt, N, W, G, K + 8, ar=ar,
                            window=None if ar else synth.gen_window(N, W, shape.vocab, seed=2),
                            prompt_ref=prompt_ref and not ar)
        for _ in range(4):
            ses.step()
        n0, s0 = len(ses.tokens), len(ses.per_step)
        import torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            if ses.done:
                break
            ses.step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        steps = len(ses.per_step) - s0
        S = (len(ses.tokens) - n0) / max(steps, 1)
        rows = ses.rows
        ses.close()
        return dt * 1e3 / max(steps, 1), S, rows

    from exact_decoding_amd import planner
    ar_ms, _, _ = time_steps(5, 0, 0, True)
    log(f"[sweep] AR step {ar_ms:.3f} ms")
    table = []
    for N in SWEEP_N:
        for W in SWEEP_W:
            if 1 + 2 * W * (N - 1) > 2048:
                continue
            ms, S, rows = time_steps(N, W, W, False)
            # the pages' acceptance model (Eq. 5/7 at their fitted alpha, f)
            # turned into a speedup on this GPU by the measured step costs
            S_pred = planner.compression(planner.PAGES_ALPHA, N, W, planner.PAGES_F)
            table.append({"N": N, "W": W, "step_ms": ms})
            print(json.dumps({"shape": shape.name, "N": N, "W": W, "G": W, "M": rows,
                              "step_ms": ms, "ar_step_ms": ar_ms, "break_even_S": ms / ar_ms,
                              "measured_S": S, "pages_model_S": S_pred,
                              "pages_model_speedup": S_pred * ar_ms / ms}), flush=True)
    best = planner.best_config(table, ar_ms)
    print(json.dumps({"shape": shape.name, "best_under_pages_model": best,
                      "alpha": planner.PAGES_ALPHA, "f": planner.PAGES_F}), flush=True)
    # the pages' ablation configurations (Table 3 ③-⑨, several with G != W):
    # the step each costs here and, with the S the pages measured for it,
    # the speedup it would give on this GPU
    for label, N, W, G, ref, S_pages, sp_pages in TABLE3:
        ms, S, rows = time_steps(N, W, G, False, prompt_ref=ref)
        print(json.dumps({"shape": shape.name, "table3": label, "N": N, "W": W, "G": G,
                          "prompt_ref": ref, "M": rows, "step_ms": ms, "ar_step_ms": ar_ms,
                          "break_even_S": ms / ar_ms, "measured_S": S, "pages_S": S_pages,
                          "pages_speedup_A100": sp_pages,
                          "speedup_here_at_pages_S": S_pages * ar_ms / ms}), flush=True)
    return {"rows": table, "ar_ms": ar_ms}


def attention_cpu_leg(bufs, out, P, N, W, G, H, hd):
    """The oracle's attention (float64 numpy, the lookahead mask
    materialised) on the same call's inputs: its time per call on the host,
    and the largest difference of the GPU's bf16 output from it."""
    import numpy as np
    import torch
    from oracle.attention import lookahead_attention
    q, kc, vc, kb, vb = (t.float().cpu().numpy() for t in bufs)
    M = q.shape[0]
    args = (q.reshape(M, H, hd), kc[:, :P].transpose(1, 0, 2), vc[:, :P].transpose(1, 0, 2),
            kb.reshape(M, H, hd), vb.reshape(M, H, hd), N, W, G)
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = lookahead_attention(*args)
        reps += 1
        dt = time.perf_counter() - t0
        if dt > 1.0 or reps == 3:
            break
    err = float(np.abs(out.float().cpu().numpy().reshape(M, H, hd) - ref).max())
    return {"value": dt / reps * 1e6, "unit": "us per call", "cores": min(blas_threads(), host_cpu()[1]),
            "kind": "oracle", "sample": f"the same call (P = {P}, {M} rows, {H} heads), float64 numpy "
                                        f"with the mask materialised, {reps} call(s)",
            "gpu_max_abs_err": err}


def attention_bench(read_gbps, cpu_leg=True):
    """The attention call alone (both kernels) on seeded N(0, 1) bf16 data,
    rotating over enough buffer sets that the K/V working set exceeds the
    256 MB memory-side cache; bytes per call = the prefix K and V plus q,
    block K/V and the output.  With `cpu_leg`, each line also carries the
    oracle's time for the same call and the GPU output's largest error
    against it."""
    import torch
    from exact_decoding_amd import binding as B
    H, hd = 32, 128
    g = torch.Generator(device="cuda").manual_seed(7)
    for P in (512, 2048, 8192):
        for (N, W, G) in ((5, 15, 15), (7, 7, 7)):
            M = 1 + (W + G) * (N - 1)
            ld = P + 64
            kv_set = 2 * H * ld * hd * 2
            nset = max(4, -(-600_000_000 // kv_set))
            sets = []
            for _ in range(nset):
                sets.append(tuple(torch.randn(*shp, device="cuda", generator=g).to(torch.bfloat16)
                                  for shp in ((M, H * hd), (H, ld, hd), (H, ld, hd), (M, H * hd),
                                              (M, H * hd))))
            out = torch.empty(M, H * hd, device="cuda", dtype=torch.bfloat16)
            ws = torch.empty(max(B.la_kernel_attention_ws_bytes(ld, H, hd, N, W, G, B.LA_BF16), 4),
                             dtype=torch.uint8, device="cuda")

            def run(i):
                q, kc, vc, kb, vb = sets[i % nset]
                B.la_kernel_attention(q, kc, vc, P, ld, kb, vb, out, H, H, hd, N, W, G, B.LA_BF16,
                                      ws, None)
            for i in range(2 * nset):
                run(i)
            torch.cuda.synchronize()
            it = 50
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(it):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / it * 1e3
            nbytes = 16384 * P + 4 * M * H * hd * 2
            gbps = nbytes / (us * 1e-6) / 1e9
            cpu = None
            if cpu_leg:
                run(0)
                torch.cuda.synchronize()
                cpu = attention_cpu_leg(sets[0], out, P, N, W, G, H, hd)
            print(json.dumps({"kernel": "lookahead attention (MFMA prefix part + per-row part)",
                              "P": P, "N": N, "W": W, "G": G, "rows": M, "us_per_call": us,
                              "bytes_per_call": nbytes, "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
                              "frac_of_achievable": gbps / read_gbps if read_gbps else None,
                              "buffer_sets": nset, "cpu_baseline": cpu}), flush=True)
            del sets, out, ws
            torch.cuda.empty_cache()


def gemm_bench(shape, rows, read_gbps, reps=10):
    """The projection GEMM call alone (la_kernel_gemm: the split-K product,
    then the in-order sum of its pieces) on seeded N(0, 0.02) bf16 weights of
    the shape's QKV, O, gate/up and down matrices, at `rows` rows and at one
    row.  Three weight sets rotate so every call streams cold weights.
    Bytes per call = weights + x + the float32 output."""
    import torch
    from exact_decoding_amd import binding as B
    d, F = shape.d_model, shape.d_ff
    nqkv = (shape.n_heads + 2 * shape.n_kv_heads) * shape.head_dim
    mats = (("QKV", nqkv, d), ("O", d, shape.n_heads * shape.head_dim), ("gate/up", 2 * F, d),
            ("down", d, F))
    g = torch.Generator(device="cuda").manual_seed(11)
    nset = 3
    for name, N, K in mats:
        sets = []
        for _ in range(nset):
            w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            dst = torch.empty(B.la_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
            B.la_pack_weight(w, N, K, dst, None)
            del w
            sets.append(dst)
        torch.cuda.synchronize()
        for M in (rows, 1):
            x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
            y = torch.empty(M, N, dtype=torch.float32, device="cuda")
            ws = torch.empty(max(B.la_kernel_gemm_ws_bytes(M, K, N), 4), dtype=torch.uint8,
                             device="cuda")
            for i in range(nset):
                B.la_kernel_gemm(x, M, K, sets[i % nset], N, y, B.LA_BF16, ws, None)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps * nset):
                B.la_kernel_gemm(x, M, K, sets[i % nset], N, y, B.LA_BF16, ws, None)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / (reps * nset) * 1e3
            nbytes = N * K * 2 + M * K * 2 + M * N * 4
            gbps = nbytes / (us * 1e-6) / 1e9
            print(json.dumps({"kernel": "projection GEMM call (product + piece sum)",
                              "matrix": name, "N": N, "K": K, "rows": M, "us_per_call": us,
                              "bytes_per_call": nbytes, "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
                              "frac_of_achievable": gbps / read_gbps if read_gbps else None}),
                  flush=True)
            del x, y, ws
        del sets
        torch.cuda.empty_cache()


def scaling_fit(sweep_table=None):
    """[LD] §4 "Scaling Law": S = tokens / steps measured through the C-ABI
    on the small random-init models that repeat n-grams, for the (N, W = G)
    grid of tests/golden/scaling_points.json; every S must equal the
    oracle's value there (the fp32 engine reproduces the oracle's steps);
    then (alpha, f) of Eq. 5/7 fitted per model, its residual, and the
    configuration the fitted model favours on the measured 7B step times."""
    import synth
    from exact_decoding_amd import planner
    from exact_decoding_amd.runtime import Model
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "scaling_points.json")))
    rec = gold["recipe"]
    fits = {}
    for name, pts in gold["models"].items():
        s = synth.SHAPES[name]
        model = Model(s, synth.gen_weights(s, 0))
        prompts = [synth.prompt_motif(s.vocab, seed=k) for k in range(rec["prompts"])]
        trip, equal = [], True
        for p in pts:
            N, W, G = p["N"], p["W"], p["G"]
            win = synth.gen_window(N, W, s.vocab, seed=2)
            toks = steps = 0
            for pr in prompts:
                ses = model.session(pr, N, W, G, rec["new_tokens"], window=win, prompt_ref=True)
                toks += len(ses.decode())
                steps += ses.stats()["steps"]
                ses.close()
            equal = equal and toks == p["tokens"] and steps == p["steps"]
            trip.append((N, W, toks / steps))
        model.close()
        alpha, f = planner.fit(trip)
        res = [planner.compression(alpha, n, w, f) - S for n, w, S in trip]
        rms = (sum(r * r for r in res) / len(res)) ** 0.5
        fits[name] = (alpha, f)
        out = {"study": "scaling-law fit", "shape": name, "points": len(trip),
               "equal_to_oracle": equal, "alpha": alpha, "f": f, "rms_residual": rms,
               "max_residual": max(abs(r) for r in res),
               "S": [[n, w, round(S, 4)] for n, w, S in trip]}
        if sweep_table:
            out["best_on_7b_steps"] = planner.best_config(sweep_table["rows"], sweep_table["ar_ms"],
                                                          alpha, f)
        print(json.dumps(out), flush=True)
    return fits


def pool_study(N=4, W=5, G=5, n_new=128, seeds=8):
    """S = tokens / steps of whole generations against the pool cap, its
    eviction policy and the candidate selection rule (the newest G, or by
    context first), on the random-init micro (vocab 8) and tiny (vocab 256)
    models, whose greedy continuations of a repeated-motif prompt repeat
    n-grams (the 7B-shape random model repeats none, so its S is 1 under any
    pool).  Also checks that every generation equals the same engine's AR
    decode, which the pool cannot change."""
    import synth
    from exact_decoding_amd.runtime import Model
    for name in ("micro", "tiny"):
        s = synth.SHAPES[name]
        model = Model(s, synth.gen_weights(s, 0))
        win = synth.gen_window(N, W, s.vocab, seed=2)
        prompts = [synth.prompt_motif(s.vocab, seed=k) for k in range(seeds)]
        ar = []
        for pr in prompts:
            ses = model.session(pr, N, W, G, n_new, ar=True)
            ar.append(ses.decode())
            ses.close()
        for cap, lru, ctx in [(c, l, x) for c in (1, 2, G, 2 * G, 4 * G) for l in (False, True)
                              for x in (False, True)]:
            S, ev, exact = [], 0, True
            for pr, ref in zip(prompts, ar):
                ses = model.session(pr, N, W, G, n_new, window=win, prompt_ref=True,
                                    pool_cap=cap, pool_lru=lru, pool_context=ctx)
                toks = ses.decode()
                st = ses.stats()
                ses.close()
                exact = exact and toks == ref
                S.append(st["tokens"] / st["steps"])
                ev += st["evictions"]
            print(json.dumps({"study": "pool cap and eviction policy", "shape": name,
                              "N": N, "W": W, "G": G, "new_tokens": n_new, "pool_cap": cap,
                              "policy": "lru" if lru else "fifo",
                              "selection": "context" if ctx else "newest",
                              "S_mean": sum(S) / len(S),
                              "S_per_prompt": [round(v, 4) for v in S],
                              "evictions_total": ev, "lookahead_equals_ar": exact}),
                  flush=True)
        # wall clock of whole generations (graph replay, default pool): does
        # the compression turn into tokens/s over the same engine's AR decode?
        import torch

        def timed(make):
            sessions = [make(pr) for pr in prompts]  # prefilled before the clock
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = sum(len(ses.decode()) for ses in sessions)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            steps = sum(ses.stats()["steps"] for ses in sessions)
            for ses in sessions:
                ses.close()
            return n / dt, dt * 1e3 / steps, n / steps

        for _ in range(2):  # the first round warms the graphs and caches
            la_tps, la_ms, la_S = timed(lambda pr: model.session(pr, N, W, G, n_new, window=win,
                                                                 prompt_ref=True))
            ar_tps, ar_ms, _ = timed(lambda pr: model.session(pr, N, W, G, n_new, ar=True))
        print(json.dumps({"study": "lookahead vs AR wall clock", "shape": name, "N": N, "W": W,
                          "G": G, "new_tokens": n_new, "prompts": seeds, "S": la_S,
                          "lookahead_tokens_per_s": la_tps, "ar_tokens_per_s": ar_tps,
                          "speedup": la_tps / ar_tps, "lookahead_ms_per_step": la_ms,
                          "ar_ms_per_step": ar_ms}), flush=True)
        model.close()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    from exact_decoding_amd.runtime import Model, upload

    shape = synth.SHAPES[args.shape]
    N, W, G = args.N, args.W, args.G
    read_gbps = None
    if args.calibrate == "on":
        read_gbps = calibrate()
        log(f"[bench] calibration: 1 GiB read at {read_gbps:.0f} GB/s")
    if args.attention:
        attention_bench(read_gbps, cpu_leg=args.cpu_baseline == "on")
        return
    if args.gemm:
        gemm_bench(shape, 1 + (W + G) * (N - 1), read_gbps)
        return
    if args.pool_study:
        pool_study()
        return
    if args.scaling_fit and not args.sweep:
        scaling_fit()
        return
    t0 = time.time()
    log(f"[bench] generating + uploading {shape.name} weights")
    weights_np = []
    dev = []
    n_w = len(synth.weight_names(shape))
    t_log = time.time()
    for i in range(n_w):
        w = synth.gen_tensor(shape, 0, i)
        dev.append(upload(w))
        if args.cpu_baseline == "on":
            weights_np.append(w)
        if time.time() - t_log > 30:
            t_log = time.time()
            log(f"[bench] {i + 1}/{n_w} tensors after {t_log - t0:.0f}s")
    torch.cuda.synchronize()
    log(f"[bench] weights ready in {time.time() - t0:.1f}s")
    model = Model(shape, dev)
    recipe = args.prompt if args.prompt != "auto" else ("code" if shape.name == "codellama13b" else "zipf")

    def make_prompt(seed):
        if recipe == "code":
            return synth.prompt_code_lines(shape.vocab, length=args.prompt_len, seed=seed)
        return synth.prompt_zipf_spans(shape.vocab, length=args.prompt_len, seed=seed)
    prompt = make_prompt(1)
    window = synth.gen_window(N, W, shape.vocab, seed=2)
    graph = not args.no_graph
    if args.sweep:
        table = sweep(args, model, shape, prompt)
        if args.scaling_fit:
            model.close()
            scaling_fit(table)
        return
    sync = torch.cuda.synchronize

    def la_session():
        return model.session(prompt, N, W, G, args.max_new, window=window, prompt_ref=True,
                             graph=graph, temperature=args.temperature, seed=args.seed,
                             top_k=args.top_k, top_p=args.top_p, pool_cap=args.pool_cap,
                             pool_lru=args.pool_lru)

    def ar_session():
        return model.session(prompt, N, W, G, args.max_new, ar=True, graph=graph,
                             temperature=args.temperature, seed=args.seed, top_k=args.top_k,
                             top_p=args.top_p)

    # warmup + steps per generation
    log("[bench] warmup")
    ses = la_session()
    for _ in range(args.warmup):
        if ses.done:
            break
        ses.step()
    ses.decode()
    gen_stats = ses.stats()
    gen_steps = gen_stats["steps"]
    pool_stats = {k: gen_stats[k] for k in ("inserts", "dup_skips", "evictions", "pool_ngrams",
                                             "pool_keys_nonempty", "gathers_nonempty", "cand_total")
                  if k in gen_stats}
    la_tokens_ref = list(ses.tokens)
    ses.close()
    S = args.max_new / gen_steps
    log(f"[bench] one generation: {gen_steps} steps, S = {S:.3f}; {len(set(la_tokens_ref))} distinct "
        f"tokens; first 48: {la_tokens_ref[:48]}; last 24: {la_tokens_ref[-24:]}")

    n_sess = math.ceil(args.steps / gen_steps) + 1
    log(f"[bench] timing {args.steps} lookahead steps over {n_sess} pre-filled sessions")
    dt, toks = timed_steps(lambda: [la_session() for _ in range(n_sess)], args.steps, sync)
    la_tps = toks / dt
    ms_per_step = dt * 1e3 / args.steps
    log(f"[bench] lookahead: {toks} tokens in {dt:.3f}s -> {la_tps:.1f} tok/s, {ms_per_step:.3f} ms/step")

    ar_steps = args.ar_steps
    n_ar = math.ceil(ar_steps / args.max_new) + 1
    ses = ar_session()
    for _ in range(min(args.warmup, args.max_new - 1)):
        ses.step()
    ses.close()
    dt_ar, toks_ar = timed_steps(lambda: [ar_session() for _ in range(n_ar)], ar_steps, sync)
    ar_tps = toks_ar / dt_ar
    log(f"[bench] autoregressive: {toks_ar} tokens in {dt_ar:.3f}s -> {ar_tps:.1f} tok/s, "
        f"{dt_ar * 1e3 / ar_steps:.3f} ms/step")

    # the same configuration with LA_ADAPTIVE_G: each step computes candidate
    # rows only as far as its candidates need (every token, step and pool
    # counter as with the fixed width)
    adaptive = None
    if args.temperature == 0 and args.adaptive == "on":
        def la_adaptive():
            return model.session(prompt, N, W, G, args.max_new, window=window, prompt_ref=True,
                                 graph=graph, pool_cap=args.pool_cap, pool_lru=args.pool_lru,
                                 adaptive_g=True)
        ses = la_adaptive()
        toks_a = ses.decode()
        st_a = ses.stats()
        ses.close()
        dt_a, toks_ad = timed_steps(lambda: [la_adaptive() for _ in range(n_sess)], args.steps, sync)
        adaptive = {"tokens_per_s": toks_ad / dt_a, "ms_per_step": dt_a * 1e3 / args.steps,
                    "rows_per_step_mean": st_a["rows_total"] / st_a["steps"],
                    "rows_per_step_max": 1 + (W + G) * (N - 1),
                    "equals_fixed_width": toks_a == la_tokens_ref and st_a["steps"] == gen_steps,
                    "speedup_vs_ar": (toks_ad / dt_a) / ar_tps}
        log(f"[bench] adaptive G: {toks_ad} tokens in {dt_a:.3f}s -> {toks_ad / dt_a:.1f} tok/s, "
            f"{dt_a * 1e3 / args.steps:.3f} ms/step, {adaptive['rows_per_step_mean']:.1f} rows/step")

    # exactness spot check: the lookahead stream equals the AR stream
    ses = ar_session()
    ar_tokens_ref = ses.decode()
    ses.close()
    # (with sampling the two streams are different draws of one distribution)
    exact = ar_tokens_ref == la_tokens_ref if args.temperature == 0 else None

    # prefill of the prompt alone (eager session set-up: no graph capture)
    t_pf = []
    for _ in range(3):
        sync()
        t1 = time.perf_counter()
        ses = model.session(prompt, N, W, G, args.max_new, window=window, prompt_ref=True,
                            graph=False)
        sync()
        t_pf.append((time.perf_counter() - t1) * 1e3)
        ses.close()
    prefill_ms = sorted(t_pf)[1]
    log(f"[bench] prefill of {len(prompt)} tokens: {prefill_ms:.2f} ms")

    # step compression over prompt seeds 0.. (one whole generation each)
    S_seeds = []
    for ps in range(args.seed_sweep):
        pr = make_prompt(ps)
        ses = model.session(pr, N, W, G, args.max_new, window=window, prompt_ref=True,
                            graph=graph, temperature=args.temperature, seed=args.seed,
                            top_k=args.top_k, top_p=args.top_p)
        ses.decode()
        st = ses.stats()
        ses.close()
        S_seeds.append(st["tokens"] / st["steps"])
    if S_seeds:
        log(f"[bench] S over prompt seeds 0..{args.seed_sweep - 1}: {S_seeds}")

    # per-kernel profile (HIP events around every launch, same stream)
    ses = la_session()
    agg = None
    n_prof = 0
    P_sum = 0
    while not ses.done and n_prof < args.profile_steps:
        P_sum += len(prompt) - 1 + len(ses.tokens)
        _, prof = ses.step_profile()
        n_prof += 1
        if agg is None:
            agg = {k: dict(v) for k, v in prof.items()}
        else:
            for k, v in prof.items():
                for f in v:
                    agg[k][f] += v[f]
    ses.close()
    P_avg = P_sum / max(n_prof, 1)
    # the dominant kernel is the projection GEMM at M = 121 (k_gemm4, or
    # k_gemm_dma for the short-run shapes); its launches are the four
    # projections per layer plus the LM head
    g = {f: agg["gemm"][f] + agg["lm_head"][f] for f in agg["gemm"]}
    gemm_ms = g["ms"] / g["launches"]
    gemm_bytes = g["bytes"] / g["launches"]
    gemm_gbps = g["bytes"] / (g["ms"] * 1e-3) / 1e9
    prof_total_ms = sum(v["ms"] for v in agg.values()) / n_prof
    breakdown = {k: {"ms_per_step": v["ms"] / n_prof, "launches_per_step": v["launches"] / n_prof,
                     "GBps": (v["bytes"] / (v["ms"] * 1e-3) / 1e9) if v["ms"] > 0 else None}
                 for k, v in agg.items()}
    log("[bench] profile per step: " + json.dumps(breakdown))

    # per-step algorithmic HBM bytes (weights + embedding rows + KV read + KV write)
    es = 2 if shape.dtype == "bf16" else 4
    M = 1 + (W + G) * (N - 1)
    wbytes = sum(int(np.prod(s_)) for n_, s_ in zip(synth.weight_names(shape), synth.weight_shapes(shape))
                 if n_ != "emb") * es
    kv_row = 2 * shape.n_layers * shape.n_kv_heads * shape.head_dim * es
    step_bytes = wbytes + M * shape.d_model * es + kv_row * P_avg + kv_row * S
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if args.cpu_baseline == "on":
        log("[bench] CPU oracle baseline")
        del dev
        cpu = cpu_baseline(shape, weights_np, prompt, args.cpu_tokens)
        log(f"[bench] cpu baseline: {cpu}")

    out = {
        "metric": METRIC if (shape.name, N, W, G) == ("llama7b", 5, 15, 15) else
                  f"batch-1 greedy tokens/sec at {shape.name} shape (N={N},W={W},G={G}); "
                  f"step compression; HBM GB/s",
        "value": la_tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"lookahead decoding step, {shape.name} shape random-init, batch 1, "
                               f"prompt {len(prompt)} " + ("code-like lines (40% repeated)" if recipe == "code" else "Zipf(1.1)+3 repeated spans") + ", prompt as reference, "
                               f"{args.max_new} new tokens per generation",
                   "prompt": recipe, "N": N, "W": W, "G": G, "rows_per_step": M,
                   "parallelism": "single GPU",
                   "graph": graph, "temperature": args.temperature, "top_k": args.top_k,
                   "top_p": args.top_p, "pool": "lru" if args.pool_lru else "fifo",
                   "pool_cap": args.pool_cap or G},
        "pool_one_generation": pool_stats,
        "step_compression": S,
        "step_compression_prompt_seeds": S_seeds,
        "prefill_ms": prefill_ms,
        "ar_tokens_per_s": ar_tps,
        "speedup_vs_ar": la_tps / ar_tps,
        "lookahead_equals_ar": exact,
        "adaptive_G": adaptive,
        "step_hbm": {"bytes_per_step": step_bytes, "GBps": step_gbps, "frac": step_gbps / HBM_PEAK_GBPS,
                     "frac_of_achievable": step_gbps / read_gbps if read_gbps else None,
                     "P_avg": P_avg},
        "roofline": {"kernel": "projection GEMM (k_gemm4 / k_gemm_dma) at M = 121 (QKV, O, gate/up, down and LM head)",
                     "bound": "hbm",
                     "achieved": gemm_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gemm_gbps / HBM_PEAK_GBPS, "traffic": gemm_traffic(),
                     "frac_of_achievable": gemm_gbps / read_gbps if read_gbps else None,
                     "avg_launch_ms": gemm_ms, "avg_launch_bytes": gemm_bytes,
                     "mfma_tflops": g["flops"] / (g["ms"] * 1e-3) / 1e12},
        "profile_ms_per_step": breakdown,
        "profile_step_ms_eager": prof_total_ms,
        "achievable_read_GBps": read_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
