#!/usr/bin/env python3
"""Benchmark of the decoder step on one MI355X.

Default workload: the 8B-class GQA decoder (hidden 4096, 32 layers, 32/8
heads of 128, SwiGLU 14336, vocab 128256, bf16 weights ~N(0, 0.02),
synthetic): a 2048-token random prompt prefilled in chunks of 128, then
batch-1 greedy decode steps with the bf16 KV cache.  One "step" is one
decode step (every row of the hot path: embedding, 32 x [RMSNorm, QKV,
RoPE + KV append, attention, o_proj + residual, RMSNorm, SwiGLU FFN +
residual], final norm, lm-head, argmax).

Prints ONE JSON line: decode tokens/s (value), prefill tokens/s, the
roofline of the dominant kernel measured live with HIP events (the
library's per-node timers) and the fp64 oracle timed on a bounded sample
on the host cores.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s @bs1 (% HBM peak) + prefill tok/s (% MFMA peak), 8B-shape GQA"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources of the batch-1 projection kernel (the dominant decode kernel)
KERNEL_SOURCES = ("gemv.hip", "common.h", "launch.h")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decoder_only_transformer_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if absent or taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def measure_prefill(dec, ids, chunk, stream, ev0, ev1, runs):
    """Whole prompt in chunks of `chunk` (median of `runs` after one untimed
    run), then once more with the per-node timers for the MFMA figures."""
    import torch
    chunks = [ids[i:i + chunk] for i in range(0, len(ids), chunk)]

    def prompt_once():
        pos = 0
        for ci, ch in enumerate(chunks):
            dec.prefill_chunk(0, ch, pos, logits_mode=1 if ci == len(chunks) - 1 else 0)
            pos += len(ch)

    times = []
    for run in range(1 + runs):
        dec.kv_reset(-1)
        torch.cuda.synchronize()
        ev0.record(stream)
        prompt_once()
        ev1.record(stream)
        torch.cuda.synchronize()
        if run:
            times.append(ev0.elapsed_time(ev1) * 1e-3)
    dec.kv_reset(-1)
    dec.stats_enable()
    prompt_once()
    pst = dec.stats_read()
    dec.stats_enable(())
    torch.cuda.synchronize()
    t_pre = statistics.median(times)
    flops = sum(v["flops"] for v in pst.values())
    gemm_nodes = ("qkv", "o", "gate_up", "down", "head", "router", "experts")
    g_ms = sum(pst[n]["ms"] for n in gemm_nodes)
    g_fl = sum(pst[n]["flops"] for n in gemm_nodes)
    g_by = sum(pst[n]["bytes"] for n in gemm_nodes)
    chunk_bytes = g_by / len(chunks)
    chunk_flops = g_fl / len(chunks)
    ceiling = min(1.0, (chunk_flops / (MFMA_BF16_PEAK_TFS * 1e12)) / (chunk_bytes / (HBM_PEAK_GBS * 1e9)))
    return {"tok_s": len(ids) / t_pre, "ms": t_pre * 1e3, "prompt": len(ids), "chunk": chunk,
            "tflops": flops / t_pre / 1e12, "mfma_frac": flops / t_pre / 1e12 / MFMA_BF16_PEAK_TFS,
            "gemm_tflops": g_fl / (g_ms * 1e-3) / 1e12,
            "gemm_mfma_frac": g_fl / (g_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
            "gemm_mfma_frac_executed": 2 * g_fl / (g_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
            "gemm_hbm_frac": g_by / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "chunk_mfma_ceiling": ceiling, "nodes": summarize_nodes(pst)}


def measure_gemm_capability(shape, rows, stream, ev0, ev1, reps=20):
    """The prefill projection kernel on the gate/up shape at `rows` rows
    (C[rows][2I] = A W^T, K = H; packed weights, no split): TFLOP/s with
    plain bf16 activations (one MFMA per product) and with the split-bf16
    activations the model runs (hi and lo planes, two MFMAs per product)."""
    import torch
    from decoder_only_transformer_step_amd.binding import diag_gemm_chunk, diag_pack_w32
    N, K = 2 * shape.ffn_inter, shape.hidden
    g = torch.Generator(device="cuda").manual_seed(5)
    A = (torch.randn((2, rows, K), device="cuda", generator=g) * 0.5).to(torch.bfloat16).view(torch.int16)
    Wt = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    P = torch.empty_like(Wt)
    diag_pack_w32(Wt, P, stream.cuda_stream)
    del Wt
    C = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    out = {"rows": rows, "N": N, "K": K}
    for m in sorted({128, rows}):
        res = {}
        for planes in (1, 2):
            a = A[:planes, :m].contiguous()
            diag_gemm_chunk(a, P, C[:m], 1, None, stream.cuda_stream)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(reps):
                diag_gemm_chunk(a, P, C[:m], 1, None, stream.cuda_stream)
            ev1.record(stream)
            torch.cuda.synchronize()
            s = ev0.elapsed_time(ev1) * 1e-3 / reps
            fl = 2.0 * m * N * K
            res[f"planes{planes}"] = {"us": s * 1e6, "tflops_algorithmic": fl / s / 1e12,
                                      "mfma_frac_algorithmic": fl / s / 1e12 / MFMA_BF16_PEAK_TFS,
                                      "mfma_frac_executed": planes * fl / s / 1e12 / MFMA_BF16_PEAK_TFS}
            log(f"[gpu] gemm {m}x{N}x{K} planes {planes}: {s * 1e6:.1f} us, "
                f"{fl / s / 1e12:.0f} TFLOP/s algorithmic")
        if m == rows:
            out.update(res)
        out[f"rows{m}"] = res
    del A, P, C
    # context only, not part of the path: the vendor library's bf16 GEMM
    # (torch's linear on this machine, fp32 accumulate, bf16 output) on the same
    # shapes at the workload's chunk (128 rows) and at `rows` rows
    import torch.nn.functional as F
    W = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    lib = {}
    for m in sorted({128, rows}):
        X = (torch.randn((m, K), device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        with torch.cuda.stream(stream):
            F.linear(X, W)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(reps):
                F.linear(X, W)
            ev1.record(stream)
        torch.cuda.synchronize()
        s = ev0.elapsed_time(ev1) * 1e-3 / reps
        fl = 2.0 * m * N * K
        lib[f"rows{m}"] = {"us": s * 1e6, "tflops": fl / s / 1e12, "mfma_frac": fl / s / 1e12 / MFMA_BF16_PEAK_TFS}
        log(f"[gpu] library bf16 gemm {m}x{N}x{K}: {s * 1e6:.1f} us, {fl / s / 1e12:.0f} TFLOP/s")
        del X
    out["library_reference"] = lib
    del W
    torch.cuda.empty_cache()
    return out


def measure_verify(dec, shape, stream, ev0, ev1, reps, ns=(2, 4, 8)):
    """Multi-position verify, the check of speculatively drafted tokens
    (pipeline.rs Pipeline::forward_pair and measure_pair_fusion): n drafted
    positions go through one prefill_chunk call with every row's logits and
    greedy id, and kv_truncate rolls the sequence back; against n single
    decode steps at the same positions, also rolled back.  Milliseconds per
    round from HIP events over `reps` rounds after one untimed round."""
    import torch
    from synth.weights import prompt
    L = dec.seq_len(0)
    nmax = max(ns)
    logits = torch.empty((nmax, shape.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(nmax, dtype=torch.int32, device="cuda")
    drafts = [int(t) for t in prompt(shape, nmax, seq=123)]
    out = {"position": L, "reps": reps}

    def timed(fn):
        for rep in range(reps + 1):
            if rep == 1:
                torch.cuda.synchronize()
                ev0.record(stream)
            fn()
            dec.kv_truncate(0, L)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    for n in ns:
        if L + n > shape.max_seq or n > shape.max_chunk:
            continue
        v_ms = timed(lambda: dec.prefill_chunk(0, drafts[:n], L, logits_mode=2, logits=logits, argmax=am))

        def singles():
            for i in range(n):
                dec.decode_step([0], [drafts[i]], logits=logits[i:i + 1], argmax=am[i:i + 1])
        s_ms = timed(singles)
        # one more verify pass with the per-node timers on
        dec.stats_enable()
        dec.prefill_chunk(0, drafts[:n], L, logits_mode=2, logits=logits, argmax=am)
        vst = dec.stats_read()
        dec.stats_enable(())
        dec.kv_truncate(0, L)
        torch.cuda.synchronize()
        out[f"n{n}"] = {"verify_ms": round(v_ms, 4), "singles_ms": round(s_ms, 4),
                        "positions_per_s": round(n / v_ms * 1e3, 1),
                        "speedup_vs_singles": round(s_ms / v_ms, 3), "nodes": summarize_nodes(vst)}
        log(f"[gpu] verify {n} positions: {v_ms:.3f} ms ({n / v_ms * 1e3:.0f} positions/s), "
            f"{n} single decode steps {s_ms:.3f} ms")
    return out


def measure_graph(dec, shape, n_steps):
    """Graph-replayed decode: decode_run captures one greedy step into a HIP
    graph and replays it, against the eager decode_step loop of the timed
    region.  Each call is synchronous and includes its capture and
    instantiation, so the replay cost per step is the difference of a long
    and a short run over the difference of their lengths (host clock, median
    of three pairs); every run starts from the same position."""
    import torch
    L = dec.seq_len(0)
    short = 8
    if n_steps <= short or L < 1 or L + n_steps > shape.max_seq:
        return None
    toks = torch.empty(n_steps, dtype=torch.int32, device="cuda")

    def run(n):
        # a rollback forgets the greedy token, so the last position is
        # decoded again (untimed) with a fixed token to start the run from
        dec.kv_truncate(0, L - 1)
        dec.decode_step([0], [1])
        torch.cuda.synchronize()
        t = time.perf_counter()
        dec.decode_run(0, n, toks)
        return time.perf_counter() - t

    run(short)                                   # untimed: first capture on this decoder
    pairs = [(run(short), run(n_steps)) for _ in range(3)]
    step_s = statistics.median([(b - a) / (n_steps - short) for a, b in pairs])
    call_s = statistics.median([b for _, b in pairs])
    out = {"position": L, "steps": n_steps, "replay_ms_per_step": round(step_s * 1e3, 4),
           "tok_s": round(1.0 / step_s, 2), "call_ms": round(call_s * 1e3, 3),
           "call_tok_s": round(n_steps / call_s, 2),
           "timing": f"host clock; per step = (t({n_steps}) - t({short})) / {n_steps - short}, median of 3"}
    log(f"[gpu] graph decode {out['tok_s']:.1f} tok/s per replayed step "
        f"({out['call_tok_s']:.1f} tok/s for a whole {n_steps}-step call)")
    return out


def cpu_baseline(shape, n_prefill, n_decode):
    """The fp64 oracle (unchanged) on the host cores: a chunk of n_prefill
    prompt tokens, then n_decode greedy decode steps; tokens/s of the decode
    steps (and of the prefill) over the tokens actually run."""
    import oracle
    from synth.weights import host_weights, prompt
    t0 = time.time()
    W = host_weights(shape)
    log(f"[cpu] host weights generated in {time.time() - t0:.1f}s")
    m = oracle.Model(shape, W, max_seq=n_prefill + n_decode + 1)
    ids = prompt(shape, n_prefill)
    t0 = time.perf_counter()
    out = m.forward(ids, 0)
    t_pre = time.perf_counter() - t0
    tok = oracle.argmax(out["logits"])
    t0 = time.perf_counter()
    for i in range(n_decode):
        out = m.forward([tok], n_prefill + i)
        tok = oracle.argmax(out["logits"])
    t_dec = time.perf_counter() - t0
    del m, W
    return {"value": n_decode / t_dec, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{shape.name}: fp64 oracle, one {n_prefill}-token prefill chunk "
                      f"({n_prefill / t_pre:.3f} tok/s) then {n_decode} decode steps at positions "
                      f"{n_prefill}..{n_prefill + n_decode - 1}; value = decode tok/s",
            "prefill_tok_s": n_prefill / t_pre, "seconds": t_pre + t_dec}


def summarize_nodes(st):
    out = {}
    for n, v in st.items():
        if v["launches"]:
            ms = v["ms"] / v["launches"]
            out[n] = {"launches": v["launches"], "avg_us": round(ms * 1e3, 2),
                      "GBps": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["ms"] else None,
                      "TFps": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["ms"] else None,
                      "ms_total": round(v["ms"], 3)}
    return out


# ------------------------------------------------ profile summaries --
# Text summaries of rocprofv3 output for the profiles folder: the per-kernel
# statistics of a --kernel-trace --stats run, and the HBM bytes of the
# dominant kernel from two --pmc runs (FETCH_SIZE, WRITE_SIZE), scaled by
# what the same counters read for a plain device copy of known size.

def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _short_name(n):
    m = re.search(r"(\w+)(<[^>]*>)?\(", n)
    return (m.group(1) + (m.group(2) or "")) if m else n[:60]


def summarize_stats(stats_csv, bench_json, out, command, plain_json=None):
    rows = _read_csv(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    res = json.loads(open(bench_json).read().strip().splitlines()[-1]) if bench_json else None
    lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", "", "```", command, "```", ""]
    if res:
        rf = res["roofline"]
        lines += [f"bench line: value {res['value']} {res['unit']}, ms_per_step {res['ms_per_step']}, "
                  f"workload {res['config']['workload']}", "",
                  f"bench roofline kernel: {rf['kernel']}: avg {rf['avg_us']} us per launch over "
                  f"{rf['launches']} sampled launches (HIP events), {rf['achieved']} GB/s, frac {rf['frac']}", ""]
    if plain_json:
        r2 = json.loads(open(plain_json).read().strip().splitlines()[-1])
        rf2 = r2["roofline"]
        lines += [f"the same bench without the profiler (`python bench.py`): value {r2['value']} {r2['unit']}, "
                  f"roofline avg {rf2['avg_us']} us per launch over {rf2['launches']} sampled launches, "
                  f"{rf2['achieved']} GB/s, frac {rf2['frac']}", ""]
    lines += ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:25]:
        lines.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def _counter_per_dispatch(path, pattern, counter):
    """Average counter value (KiB) per dispatch of kernels whose name matches."""
    vals, grids = {}, {}
    for r in _read_csv(path):
        if r.get("Counter_Name") != counter or not re.search(pattern, r["Kernel_Name"]):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        grids[key] = int(r.get("Grid_Size", "0") or 0)
    return vals, grids


def summarize_counters(fetch_csv, write_csv, kernel_pattern, copy_bytes, algo_bytes, out, commands):
    copy_pat = r"copyBuffer|elementwise|copy"
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        kv, _ = _counter_per_dispatch(path, kernel_pattern, name)
        cv, cg = _counter_per_dispatch(path, copy_pat, name)
        # the calibration copy: the dispatches with the largest grid
        big = max(cg.values())
        cvals = [cv[k] for k in cv if cg[k] == big]
        kib_copy = statistics.mean(cvals)
        factor = copy_bytes / (kib_copy * 1024.0)
        kib = statistics.mean(kv.values())
        res[name] = {"dispatches": len(kv), "kib_per_dispatch": kib, "copy_kib": kib_copy,
                     "copy_dispatches": len(cvals), "factor": factor, "bytes": kib * 1024.0 * factor}
    traffic = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    lines = ["# HBM traffic of the dominant decode kernel (rocprofv3 --pmc)", "",
             "Commands (from the repository root), one counter per run:", ""]
    lines += ["```"] + commands + ["```", ""]
    lines += [f"kernel: `{kernel_pattern}` (regex on the kernel name)", "",
              f"calibration: a plain device copy of {copy_bytes} bytes in the same process "
              "(the counters of its dispatches give the scale factor bytes / (KiB x 1024))", "",
              "| counter | kernel dispatches | KiB per dispatch | copy KiB | factor | bytes per launch |",
              "|---|---:|---:|---:|---:|---:|"]
    for name, r in res.items():
        lines.append(f"| {name} | {r['dispatches']} | {r['kib_per_dispatch']:.0f} | {r['copy_kib']:.0f} | "
                     f"{r['factor']:.4f} | {r['bytes']:.4g} |")
    lines += ["", f"algorithmic bytes per launch: {algo_bytes:.6g}",
              f"traffic / algorithmic: {traffic / algo_bytes:.4f}", "",
              f"traffic_bytes_per_launch: {traffic:.6g}",
              f"kernel_source_sha256: {kernel_source_hash()}", ""]
    open(out, "w").write("\n".join(lines) + "\n")


def summarize_mfma(pmc_csv, out, commands):
    """MFMA work of the prefill chunk projections from one rocprofv3 --pmc run
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 MFMA work in units of 512 flops;
    durations from the same run's dispatch timestamps)."""
    import collections
    import csv
    disp = collections.defaultdict(dict)
    for r in csv.DictReader(open(pmc_csv)):
        name = r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "")
        name = re.sub(r"\([^()]*\)$", "", name)
        d = disp[r["Dispatch_Id"]]
        d["name"], d["grid"] = name, int(r["Grid_Size"])
        d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    # one group per GEMM shape: same kernel, same grid, same MFMA work per dispatch
    groups = collections.defaultdict(list)
    for d in disp.values():
        groups[(d["name"], d["grid"], d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))].append(d)
    lines = ["# MFMA work of the prefill chunk projections (rocprofv3 --pmc)", "",
             "Command (from the repository root):", "", "```"] + commands + ["```", "",
             "`gemm_chunk_kernel<MT, EPI, SPLIT, GR>` (GR: the grouped MoE form) and "
             "`gemm_wide_kernel<EPI, SPLIT>` (chunks of 256+ rows): EPI 0 = plain product (the bench's "
             "gate_up GEMM capability probe), 1 = residual add (o_proj, down), 2 = SwiGLU (gate_up), "
             "3 = QKV. One row per GEMM shape (kernel, grid size, MFMA work per dispatch). The model's "
             "activations enter the MFMAs as two bf16 planes (SPLIT), so their executed flops are twice "
             "the algorithmic 2 M N K.", "",
             f"peak: {MFMA_BF16_PEAK_TFS:.0f} TFLOP/s dense bf16", "",
             "| kernel | grid | dispatches | avg us (counter run) | MFMA flops / dispatch | executed TFLOP/s | "
             "% of peak | MFMA-busy cycles / dispatch |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, grid, mops), ds in sorted(groups.items()):
        busy = statistics.mean(d.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) for d in ds)
        t = statistics.mean(d["dur"] for d in ds)
        tfs = mops * 512 / t / 1e12
        lines.append(f"| `{name}` | {grid} | {len(ds)} | {t * 1e6:.2f} | {mops * 512:.4g} | {tfs:.1f} | "
                     f"{100 * tfs / MFMA_BF16_PEAK_TFS:.1f} | {busy:.4g} |")
    open(out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default: the workload's decode steps minus the first "
                         "step and the warmup)")
    ap.add_argument("--warmup", type=int, default=3, help="untimed decode steps before timing")
    ap.add_argument("--workload", default="8b", help="8b (default), 135m, tiny, moe, longctx")
    ap.add_argument("--prefill-runs", type=int, default=5, help="timed whole-prompt prefills (median)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill measurement: the decode context is a synthetic N(0,1) KV "
                         "prefix of the prompt's length (for counter runs of the decode kernels)")
    ap.add_argument("--sliding-window", type=int, default=0,
                    help="attention variant: every query sees only the W most recent positions")
    ap.add_argument("--attn-softcap", type=float, default=0.0, help="attention variant: logit soft-cap")
    ap.add_argument("--attn-sinks", action="store_true", help="attention variant: per-head sink logits")
    ap.add_argument("--qk-norm", action="store_true", help="attention variant: per-head RMSNorm of q and k")
    ap.add_argument("--weight-quant", nargs="?", const=8, type=int, default=0, choices=(0, 8, 4),
                    help="quantised weights: 8 = int8 with a power-of-two scale per row, 4 = 4-bit with a "
                         "power-of-two scale per group of 32 (decode streams the codes)")
    ap.add_argument("--kv-page", type=int, default=0,
                    help="paged KV cache: pages of this many positions (the pool holds every sequence's max_seq)")
    ap.add_argument("--wide-chunk", type=int, default=512,
                    help="also time the prompt in chunks of this many tokens (0: off), and the gate_up "
                         "GEMM at that many rows")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the multi-position verify measurement (batch-1 workloads)")
    ap.add_argument("--verify-reps", type=int, default=20)
    ap.add_argument("--graph-steps", type=int, default=128,
                    help="steps of the graph-replayed decode_run measurement (0: skip; batch-1 workloads)")
    ap.add_argument("--cpu-prefill", type=int, default=16, help="oracle sample: prompt tokens")
    ap.add_argument("--cpu-decode", type=int, default=2, help="oracle sample: decode steps")
    ap.add_argument("--sample-every", type=int, default=8,
                    help="time the dominant kernel with HIP events in every N-th timed step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "BENCH_JSON"),
                    help="write a kernel statistics summary (with --out and --command) and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary of --kernel (with --out, --command, "
                         "--algo-bytes) and exit")
    ap.add_argument("--kernel", default=r"gemv_kernel<2,")
    ap.add_argument("--algo-bytes", type=float, default=0.0)
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--plain-json", help="with --summarize-stats: the bench line of an unprofiled run")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="write the MFMA summary of a --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 run (with --out, --command)")
    ap.add_argument("--out")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()

    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.out, "\n".join(args.command),
                        args.plain_json)
        return 0
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.out, args.command)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.kernel, args.copy_bytes,
                           args.algo_bytes, args.out, args.command)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "the library runs the whole step on a single MI355X (no sharding across GPUs)", file=sys.stderr)
        return 2

    import torch

    from decoder_only_transformer_step_amd import Decoder
    from synth.device import device_kv, device_weights
    from synth.weights import prompt
    from synth.workloads import WORKLOADS

    shape, work = WORKLOADS[args.workload]
    variant = {}
    if args.sliding_window:
        variant["sliding_window"] = args.sliding_window
    if args.attn_softcap:
        variant["attn_softcap"] = args.attn_softcap
    if args.attn_sinks:
        variant["attn_sinks"] = True
    if args.qk_norm:
        variant["qk_norm"] = True
    if args.weight_quant:
        variant["weight_quant"] = 1 if args.weight_quant == 8 else 2
    if args.kv_page:
        variant["kv_page_size"] = args.kv_page
        variant["kv_pages"] = work.batch * -(-shape.max_seq // args.kv_page)
    if variant:
        shape = shape.with_(name=shape.name + "-" + "-".join(f"{k}{v}" for k, v in variant.items()), **variant)
    # the first decode step (reported on its own), the warmup and the timed
    # steps together make the workload's decode steps
    if args.steps is None:
        args.steps = max(1, work.decode_steps - args.warmup - 1)
    room = shape.max_seq - (work.prompt or work.context)
    if 1 + args.warmup + args.steps > room:
        log(f"{shape.name}: 1 + {args.warmup} warmup + {args.steps} timed decode steps exceed the "
            f"{room} positions left after the prompt (max_seq {shape.max_seq})")
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    W = device_weights(shape)
    torch.cuda.synchronize()
    log(f"[gpu] {shape.name}: {shape.n_params() / 1e9:.2f}B params generated on device in {time.time() - t0:.1f}s")
    dec = Decoder(shape, W)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    result = {"metric": METRIC, "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded SplitMix64/Box-Muller bf16 weights and uniform token ids)"}
    if variant.get("weight_quant") == 1:
        result["dtype"] = "int8 weights (power-of-two row scales), fp32 accumulate"
    elif variant.get("weight_quant") == 2:
        result["dtype"] = "4-bit weights (power-of-two scale per 32), fp32 accumulate"
    batch = work.batch
    seqs = list(range(batch))

    # ------------------------------------------------------------ prefill --
    prefill = prefill_wide = gemm_cap = None
    context = work.context or (work.prompt if args.no_prefill else 0)
    if work.prompt and not args.no_prefill:
        ids = [int(t) for t in prompt(shape, work.prompt)]
        if args.wide_chunk and shape.max_chunk >= args.wide_chunk and work.prompt >= args.wide_chunk:
            prefill_wide = measure_prefill(dec, ids, args.wide_chunk, stream, ev0, ev1, args.prefill_runs)
            log(f"[gpu] prefill in chunks of {args.wide_chunk}: {prefill_wide['tok_s']:.0f} tok/s "
                f"(GEMM nodes {prefill_wide['gemm_mfma_frac']:.3f} of bf16 MFMA peak)")
        prefill = measure_prefill(dec, ids, work.chunk, stream, ev0, ev1, args.prefill_runs)
        log(f"[gpu] prefill {prefill['tok_s']:.0f} tok/s ({prefill['ms']:.1f} ms for {len(ids)} tokens)")
        if args.wide_chunk and shape.max_chunk >= args.wide_chunk and not shape.is_moe:
            gemm_cap = measure_gemm_capability(shape, args.wide_chunk, stream, ev0, ev1)
    elif context:
        # every sequence starts with a synthetic N(0,1) KV prefix (long-context batched decode)
        t0 = time.time()
        buf = None
        for s in seqs:
            for l in range(shape.n_layers):
                buf = device_kv(shape, s, l, context, out=buf)
                dec.kv_load(s, l, buf[0], buf[1], context)
        del buf
        torch.cuda.synchronize()
        log(f"[gpu] KV prefix {batch} x {context} filled in {time.time() - t0:.1f}s")

    # ------------------------------------------------------------- decode --
    first_tokens = None if prefill else [int(t) for t in prompt(shape, batch, seq=99)]
    am = torch.empty(batch, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    ev0.record(stream)
    dec.decode_step(seqs, first_tokens, argmax=am)
    ev1.record(stream)
    torch.cuda.synchronize()
    first_ms = ev0.elapsed_time(ev1)
    # warm-up steps, with every node timed once for the breakdown
    dec.stats_enable()
    for _ in range(args.warmup):
        dec.decode_step(seqs, None, argmax=am)
    wst = dec.stats_read()
    dec.stats_enable(())
    cand = {n: v for n, v in wst.items() if n in ("gate_up", "qkv", "o", "down", "head", "experts", "attn")}
    dom = max(cand, key=lambda n: cand[n]["ms"])
    # timed region: the dominant node's launches are bracketed by HIP events in
    # every SAMPLE-th step (bracketing every launch adds a few microseconds of
    # gap around each one, which would show up in the step time)
    dec.stats_enable([dom])
    dec.stats_mask([])
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        if i % args.sample_every == 0:
            dec.stats_mask([dom])
        dec.decode_step(seqs, None, argmax=am)
        if i % args.sample_every == 0:
            dec.stats_mask([])
    ev1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    dst = dec.stats_read()
    dec.stats_enable(())
    t_dec = ev0.elapsed_time(ev1) * 1e-3
    tok_s = args.steps * batch / t_dec
    step_bytes = sum(v["bytes"] for v in wst.values()) / max(1, args.warmup)
    log(f"[gpu] decode {tok_s:.1f} tok/s, {t_dec / args.steps * 1e3:.3f} ms/step "
        f"({step_bytes / 1e9:.2f} GB/step algorithmic)")

    # multi-position verify, after the timed decode region
    verify = None
    if batch == 1 and not args.no_verify:
        verify = measure_verify(dec, shape, stream, ev0, ev1, args.verify_reps)
    graph = None
    if batch == 1 and args.graph_steps > 0:
        graph = measure_graph(dec, shape, args.graph_steps)

    d = dst[dom]
    per_launch_bytes = d["bytes"] / d["launches"]
    per_launch_s = d["ms"] / d["launches"] * 1e-3
    achieved = per_launch_bytes / per_launch_s / 1e9
    qsuf = {1: "_q8", 2: "_q4"}.get(variant.get("weight_quant", 0), "")
    traffic = counter_traffic(f"counters_{dom}_decode_{args.workload}{qsuf}.md")
    kname = "attn_kernel" if dom == "attn" else "gemv_kernel, batch-1 projection"
    if dom == "gate_up" and not wst.get("down", {}).get("launches", 0):  # the dense FFN in one launch
        kname = "gemv_ffn_kernel, batch-1 gate/up and down projections"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"{dom} ({kname}, decode)", "bytes_per_launch": per_launch_bytes,
                "avg_us": round(per_launch_s * 1e6, 2), "launches": d["launches"],
                "timing": f"HIP events (no system fence) around every {dom} launch of every {args.sample_every}th "
                          "timed step; an event pair adds about 4.5 us of dispatch latency to the "
                          "bracketed kernel, so this is an upper bound on the kernel's own duration"}

    result.update({
        "value": round(tok_s, 2),
        "ms_per_step": round(t_dec / args.steps * 1e3, 4),
        "config": {"workload": shape.name, "global_batch": batch, "decode_positions":
                   [work.prompt or work.context, (work.prompt or work.context) + 1 + args.warmup + args.steps],
                   "kv_prefix": "prefill" if prefill else "synthetic N(0,1)",
                   "prefill_prompt": work.prompt, "prefill_chunk": work.chunk, "parallelism": "single-gpu",
                   **({"attention_variant": variant} if variant else {})},
        "decode": {"tok_s": tok_s, "first_step_ms": round(first_ms, 3), "hbm_GBps": step_bytes / (t_dec / args.steps) / 1e9,
                   "hbm_frac": step_bytes / (t_dec / args.steps) / 1e9 / HBM_PEAK_GBS,
                   "bytes_per_step": step_bytes, "host_s": t_host,
                   "nodes_warmup": summarize_nodes(wst)},
        "prefill": prefill,
        "prefill_wide_chunk": prefill_wide,
        "prefill_gemm_capability": gemm_cap,
        "verify": verify,
        "graph_decode": graph,
        "roofline": roofline,
        "kernel_source_sha256": kernel_source_hash(),
    })
    dec.close()
    del W
    torch.cuda.empty_cache()

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = n
        del a, b

    if not args.no_cpu_baseline:
        cpu_shape = shape.with_(max_batch=1)
        result["cpu_baseline"] = cpu_baseline(cpu_shape, args.cpu_prefill, args.cpu_decode)
        log(f"[cpu] oracle {result['cpu_baseline']['value']:.4f} tok/s on {result['cpu_baseline']['cores']} threads")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
