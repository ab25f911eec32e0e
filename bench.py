#!/usr/bin/env python3
"""Round microbenchmark: committed tokens/s of greedy self-speculative rounds.

Workload (the round microbenchmark): the 24-layer bf16 decoder (hidden 1024,
16 query heads over 4 KV heads of 64, SwiGLU 4096, vocab 60000) with a KV
cache prefilled from 1280 synthetic prefix embeddings, block size B = 32,
batch 1.  One step = one full round on the GPU: draft forward over
[x0, [M] x 32], verify forward over [a0, d1..d32], greedy argmax, accept,
commit and rollback (GravityOCR review, section 3.2 and Appendix B.2).
Every rep restarts from the same state (n = 1280, x0 = y1).  Drafts are
planted from the GPU's own AR continuation with the first mismatch at
min(Geometric(1/20), B), so accept lengths cover 0..32 with mean ~15.3.

Prints one JSON line.  Extra diagnostics go to stderr.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA peak of MI355X
COPY_CALIB_BYTES = 64 << 20


def expected_committed(B, p):
    """E[committed tokens per round] of the planted schedule: A* = min(G, B) with G geometric on
    {0, 1, ...} (P(G >= k) = (1 - p)^k), and every round commits A* + 2 tokens (no EOS, no budget
    cut in the microbenchmark): E[A*] = sum_{k=1..B} (1 - p)^k."""
    return 2.0 + sum((1.0 - p) ** k for k in range(1, B + 1))


def alg_bytes_round(cfg, n, B):
    """Algorithmic bytes of one round: weights streamed twice, KV read by both
    forwards, KV written for B+1 rows by each forward (bf16)."""
    layer_w = cfg.layer_params() * 2
    w = cfg.n_layers * layer_w + cfg.hidden * 4 + cfg.vocab * cfg.hidden * 2
    kvp = cfg.kv_bytes_per_position(2)
    return 2 * w + kvp * ((n + B + 1) + (n + B + 2)) + 2 * kvp * (B + 1)


def alg_bytes_kernel(kind, cfg, M, n_keys):
    """Algorithmic bytes one launch must move (weights + inputs + outputs)."""
    H, F, V, qd, kvd = cfg.hidden, cfg.ffn, cfg.vocab, cfg.q_dim, cfg.kv_dim
    e = 2
    if kind == "qkv":
        return (qd + 2 * kvd) * H * e + M * H * e + M * (qd + 2 * kvd) * e
    if kind == "o":
        return H * qd * e + M * qd * e + M * H * (4 + 4 + e)
    if kind == "gate_up":
        return 2 * F * H * e + M * H * e + M * F * e
    if kind == "down":      # one K range: weights + input + residual in and out, next input
        return H * F * e + M * F * e + M * H * (4 + 4 + e)
    if kind == "reduce":    # S partials + residual in, residual + next input + norm partials out
        return 4 * M * H * 4 + M * H * 4 + M * H * (4 + e) + M * (H // 16) * 4
    if kind == "lm_head":
        return V * H * e + M * H * e + M * 12
    if kind == "tail":      # the fused O + gate|up + down of one layer
        return sum(alg_bytes_kernel(k, cfg, M, n_keys) for k in ("o", "gate_up", "down"))
    if kind == "attention":
        return n_keys * 2 * kvd * e + M * qd * e
    if kind == "combine":
        return M * qd * e
    return M * 12


def batched_round_bound_us(cfg, ns, B):
    """Per-kernel bound of one batched round over requests with ns cached positions each:
    sum over launches of max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) (bf16 dense peak), for two
    forwards of M = R (B + 1) rows (GEMMs of every layer, one attention launch over all requests)
    and two LM heads.  GEMM flops count the M real rows only."""
    H, F, V, qd, kvd = cfg.hidden, cfg.ffn, cfg.vocab, cfg.q_dim, cfg.kv_dim
    R = len(ns)
    M = R * (B + 1)
    bw, pf = PEAK_HBM_GBS * 1e9, PEAK_BF16_TFLOPS * 1e12
    gemms = [("qkv", qd + 2 * kvd, H), ("o", H, qd), ("gate_up", 2 * F, H), ("down", H, F)]
    t = 0.0
    for fwd in range(2):
        keys = [n + B + 1 + fwd for n in ns]
        per_layer = 0.0
        for kind, N, K in gemms:
            per_layer += max(alg_bytes_kernel(kind, cfg, M, 0) / bw, 2.0 * M * N * K / pf)
        att_bytes = sum(k * 2 * kvd * 2 for k in keys) + M * qd * 2 * 2
        att_flops = sum(2 * 2 * (B + 1) * k * qd for k in keys)
        per_layer += max(att_bytes / bw, att_flops / pf)
        t += cfg.n_layers * per_layer
        t += max(alg_bytes_kernel("lm_head", cfg, M, 0) / bw, 2.0 * M * V * H / pf)
    return t * 1e6


def traffic_from_profiles(kind):
    """HBM bytes per launch of `kind` from a committed rocprofv3 counter summary
    (profiles/*_traffic.txt), or None when there is none or the kernel source has
    changed since the counters were taken."""
    sha = kernel_source_sha()
    pdir = os.path.join(ROOT, "profiles")
    for fn in sorted(os.listdir(pdir)) if os.path.isdir(pdir) else []:
        if not fn.endswith("_traffic.txt"):
            continue
        kv = {}
        with open(os.path.join(pdir, fn)) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_kind") == kind and kv.get("source_sha256") == sha:
            return int(kv["traffic_bytes_per_launch"])
    return None


KERNEL_LABELS = {   # (kernel template, EPI, KPW) of the GEMMs at the benchmark's shapes
    ("k_gemm", "0", "4"): "QKV GEMM + RoPE + KV write", ("k_gemm", "1", "4"): "O GEMM + residual",
    ("k_gemm", "2", "8"): "gate|up GEMM + SwiGLU", ("k_gemm", "1", "16"): "down GEMM + residual",
    ("k_gemm", "3", "16"): "LM head GEMM + top-2 records",
}


KERNEL_NAMES = {
    "k_layer_tail": "fused layer tail: O + gate|up + down", "k_attn": "attention (64-key chunks)",
    "k_attn_combine": "attention combine", "k_argmax": "vocabulary argmax merge",
    "k_prep_embed": "row prep + embedding gather", "k_accept": "accept + commit",
    "k_resid_reduce": "K-split residual reduce", "k_gemm_big": "large-tile GEMM",
}


def kernel_label(name, grid, prev=None):
    """A readable label for a dispatch.  The fused layer tail has one grid for any row count, so its
    launches are told apart by the grid of the attention combine that precedes them (one wave per
    row and head: 33 rows x 16 heads x 64 lanes = 33792 in a B=32 round, 1024 in an AR step)."""
    import re
    m = re.search(r"ssb::(k_\w+)(<[^>]*>)?", name)
    if not m:
        return re.sub(r"^void ", "", name)
    k = m.group(1)
    if k == "k_gemm":
        g = re.search(r"k_gemm<[^,]+, (\d+), (\d+), (\d+)", name)
        if g:
            return KERNEL_LABELS.get(("k_gemm", g.group(2), g.group(3)), name)
    label = KERNEL_NAMES.get(k, k)
    if k == "k_gemm_big":
        label += m.group(2) or ""
    if k == "k_layer_tail" and prev is not None and "k_attn_combine" in prev[0]:
        label += f" (after combine {prev[1]})"
    return label


def _dispatches(path, value_cols=False):
    """Rows of a rocprofv3 CSV (kernel trace or counter collection) as dispatches in launch order:
    (order key, kernel name, grid, duration in us or None, {counter: value})."""
    import csv
    rows = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            did = row.get("Dispatch_Id") or row.get("Correlation_Id")
            if "Grid_Size_X" in row:
                grid = "x".join(row.get(f"Grid_Size_{a}", "") for a in "XYZ")
            else:
                grid = row.get("Grid_Size", "")
            d = rows.get(did)
            if d is None:
                dur = None
                if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                    dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
                start = int(row.get("Start_Timestamp") or 0)
                d = rows[did] = [(start, int(did)), row.get("Kernel_Name", ""), grid, dur, {}]
            if value_cols and row.get("Counter_Name"):
                c = row["Counter_Name"]
                d[4][c] = d[4].get(c, 0.0) + float(row["Counter_Value"])
    return sorted(rows.values(), key=lambda d: d[0])


def _grouped(path, value_cols=False):
    import collections
    groups = collections.defaultdict(list)
    prev = None
    for d in _dispatches(path, value_cols):
        groups[(kernel_label(d[1], d[2], prev), d[2])].append(d)
        prev = (d[1], d[2])
    return groups


def summarize_trace(path):
    """Group a rocprofv3 kernel trace (CSV) by kernel and grid: the decode GEMMs of a round
    (33 rows) and of an AR step (1 row) share a kernel and differ in their grid."""
    groups = _grouped(path)
    dur = {key: [d[3] for d in v] for key, v in groups.items()}
    total = sum(sum(v) for v in dur.values())
    out = [f"{'kernel':62s} {'grid':>16s} {'calls':>7s} {'avg us':>8s} {'med us':>8s} {'min us':>8s} {'% time':>7s}"]
    for (label, grid), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{label[:62]:62s} {grid:>16s} {len(v):7d} {sum(v) / len(v):8.2f} "
                   f"{statistics.median(v):8.2f} {min(v):8.2f} {100 * sum(v) / total:7.2f}")
    return "\n".join(out)


def summarize_counters(fetch_csv, write_csv):
    """HBM bytes per dispatch from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the same counter reads for the calibration copy of
    COPY_CALIB_BYTES (the largest-grid device-to-device copy of the run: it reads and writes that
    many bytes).  Returns the text of the summary and {label: bytes per launch (median)}."""
    out, med = [], {}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        groups = _grouped(path, value_cols=True)
        copies = [(int(g.split("x")[0] or 0), v) for (lab, g), v in groups.items() if "copyBuffer" in lab]
        if not copies:
            raise SystemExit(f"{path}: no device-to-device copy to calibrate {counter} with")
        gmax = max(c[0] for c in copies)
        cal = statistics.median(d[4][counter] for c in copies if c[0] == gmax for d in c[1])
        scale = (COPY_CALIB_BYTES / 1024) / cal
        out.append(f"  calibration copy ({COPY_CALIB_BYTES >> 20} MiB read and written, grid {gmax}): "
                   f"{counter} {cal:.1f} KiB -> scale {scale:.5f}")
        for (label, grid), v in groups.items():
            vals = [d[4].get(counter, 0.0) for d in v]
            per.setdefault((label, grid), {})[counter] = (statistics.median(vals), scale, len(v))
    out.append("")
    out.append(f"  {'kernel':62s} {'grid':>16s} {'calls':>6s} {'FETCH KiB':>10s} {'WRITE KiB':>10s} {'-> MB':>9s}")
    rows = []
    for key, c in per.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        f_kib, f_s, n = c["FETCH_SIZE"]
        w_kib, w_s, _ = c["WRITE_SIZE"]
        b = (f_kib * f_s + w_kib * w_s) * 1024
        rows.append((b * n, key, n, f_kib, w_kib, b))
    for _, (label, grid), n, f_kib, w_kib, b in sorted(rows, reverse=True):
        if not label.startswith(("__amd", "at::")):
            out.append(f"  {label[:62]:62s} {grid:>16s} {n:6d} {f_kib:10.1f} {w_kib:10.1f} {b / 1e6:9.3f}")
        med[(label, grid)] = int(round(b))
    return "\n".join(out), med


KIND_LABELS = {"tail": "fused layer tail", "qkv": "QKV GEMM", "o": "O GEMM", "gate_up": "gate|up GEMM",
               "down": "down GEMM", "lm_head": "LM head GEMM", "attention": "attention (",
               "combine": "attention combine", "argmax": "vocabulary argmax"}


def kernel_source_sha():
    import hashlib
    with open(os.path.join(ROOT, "self_speculative_block_amd", "csrc", "ssb_kernels.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_summary(fetch_csv, write_csv, kind=None):
    """The text of a profiles/*_traffic.txt record (without its command lines): every kernel's
    scaled HBM bytes per launch and, for ``kind``, the record that later bench lines read (the
    group of that kind with the most launches: the round's own, not the AR continuation's)."""
    text, med = summarize_counters(fetch_csv, write_csv)
    if kind is None:
        return text
    from ssb_inputs import workload
    wl = workload(2)
    groups = _grouped(fetch_csv)
    cands = [key for key in med if key[0].startswith(KIND_LABELS[kind])]
    if not cands:
        raise SystemExit(f"no dispatch of kind {kind} in the counter runs")
    key = max(cands, key=lambda k: len(groups.get(k, ())))
    ab = alg_bytes_kernel(kind, wl.model, wl.block + 1, wl.prefix_len + wl.block + 1)
    return (text + f"\n\nkernel {key[0]}, grid {key[1]}: {med[key]} bytes per launch against {ab} "
            f"algorithmic ({med[key] / ab:.3f}x)\nkernel_kind: {kind}\nsource_sha256: {kernel_source_sha()}\n"
            f"traffic_bytes_per_launch: {med[key]}")


class no_gc:
    """Collect garbage before a timed loop and keep the collector off during it (as timeit does):
    a full collection over the heap of torch and numpy takes tens of milliseconds and would land
    on one arbitrary round."""

    def __enter__(self):
        import gc
        gc.collect()
        self.was = gc.isenabled()
        gc.disable()

    def __exit__(self, *exc):
        import gc
        if self.was:
            gc.enable()
        return False


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, weights, prefix, planted_rows, B, committed_per_round, reps=10, budget_s=12.0):
    """The oracle timed on the host on a bounded sample of the same rounds: numpy in float32 on
    every BLAS thread (the reported value), then float32 on one thread and float64 (the parity
    reference) as side notes.

    Each timed call is one full round (draft forward, verify forward, accept, rollback) from the
    same state with the same planted drafts as the GPU's rounds; the rate is the median over up
    to ``reps`` rounds (fewer if ``budget_s`` of CPU time runs out first).  The drafts are planted
    from the GPU's AR continuation; where the oracle's own greedy path departs from it at a
    near-tie the oracle accepts fewer of them, although it does the same work per round.  So the
    oracle's rate is stated in rounds/s and converted to tokens/s with the committed tokens per
    round of the GPU line (the planted schedule); the oracle's own committed count is reported
    beside it.
    """
    import numpy as np
    from oracle import Decoder, prefill, spec_round
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        cores = os.cpu_count()

    P = prefix.shape[0]

    def setup(dtype):
        model = Decoder(cfg, weights, dtype=dtype)
        st, y1, _ = prefill(model, np.asarray(prefix, dtype=dtype), P + B + 4)
        return model, st, y1

    def timed(setup_out, n_reps, budget):
        model, st, y1 = setup_out
        times, committed = [], 0
        for planted in planted_rows[:n_reps]:
            st.n, st.x0 = P, y1
            t0 = time.perf_counter()
            r = spec_round(model, st, B, planted=[int(x) for x in planted])
            times.append(time.perf_counter() - t0)
            committed += len(r.committed)
            if sum(times) >= budget:
                break
        return len(times), statistics.median(times), committed / len(times)

    f32 = setup(np.float32)
    n32, t32, c32 = timed(f32, reps, budget_s)
    out = {"value": committed_per_round / t32, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu": host_cpu_model(), "rounds_per_s": 1.0 / t32}
    note = ""
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, t1, _ = timed(f32, 3, budget_s / 3)
        out["rounds_per_s_1core"] = 1.0 / t1
        note += f"; float32 on 1 thread: median of {n1} rounds {t1:.2f} s"
    del f32
    n64, t64, _ = timed(setup(np.float64), 3, budget_s / 3)
    out["rounds_per_s_float64"] = 1.0 / t64
    note += f"; float64 on {cores} threads: median of {n64} rounds {t64:.2f} s"
    out["sample"] = (f"median of {n32} rounds of the round microbenchmark (numpy float32 oracle on {cores} "
                     f"threads, n=1280, B=32, same states and planted drafts), {t32:.2f} s per round, prefill "
                     f"excluded; tokens/s = rounds/s x {committed_per_round:.2f} committed tokens per round of "
                     f"the planted schedule (the oracle itself committed {c32:.2f} per round)" + note)
    return out


def plant_rows(cont, c, astar, B, vocab):
    """Draft for a round that starts after output token y_c (1-based), from the GPU's own AR
    output cont = [y1, y2, ...]: d_j = y_{c+1+j} for j <= A*, then a token different from
    y_{c+A*+2}; -1 (keep the draft's own token) elsewhere and past the end of cont."""
    row = [-1] * B
    for j in range(1, B + 1):
        idx = c + j
        if idx >= len(cont):
            break
        if j <= astar:
            row[j - 1] = int(cont[idx])
        elif j == astar + 1:
            row[j - 1] = int((cont[idx] + 1) % (vocab - 1))
            break
    return row


def round_vs_n(torch, model, kv, cfg, wid, B, ns, reps=20):
    """Device time of one round (draft + verify + accept, no planting) from a state with n cached
    positions, for each n: a synthetic prefix of n embeddings is prefilled, then the same round is
    repeated from that state; the roofline fraction is the round's algorithmic bytes at that n."""
    from ssb_inputs import prefix_embeddings
    out = {}
    for n in ns:
        kv.reset()
        y1 = kv.prefill(model.prefix_tensor(prefix_embeddings(wid, 10_000 + n, n, cfg.hidden)))
        evs = []
        with no_gc():
            for r in range(reps + 3):
                kv.rewind(n, y1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                kv.round(B)
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs[3:])
        ab = alg_bytes_round(cfg, n, B)
        out[str(n)] = {"round_us": us, "alg_bytes": ab, "roofline_frac": ab / (us * 1e-6) / (PEAK_HBM_GBS * 1e9)}
    return out


def decode_cpu_baseline(wl, weights, lengths, ar_outputs, gpu_tokens_per_round, budget_s=15.0):
    """The float32 oracle on a bounded sample of the workload's regions: region by region, prefill
    (not timed), then self-speculative rounds with the GPU line's planted drafts (built from the
    GPU's AR output and the same planted accept lengths), each round timed, until budget_s of
    round time.  Where the oracle's own greedy path departs from the GPU's at a near-tie, the
    planted drafts stop matching and its rounds commit fewer tokens for the same work, so the rate
    is measured in rounds/s and converted with the GPU line's committed tokens per round; the
    oracle's own count is reported beside it."""
    import numpy as np
    from oracle import Decoder, build_plant, prefill, spec_round
    from ssb_inputs import plant_accept_lengths, prefix_embeddings
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    model = Decoder(cfg, weights, dtype=np.float32)
    t_rounds, committed, rounds, regions = 0.0, 0, 0, 0
    for i, L in enumerate(lengths):
        if t_rounds >= budget_s:
            break
        print(f"oracle baseline: region {i}", file=sys.stderr, flush=True)
        pre = np.asarray(prefix_embeddings(wl.wid, i, P, cfg.hidden), dtype=np.float32)
        st, y1, _ = prefill(model, pre, P + L + B + 3)
        astar = plant_accept_lengths(wl.wid, i, L, B, wl.plant_p, wl.full_accept_p)
        out, k = [y1], 0
        while out[-1] != cfg.eos_id and len(out) < L and t_rounds < budget_s:
            plant = build_plant(ar_outputs[i], len(out), int(astar[k]) if k < len(astar) else B, B, cfg.vocab,
                                cfg.mask_id)
            t0 = time.perf_counter()
            r = spec_round(model, st, B, planted=plant, budget=L - len(out))
            t_rounds += time.perf_counter() - t0
            out += r.committed
            committed += len(r.committed)
            rounds += 1
            k += 1
        regions += 1
    rps = rounds / t_rounds
    return {"value": rps * gpu_tokens_per_round, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": host_cpu_model(), "rounds_per_s": rps,
            "sample": f"numpy float32 oracle on {cores} threads: {rounds} rounds over the first {regions} "
                      f"regions of the workload, {t_rounds:.1f} s of round time (prefill excluded), drafts "
                      f"planted from the GPU's AR output with the same accept lengths; tokens/s = rounds/s x "
                      f"{gpu_tokens_per_round:.2f} committed tokens per round of the GPU line (the oracle "
                      f"itself committed {committed / max(rounds, 1):.2f} per round)"}


def decode_workload(args, wid):
    """Configs 3 and 4: per region, GPU AR decode (its output plants the drafts), then GPU
    self-speculative decode of the same region; decode-only committed tokens/s of both."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, plant_accept_lengths, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool

    wl = workload(wid)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    lengths = target_lengths(wl)
    n = min(args.regions or wl.n_regions, wl.n_regions)
    # room for the longest region; for tables, for the length cap (round_vs_n reaches prefix + 4096)
    cap = max(max(lengths[:n]), 4096 if wid == 4 else 0)
    torch.cuda.set_device(0)
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=2048, max_positions=P + cap + 2 * B + 8,
                  max_batch=1, sampling=False)
    pool = Pool(model, n_pages=(P + cap + 2 * B + 8) // 16 + 8)
    kv = KV(pool, P + cap + 2 * B + 8)
    tot = {"spec_tokens": 0, "spec_us": 0.0, "ar_tokens": 0, "ar_us": 0.0, "rounds": 0, "forwards": 0,
           "accepted": 0}
    hist = np.zeros(B + 1, dtype=np.int64)
    ar_outputs = []
    for i in range(n):
        if i % 16 == 0:
            print(f"{wl.name}: region {i} of {n}", file=sys.stderr, flush=True)
        pre_dev = model.prefix_tensor(prefix_embeddings(wl.wid, i, P, cfg.hidden))
        L = lengths[i]
        kv.reset()
        ar, st_ar = kv.decode_ar(pre_dev, L)
        ar_outputs.append(ar)
        astar = plant_accept_lengths(wl.wid, i, L, B, wl.plant_p, wl.full_accept_p)
        kv.reset()
        spec, st = kv.decode(pre_dev, B, L, cont_dev=torch.tensor(ar, dtype=torch.int32, device="cuda"),
                             astar=astar)
        assert spec == ar, f"region {i}: self-speculative output differs from AR"
        tot["spec_tokens"] += st.tokens - 1
        tot["spec_us"] += st.decode_us
        tot["ar_tokens"] += st_ar.tokens - 1
        tot["ar_us"] += st_ar.decode_us
        tot["rounds"] += st.rounds
        tot["forwards"] += st.forwards
        tot["accepted"] += st.accepted
        for a in astar[: st.rounds]:
            hist[min(int(a), B)] += 1
    spec_tps = tot["spec_tokens"] / (tot["spec_us"] * 1e-6)
    ar_tps = tot["ar_tokens"] / (tot["ar_us"] * 1e-6)
    # round time against the HBM roofline across the cached lengths the workload reaches
    top = P + min(cap, 4096)
    ns = sorted({P, (P + top) // 2, top} if wid == 3 else {P, 2048, 3072, 4096, top})
    print(f"{wl.name}: round time against cached length", file=sys.stderr, flush=True)
    per_n = round_vs_n(torch, model, kv, cfg, wl.wid, B, [x for x in ns if x + B + 2 <= P + cap + 2 * B + 8])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = decode_cpu_baseline(wl, generate_weights(cfg), lengths[:n], ar_outputs,
                                  tot["spec_tokens"] / max(tot["rounds"], 1))
    line = {
        "metric": "decode-only committed tokens/s, self-speculative (B=32, batch 1), prefill excluded",
        "value": spec_tps, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "regions": n, "prefix": P, "block_B": B,
                   "mean_target_len": float(np.mean(lengths[:n]))},
        "ar_tokens_per_s": ar_tps, "speedup_vs_ar": spec_tps / ar_tps,
        "tpf": tot["spec_tokens"] / max(tot["forwards"], 1),
        "mean_accept": tot["accepted"] / max(tot["rounds"], 1), "rounds": tot["rounds"],
        "planted_accept_histogram": hist.tolist(),
        "outputs_identical_to_ar": True,
        "round_vs_n": per_n,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def batched_workload(args):
    """Config 5: 16 concurrent requests (12 text, 3 table, 1 formula), one launch per stage per
    round for all unfinished requests; aggregate committed tokens/s and page decode time."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, plant_accept_lengths, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool, round_batch

    wl = workload(5)
    cfg, P = wl.model, wl.prefix_len
    lengths = target_lengths(wl)
    R = len(lengths)
    torch.cuda.set_device(0)
    Bmax = max((wl.block,) + tuple(wl.blocks_extra))
    cap = max(lengths) + 2 * Bmax + 8
    model = Model(cfg, generate_weights(cfg), block_B=Bmax, max_rows=2048, max_positions=P + cap,
                  max_batch=16, sampling=False)
    pool = Pool(model, n_pages=R * ((P + cap) // 16 + 2))
    kvs = [KV(pool, P + cap) for _ in range(R)]
    pres = [model.prefix_tensor(prefix_embeddings(wl.wid, r, P, cfg.hidden)) for r in range(R)]
    # AR reference per request (plants the drafts), and the AR page time when requests run one by one
    ars, ar_us = [], 0.0
    for r in range(R):
        kvs[r].reset()
        out, st = kvs[r].decode_ar(pres[r], lengths[r])
        ars.append(out)
        ar_us += st.decode_us
    results = {}
    for B in (wl.block,) + tuple(wl.blocks_extra):
        astars = [plant_accept_lengths(wl.wid, r, lengths[r], B, wl.plant_p) for r in range(R)]
        outs = []
        for r in range(R):
            kvs[r].reset()
            outs.append([kvs[r].prefill(pres[r])])
        rounds = [0] * R
        n_launch = 0
        torch.cuda.synchronize()
        with no_gc():
            t0 = time.perf_counter()
            while True:
                act = [r for r in range(R) if len(outs[r]) < lengths[r] and outs[r][-1] != cfg.eos_id]
                if not act:
                    break
                rows = [plant_rows(ars[r], len(outs[r]), int(astars[r][rounds[r]]), B, cfg.vocab) for r in act]
                planted = torch.tensor(rows, dtype=torch.int32, device="cuda")
                res = round_batch(model, [kvs[r] for r in act], B, [lengths[r] - len(outs[r]) for r in act],
                                  planted_dev=planted)
                for r, (c, _A) in zip(act, res):
                    outs[r] += c
                    rounds[r] += 1
                n_launch += 1
            t = time.perf_counter() - t0
        for r in range(R):
            assert outs[r] == ars[r], f"request {r}: batched self-speculative output differs from AR"
        toks = sum(len(o) - 1 for o in outs)
        results[B] = {"tokens_per_s": toks / t, "page_decode_ms": t * 1e3, "batched_rounds": n_launch,
                      "tokens": toks}
    ar_tps = sum(len(o) - 1 for o in ars) / (ar_us * 1e-6)
    # fixed occupancy: every request at its prefill state, the same batched round repeated;
    # device time per round against the per-kernel bound
    occupancy = {}
    for B in (wl.block,) + tuple(wl.blocks_extra):
        y1s = []
        for r in range(R):
            kvs[r].reset()
            y1s.append(kvs[r].prefill(pres[r]))
        evs = []
        with no_gc():
            for rep in range(25):
                for r in range(R):
                    kvs[r].rewind(P, y1s[r])
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                round_batch(model, kvs, B, [B + 2] * R)
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs[5:])
        bound = batched_round_bound_us(cfg, [P] * R, B)
        occupancy[str(B)] = {"rows": R * (B + 1), "round_us_median": us, "bound_us": bound,
                             "frac_of_bound": bound / us}
    line = {
        "metric": "aggregate decode-only committed tokens/s, batched self-speculative page (16 requests)",
        "value": results[wl.block]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "requests": R, "prefix": P, "lengths": lengths},
        "by_block": {str(k): v for k, v in results.items()},
        "ar_one_by_one_tokens_per_s": ar_tps,
        "outputs_identical_to_ar": True,
        "full_occupancy_round": occupancy,
    }
    print(json.dumps(line))


def direct_workload(args):
    """Direct block-diffusion decoding of the text regions (config 3 shapes: prefix 1088,
    lengths of mean 73), B = 32, batch 1.  The random-init decoder's confidences all sit near
    1/vocab, so each threshold is a quantile of the first denoising step's confidences on the
    first region; the sweep over quantiles plays the pages' threshold sweep.  Reports decode-only
    tokens/s, tokens per forward in the pages' accounting (committing forwards only) and with the
    cache-write forwards, and the device time of one denoising step and one cache-write."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool

    wl = workload(3)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    lengths = target_lengths(wl)
    n = min(args.regions or wl.n_regions, wl.n_regions)
    cap = max(lengths[:n])
    torch.cuda.set_device(0)
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=2048, max_positions=P + cap + 2 * B + 8,
                  max_batch=1, sampling=False)
    pool = Pool(model, n_pages=(P + cap + 2 * B + 8) // 16 + 8)
    kv = KV(pool, P + cap + 2 * B + 8)
    pres = [model.prefix_tensor(prefix_embeddings(wl.wid, i, P, cfg.hidden)) for i in range(n)]
    kv.reset()
    kv.prefill(pres[0])
    _, _, _, ex = kv.dd_block(B, 0.0, write_cache=False, want_steps=True)
    conf0 = np.sort(ex["conf"][0])
    # device time of one denoising step and of one cache-write forward (graph replays)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kv.reset()
    y1 = kv.prefill(pres[0])
    step_ms = []
    for rep in range(20):
        kv.rewind(P, y1)
        torch.cuda.synchronize()
        ev[0].record()
        kv.dd_block(B, 0.0, write_cache=False)       # one step, no cache-write
        ev[1].record()
        torch.cuda.synchronize()
        step_ms.append(ev[0].elapsed_time(ev[1]))
    blk_ms = []
    for rep in range(20):
        kv.rewind(P, y1)
        torch.cuda.synchronize()
        ev[0].record()
        kv.dd_block(B, 0.0, write_cache=True)        # one step + the cache-write forward
        ev[1].record()
        torch.cuda.synchronize()
        blk_ms.append(ev[0].elapsed_time(ev[1]))
    step_med, blk_med = float(np.median(step_ms[5:])), float(np.median(blk_ms[5:]))
    sweep = {}
    for q in (0.25, 0.5, 0.75, 0.9):
        tau = float(conf0[min(int(q * len(conf0)), len(conf0) - 1)])
        toks = steps = cws = blocks = 0
        us = 0.0
        for i in range(n):
            kv.reset()
            out, st = kv.decode_dd(pres[i], B, tau, lengths[i])
            toks += st.tokens - 1
            steps += st.forwards
            cws += st.cache_forwards
            blocks += st.rounds
            us += st.decode_us
        sweep[str(q)] = {"tau": tau, "tokens_per_s": toks / (us * 1e-6), "tpf": toks / max(steps, 1),
                         "tokens_per_forward_with_cache_writes": toks / max(steps + cws, 1),
                         "steps_per_block": steps / max(blocks, 1), "blocks": blocks, "tokens": toks}
    line = {
        "metric": "decode-only tokens/s, direct block-diffusion decoding (B=32, batch 1), prefill excluded",
        "value": sweep["0.5"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_direct_diffusion", "regions": n, "prefix": P, "block_B": B,
                   "tau_rule": "quantile of the first step's confidences", "quantile": 0.5},
        "sweep": sweep,
        "denoising_step_device_ms": step_med,
        "cache_write_device_ms": blk_med - step_med,
    }
    print(json.dumps(line))


def sample_workload(args):
    """Stochastic self-speculative decoding of the text regions (config 3 shapes), B = 32,
    batch 1, against AR sampling through the same kernels, at temperatures 1.0 and 0.7.
    Uniforms are seeded per region.  The random-init decoder's draft and target
    distributions are both close to uniform, so acceptance here says nothing about a trained
    model; the line measures the cost of a stochastic round (logits written, sampled rows,
    the acceptance test and residual draw) against a greedy one."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool

    wl = workload(3)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    lengths = target_lengths(wl)
    n = min(args.regions or 64, wl.n_regions)
    cap = max(lengths[:n])
    torch.cuda.set_device(0)
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=2048, max_positions=P + cap + 2 * B + 8,
                  max_batch=1)
    pool = Pool(model, n_pages=(P + cap + 2 * B + 8) // 16 + 8)
    kv = KV(pool, P + cap + 2 * B + 8)
    pres = [model.prefix_tensor(prefix_embeddings(wl.wid, i, P, cfg.hidden)) for i in range(n)]
    res = {}
    for T in (1.0, 0.7):
        tot = {"spec_tokens": 0, "spec_us": 0.0, "ar_tokens": 0, "ar_us": 0.0, "rounds": 0, "accepted": 0}
        for i in range(n):
            L = lengths[i]
            U = torch.tensor(np.random.default_rng([7, i, int(T * 10)]).random((L + 1, 2 * B + 2)),
                             dtype=torch.float32, device="cuda")
            kv.reset()
            out, st = kv.decode_sample(pres[i], B, L, U, temperature=T)
            tot["spec_tokens"] += st.tokens - 1
            tot["spec_us"] += st.decode_us
            tot["rounds"] += st.rounds
            tot["accepted"] += st.accepted
            kv.reset()
            ar, sta = kv.decode_ar_sample(pres[i], L, U[:, 0].contiguous(), temperature=T)
            tot["ar_tokens"] += sta.tokens - 1
            tot["ar_us"] += sta.decode_us
        spec_tps = tot["spec_tokens"] / (tot["spec_us"] * 1e-6)
        ar_tps = tot["ar_tokens"] / (tot["ar_us"] * 1e-6)
        res[str(T)] = {"tokens_per_s": spec_tps, "ar_sampling_tokens_per_s": ar_tps, "speedup_vs_ar": spec_tps / ar_tps,
                       "tpf": tot["spec_tokens"] / max(2 * tot["rounds"], 1),
                       "mean_accept": tot["accepted"] / max(tot["rounds"], 1), "rounds": tot["rounds"],
                       "round_ms_mean": tot["spec_us"] / max(tot["rounds"], 1) / 1e3}
    line = {
        "metric": "decode-only tokens/s, stochastic self-speculative decoding (B=32, batch 1), prefill excluded",
        "value": res["1.0"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_sampling", "regions": n, "prefix": P, "block_B": B, "temperature": 1.0},
        "by_temperature": res,
    }
    print(json.dumps(line))


def multistep_workload(args):
    """Greedy self-speculative decoding of the text regions (config 3 shapes) with draft
    schedules of 1, 2 and 4 steps, B = 32, batch 1.  The draft-side threshold is the median of
    the first draft step's confidences on the first region.  Outputs are checked equal to AR.
    The random-init decoder's drafts rarely match the verifier, so acceptance stays near zero
    here; the line measures what each extra draft forward costs per round."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool

    wl = workload(3)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    lengths = target_lengths(wl)
    n = min(args.regions or 32, wl.n_regions)
    cap = max(lengths[:n])
    torch.cuda.set_device(0)
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=2048, max_positions=P + cap + 2 * B + 8,
                  max_batch=1, sampling=False)
    pool = Pool(model, n_pages=(P + cap + 2 * B + 8) // 16 + 8)
    kv = KV(pool, P + cap + 2 * B + 8)
    pres = [model.prefix_tensor(prefix_embeddings(wl.wid, i, P, cfg.hidden)) for i in range(n)]
    kv.reset()
    kv.prefill(pres[0])
    _, _, _, ex = kv.dd_block(B, 0.0, write_cache=False, want_steps=True)
    tau = float(np.median(ex["conf"][0]))
    ars = []
    for i in range(n):
        kv.reset()
        ars.append(kv.decode_ar(pres[i], lengths[i])[0])
    res = {}
    for steps in (1, 2, 4):
        toks = fw = rounds = acc = 0
        us = 0.0
        for i in range(n):
            kv.reset()
            out, st = kv.decode_multistep(pres[i], B, steps, tau, lengths[i])
            assert out == ars[i], f"region {i}: output differs from AR"
            toks += st.tokens - 1
            fw += st.forwards
            rounds += st.rounds
            acc += st.accepted
            us += st.decode_us
        res[str(steps)] = {"tokens_per_s": toks / (us * 1e-6), "tpf": toks / max(fw, 1),
                           "mean_accept": acc / max(rounds, 1), "draft_forwards_per_round": (fw - rounds) / rounds,
                           "round_ms_mean": us / rounds / 1e3, "rounds": rounds}
    line = {
        "metric": "decode-only tokens/s, self-speculative decoding with a multi-step draft schedule (B=32, batch 1)",
        "value": res["1"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_draft_schedule", "regions": n, "prefix": P, "block_B": B,
                   "draft_tau": tau},
        "by_steps": res, "outputs_identical_to_ar": True,
    }
    print(json.dumps(line))


def sweep_workload(args):
    """Throughput against the cap on running requests (GravityOCR review, section 4.3, Figure 6;
    Appendix C: a full client queue and a running-request cap).  A queue of text regions (config 3
    shapes: prefix 1088, lengths of mean ~68) is served by continuous batching at caps 1..64, with
    greedy AR steps and with self-speculative rounds (B = 32, drafts planted from the AR output with
    the config's accept-length schedule).  Reports tokens/s over the whole queue (prefills
    included, as a server's clock runs) and decode-only, per cap, and their ratio."""
    import numpy as np
    import torch
    from ssb_inputs import generate_weights, plant_accept_lengths, prefix_embeddings, workload
    from ssb_inputs.schedule import target_lengths
    from self_speculative_block_amd.engine import KV, Model, Pool, serve
    from self_speculative_block_amd._lib import SSB_SERVE_AR, SSB_SERVE_SPEC

    wl = workload(3)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    lengths = target_lengths(wl)
    n = min(args.regions or 128, wl.n_regions)
    caps = (1, 2, 4, 8, 16, 32, 64)
    cap_len = max(lengths[:n])
    max_tokens = P + cap_len + 2 * B + 8
    torch.cuda.set_device(0)
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=max(caps) * (B + 1), max_positions=max_tokens,
                  sampling=False)
    pool = Pool(model, n_pages=(max(caps) + 1) * (max_tokens // 16 + 2))
    reqs = [{"prefix_dev": model.prefix_tensor(prefix_embeddings(wl.wid, i, P, cfg.hidden)), "max_len": lengths[i]}
            for i in range(n)]
    # AR reference outputs (they plant the drafts), one request at a time
    kv = KV(pool, max_tokens)
    ref = []
    for q in reqs:
        kv.reset()
        ref.append(kv.decode_ar(q["prefix_dev"], q["max_len"])[0])
    kv.close()
    planted = [dict(q, cont_dev=torch.tensor(ref[i], dtype=torch.int32, device="cuda"),
                    astar=[int(a) for a in plant_accept_lengths(wl.wid, i, q["max_len"], B, wl.plant_p)])
               for i, q in enumerate(reqs)]
    toks = sum(len(o) - 1 for o in ref)
    res = {}
    for cap in caps:
        row = {}
        for name, mode, qs in (("ar", SSB_SERVE_AR, reqs), ("spec", SSB_SERVE_SPEC, planted)):
            out, info, st = serve(model, pool, qs, cap, mode, B=B if mode == SSB_SERVE_SPEC else 0,
                                  max_tokens=max_tokens)
            assert out == ref, f"cap {cap} {name}: output differs from AR"
            row[name] = {"tokens_per_s": toks / (st["total_us"] * 1e-6),
                         "decode_tokens_per_s": toks / (st["decode_us"] * 1e-6),
                         "launches": st["steps"], "mean_running": st["mean_running"],
                         "total_ms": st["total_us"] / 1e3, "prefill_ms": st["prefill_us"] / 1e3}
        row["speedup"] = row["spec"]["tokens_per_s"] / row["ar"]["tokens_per_s"]
        row["decode_speedup"] = row["spec"]["decode_tokens_per_s"] / row["ar"]["decode_tokens_per_s"]
        res[str(cap)] = row
        print(f"cap {cap}: ar {row['ar']['tokens_per_s']:.0f} spec {row['spec']['tokens_per_s']:.0f} tok/s "
              f"(x{row['speedup']:.2f}; decode-only x{row['decode_speedup']:.2f})", file=sys.stderr, flush=True)
    line = {
        "metric": "tokens/s over a queue of text regions under continuous batching, self-speculative vs AR",
        "value": res["64"]["spec"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_batch_sweep", "requests": n, "prefix": P, "block_B": B,
                   "caps": list(caps), "output_tokens": toks},
        "by_cap": res, "outputs_identical_to_ar": True,
    }
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--workload", choices=["round", "text", "table", "batched", "direct", "sample", "multistep", "sweep"], default="round",
                    help="round: the round microbenchmark (the headline line); text / table: decode "
                         "of text or table regions; batched: the 16-request page; direct: direct "
                         "block-diffusion decoding of the text regions; sample: stochastic decoding "
                         "of the text regions; multistep: draft schedules of 1, 2, 4 steps; sweep: "
                         "continuous batching at running caps 1..64, AR vs self-speculative")
    ap.add_argument("--regions", type=int, default=0, help="text / table: number of regions (0 = all)")
    ap.add_argument("--summarize-trace", default=None,
                    help="print a rocprofv3 kernel trace (CSV) grouped by kernel and grid, then exit")
    ap.add_argument("--summarize-counters", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM traffic per dispatch from a FETCH_SIZE run and a WRITE_SIZE run of "
                         "rocprofv3 --pmc (counter_collection CSVs), then exit; with --traffic-kind, "
                         "also the lines that give that kernel kind's traffic to later bench lines")
    ap.add_argument("--traffic-kind", default=None, help="kernel kind of --summarize-counters' record")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(traffic_summary(*args.summarize_counters, args.traffic_kind))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the round engine is a single-GPU path "
              "(requests would shard across GPUs with no exchange step); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "text":
        return decode_workload(args, 3)
    if args.workload == "table":
        return decode_workload(args, 4)
    if args.workload == "batched":
        return batched_workload(args)
    if args.workload == "direct":
        return direct_workload(args)
    if args.workload == "sample":
        return sample_workload(args)
    if args.workload == "multistep":
        return multistep_workload(args)
    if args.workload == "sweep":
        return sweep_workload(args)

    import numpy as np
    import torch

    from ssb_inputs import generate_weights, plant_accept_lengths, prefix_embeddings, workload
    from self_speculative_block_amd.engine import KV, Model, Pool

    wl = workload(2)
    cfg = wl.model
    B = wl.block
    P = wl.prefix_len
    torch.cuda.set_device(0)
    weights = generate_weights(cfg)
    # one request, greedy rounds only: the workspace holds one window's rows
    model = Model(cfg, weights, block_B=B, max_rows=2048, max_positions=P + 256, max_batch=1, sampling=False)
    pool = Pool(model, n_pages=(P + 256) // 16 + 8)
    kv = KV(pool, P + 200)
    prefix = prefix_embeddings(wl.wid, 0, P, cfg.hidden)
    pre_dev = model.prefix_tensor(prefix)
    y1 = kv.prefill(pre_dev)
    # GPU AR continuation y1..y_{B+3}: the drafts are planted from it
    cont = [y1]
    for _ in range(B + 3):
        cont.append(kv.ar_step()[0])
    kv.rewind(P, y1)
    n_reps = args.warmup + max(args.steps, args.profile_steps)
    astar = plant_accept_lengths(wl.wid, 0, n_reps, B, wl.plant_p)
    planted = np.full((n_reps, B), -1, dtype=np.int32)
    for r, a in enumerate(astar):
        # output so far is [y1] (c = 1); a0 = y2, so d_j = y_{2+j} = cont[j + 1] for j <= A*,
        # and d_{A*+1} differs from y_{A*+3}
        for j in range(1, B + 1):
            if j <= a:
                planted[r, j - 1] = cont[j + 1]
            elif j == a + 1:
                planted[r, j - 1] = (cont[j + 1] + 1) % (cfg.vocab - 1)
                break
    planted_dev = torch.from_numpy(planted).to("cuda")

    def run(rep):
        kv.rewind(P, y1)
        c, A, _, _ = kv.round(B, planted_dev=planted_dev[rep])
        return len(c), A

    for r in range(args.warmup):
        run(r)
    torch.cuda.synchronize()
    committed = 0
    accepts = []
    per_round = []
    events = []
    st = torch.cuda.current_stream()
    with no_gc():
        t0 = time.perf_counter()
        for k in range(args.steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            ts = time.perf_counter()
            e0.record(st)
            n, A = run(args.warmup + k)
            e1.record(st)
            per_round.append(time.perf_counter() - ts)
            events.append((e0, e1))
            committed += n
            accepts.append(A)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    dev_us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in events)

    # the same rounds with each layer's O, gate|up and down as three launches instead of the fused
    # layer tail (bit-identical results; device time only, for comparison)
    def device_median(n):
        evs = []
        with no_gc():
            for k in range(n):
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(st)
                run(args.warmup + k)
                a1.record(st)
                evs.append((a0, a1))
            torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)
    model.set_debug(False, unfused=True)
    run(args.warmup)
    unfused_us = device_median(min(args.steps, 50))
    model.set_debug(False, unfused=False)
    run(args.warmup)

    # rounds without planting (the draft's own proposals), same state
    unplanted = []
    for k in range(min(args.steps, 50)):
        kv.rewind(P, y1)
        ts = time.perf_counter()
        kv.round(B)
        unplanted.append(time.perf_counter() - ts)
    for k in range(args.steps):
        assert accepts[k] == min(int(astar[args.warmup + k]), B), "planted accept length not realized"
    assert cfg.eos_id not in cont[1:B + 3], "the planted continuation holds EOS (rounds would be cut)"
    ms_step = elapsed * 1e3 / args.steps
    t_med = statistics.median(per_round)
    # headline: the schedule's expected committed tokens per round over the median round time (the
    # realised mean of the timed sample is reported beside it; it moves with --steps)
    e_committed = expected_committed(B, wl.plant_p)
    value = e_committed / t_med
    bytes_round = alg_bytes_round(cfg, P, B)

    # per-kernel timing of graph-replayed launches (as in the timed region): for each kernel kind
    # the engine replays a round graph in which every launch stamps its latest workgroup end on the
    # device's real-time counter; a launch of the kind counts from the end of the launch before it
    kinds = ["qkv", "attention", "combine", "o", "gate_up", "down", "reduce", "tail", "lm_head", "argmax"]
    breakdown = {}
    for kind in kinds:
        model.profile_kernel(kind, in_graph=True)
        run(args.warmup)                    # capture the timing graph outside the sample
        model.profile_read(reset=True)
        for k in range(args.profile_steps):
            run(args.warmup + k)
        us, launches = model.profile_read(reset=True)
        if launches == 0:       # a kind this model's shapes never launch (the K-split reduce)
            continue
        breakdown[kind] = {"avg_us": us / launches, "us_per_round": us / args.profile_steps,
                           "launches_per_round": launches / args.profile_steps}
    model.profile_kernel(None)
    dom = max(breakdown, key=lambda k: breakdown[k]["us_per_round"])
    M = B + 1
    n_keys = P + B + 1
    ab = alg_bytes_kernel(dom, cfg, M, n_keys)
    achieved = ab / (breakdown[dom]["avg_us"] * 1e-6) / 1e9
    print(json.dumps({"kernel_breakdown_us": breakdown, "dominant": dom}), file=sys.stderr)

    # calibration copy for the HBM byte counters: one device-to-device copy of a known size
    # (outside the timed region); its FETCH_SIZE / WRITE_SIZE scale the counters of the GEMM
    calib_src = torch.ones(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    # attainable-bandwidth probe: the same copy, timed (read + write bytes / time)
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    for _ in range(10):
        calib_dst.copy_(calib_src)
    ce1.record()
    ce1.synchronize()
    copy_gbs = 10 * 2 * COPY_CALIB_BYTES / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del calib_src, calib_dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, weights, prefix, planted[args.warmup:], B, e_committed)

    line = {
        "metric": "committed tokens/s (B=32, batch 1) + round time as % of HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": cfg.n_layers, "hidden": cfg.hidden, "heads": cfg.n_heads,
                   "kv_heads": cfg.n_kv_heads, "ffn": cfg.ffn, "vocab": cfg.vocab, "block_B": B,
                   "cached_positions": P, "batch": 1},
        "committed_per_round_expected": e_committed,
        "committed_per_round_realised": committed / args.steps,
        "mean_accept_realised": float(np.mean(accepts)),
        "tokens_per_s_realised": committed / elapsed,
        "round_us_median": t_med * 1e6,
        "round_us_wall": {"p90": sorted(per_round)[len(per_round) * 9 // 10] * 1e6, "max": max(per_round) * 1e6,
                          "mean": elapsed / args.steps * 1e6},
        "round_device_us": {"median": statistics.median(dev_us), "p10": dev_us[len(dev_us) // 10],
                            "p90": dev_us[(len(dev_us) * 9) // 10]},
        "round_us_unplanted_median": statistics.median(unplanted) * 1e6,
        "round_device_us_unfused_tail_median": unfused_us,
        "copy_probe_GBs": copy_gbs,
        "round_roofline_frac": bytes_round / t_med / (PEAK_HBM_GBS * 1e9),
        "round_alg_bytes": bytes_round,
        "device_memory_MB": {k: v / 2 ** 20 for k, v in zip(("packed_weights", "workspace"), model.memory())},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profiles(dom), "alg_bytes_per_launch": ab,
                     "avg_launch_us": breakdown[dom]["avg_us"],
                     "timing": "graph-replayed launches, device real-time stamps: from the end of the launch "
                               "before to the last workgroup end (the dispatch interval of a kernel trace)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
