#!/usr/bin/env python3
"""Benchmark of libattn on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
a varlen prefill call on the 16742-token, 32-head, head_dim-128 sequence and a
paged-decode call on 256 sequences of 64 tokens (16 query / 16 KV heads,
head_size 128, block_size 16), sizes from the Shapes tables of the atrex-bench
pages "attention_forward" (#001, row 9) and "paged_attention_decode" (#024,
row 0).  Inputs are seeded standard-normal bf16, resident in HBM before the
timed region.  Each call is bracketed by HIP events on the stream it is
launched on; the decode inputs rotate over several copies (more bytes than
the 256 MB Infinity Cache) so every decode call reads HBM, not the cache.
The decode roofline figure comes from the same decode calls issued back to
back after the step loop (a lone 26-us call's event pair would also time its
dispatch).

Printed: one JSON line with prefill TFLOP/s (the headline value), decode
GB/s, both against MI355X roofline peaks and with the shader clock sampled
during the timed prefill launches; under "configs" the other prefill
workloads of the configuration list, each timed on its own; the CPU oracle's
rate on a bounded sample and its time on every workload (in full where that
takes seconds, else a sample with the full time extrapolated, labelled); and
under "page_context" the pages' own T_SOL and T_Prod for the same workloads
(hardware labelled only "XPU-A"; context, not a target) beside this run's
per-launch times.  Only one GPU is used: --gpus above 1 exits
with a message.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PREFILL = "prefill_s16742_h32_d128"
DECODE = "decode_b256_ctx64_h16_kv16_d128"
CHUNK = "chunk_t14807_h32_hq16"
# the sources each kernel's counter figures depend on
KERNEL_SOURCES = {
    "prefill_fwd_d128_kernel": ["prefill_d128_kernel.hpp", "prefill_kernel.hpp", "device_common.hpp"],
    "prefill_fwd_d72_kernel": ["prefill_d72_kernel.hpp", "prefill_kernel.hpp", "device_common.hpp"],
    "prefill_fwd_kernel": ["prefill_kernel.hpp", "device_common.hpp"],
    "prefill_fwd_split_kernel": ["prefill_split_kernel.hpp", "prefill_kernel.hpp", "device_common.hpp"],
    "decode_partition_kernel": ["decode_kernel.hpp", "device_common.hpp"],
    "decode_mfma_kernel": ["decode_mfma_kernel.hpp", "decode_kernel.hpp", "device_common.hpp"],
    "chunk_delta_out_kernel": ["chunk_kernel.hpp", "device_common.hpp"],
}
ALL_SOURCES = ["prefill_d128_kernel.hpp", "prefill_d72_kernel.hpp", "prefill_kernel.hpp",
               "prefill_split_kernel.hpp", "decode_kernel.hpp", "decode_mfma_kernel.hpp", "chunk_kernel.hpp",
               "device_common.hpp"]
# the page rows ("attention_forward" Shapes table) of the prefill workloads
WORKLOAD_PAGE_ROWS = {"prefill_s276_h4_d72": 11, "prefill_s8136_h16_d72": 4,
                      "prefill_s16742_h32_d128": 9, "prefill_s65556_h16_d72": 8}
# the prefill workloads of the benchmark configuration list
PREFILL_CONFIGS = ["prefill_s276_h4_d72", "prefill_s8136_h16_d72", "prefill_s16742_h32_d128",
                   "prefill_s65556_h16_d72"]


def prefill_kernel(head_dim, seq_len, num_heads):
    """(name prefix, label) of the kernel the library runs for a one-sequence
    prefill of these sizes on a 256-CU device: the choice the library makes
    (choose_prefill in csrc/attn_api.hip), restated for the label only."""
    if head_dim == 128:
        return "prefill_fwd_d128_kernel", "prefill_fwd_d128_kernel<bf16>"
    if num_heads * -(-seq_len // 32) <= 512 and seq_len <= 8192:
        return "prefill_fwd_split_kernel", "prefill_fwd_split_kernel<bf16, 4>"
    items256 = num_heads * -(-seq_len // 256)
    if items256 >= 512 or seq_len >= 6144:
        return "prefill_fwd_d72_kernel", "prefill_fwd_d72_kernel<bf16>"
    waves = 8 if items256 >= 256 else 4
    return "prefill_fwd_kernel", f"prefill_fwd_kernel<72, bf16, {waves}>"


class ClockSampler:
    """Samples the GPU shader clock (the current level of pp_dpm_sclk in sysfs)
    from a background thread while a timed region runs."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for path in self.paths:
            try:
                with open(path) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            return float(re.search(r"(\d+)\s*[Mm]hz", line).group(1))
            except (OSError, AttributeError, ValueError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"source": "pp_dpm_sclk", "samples": 0, "note": "not readable on this machine"}
        v = sorted(self.samples)
        return {"source": "sysfs pp_dpm_sclk (current level), sampled during the timed prefill launches",
                "samples": len(v), "mean_mhz": round(sum(v) / len(v)), "median_mhz": v[len(v) // 2],
                "min_mhz": v[0], "max_mhz": v[-1]}


def kernel_source_hash(names):
    """Hash of the code of kernel source files, comments and blank space left
    out (so that an edited comment keeps the counter figures taken on the
    same code)."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "softmax_attention_flashattention_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(kernel_prefix, src_hash):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_prefix)
    if not entry or entry.get("source_hash") != src_hash:
        return None
    return entry.get("bytes_per_launch")


def prefill_flops(inp):
    cq = inp["cu_seqlens_q"].tolist()
    ck = inp["cu_seqlens_k"].tolist()
    H, D = inp["q"].shape[1], inp["q"].shape[2]
    return sum(4.0 * (cq[i + 1] - cq[i]) * (ck[i + 1] - ck[i]) * H * D for i in range(len(cq) - 1))


def decode_bytes(inp):
    """Algorithmic bytes of one decode call: K and V of the tokens in context,
    the query, the output, the block table and seq_lens."""
    S, Hq, D = inp["query"].shape
    Hkv = inp["v_cache"].shape[1]
    el = inp["query"].element_size()
    tokens = int(inp["seq_lens"].clamp(min=0).sum())
    return (2 * tokens * Hkv * D * el + 2 * S * Hq * D * el
            + inp["block_tables"].numel() * 4 + inp["seq_lens"].numel() * 4)


def chunk_bytes(inp):
    """Algorithmic bytes of one chunked delta-rule output call: q, k, v, h
    and g read once, the output written once."""
    return sum(inp[n].numel() * inp[n].element_size() for n in ("q", "k", "v", "h", "g")) \
        + inp["v"].numel() * inp["v"].element_size()


def oracle_prefill_sample(name, budget_s):
    """The oracle's whole-workload prefill entry point on the first n query
    rows of the first h heads of a prefill workload (a query segment of n rows
    against all of the sequence's keys: the definition for those rows,
    computed the way a whole run computes them), sized to about budget_s
    seconds: rows of head 0 first, then whole heads."""
    import oracle
    import torch
    from softmax_attention_flashattention_amd import inputs as gen
    inp = gen.workload_inputs(name)
    S, H, D = inp["q"].shape

    def run(n, h):
        q = inp["q"][:n, :h].contiguous()
        k, v = inp["k"][:, :h].contiguous(), inp["v"][:, :h].contiguous()
        cu_q = torch.tensor([0, n], dtype=torch.int32)
        t0 = time.perf_counter()
        oracle.varlen_fwd(q, k, v, cu_q, inp["cu_seqlens_k"])
        return time.perf_counter() - t0

    n, h = min(S, max(oracle.num_threads(), 16)), 1
    t = run(n, h)
    runs = [(n, h, t)]
    for _ in range(2):
        target = int(n * h * budget_s / max(t, 1e-3))
        if target <= S:
            n, h = max(n, target), 1
        else:
            n, h = S, int(min(H, max(1, target // S)))
        t = run(n, h)
        runs.append((n, h, t))
    # A whole run gathers each head's keys and values once, then computes
    # its rows: per head, time = a + b x rows.  a and b from the smallest and
    # largest sample; the whole workload takes H (a + b S).
    (n1, h1, t1), (n2, h2, t2) = runs[0], runs[-1]
    b = (t2 / h2 - t1 / h1) / (n2 - n1) if n2 > n1 else t2 / (h2 * n2)
    a = max(0.0, t2 / h2 - b * n2)
    b = (t2 / h2 - a) / n2
    flops = prefill_flops(inp)
    if n * h == S * H:   # the budget covered the whole workload
        return {"mode": "full", "seconds": round(t, 3), "tflops": flops / t / 1e12}
    return {"mode": "sample", "rows": n, "heads": h, "of_row_heads": S * H, "keys": S,
            "seconds": round(t, 3), "tflops": flops * n * h / (S * H) / t / 1e12,
            "extrapolated_full_seconds": round(H * (a + b * S), 1),
            "extrapolation": f"per head {a:.3g} s for the keys + {b:.3g} s per row, times {H} heads"}


def cpu_baseline(budget_s):
    """The oracle, as it stands, on a bounded sample of the step's prefill
    workload: its first query rows (of head 0, then of whole heads), each
    against all keys."""
    import oracle
    smp = oracle_prefill_sample(PREFILL, budget_s)
    if smp["mode"] == "full":
        return {"value": smp["tflops"], "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"all of {PREFILL} through the oracle's whole-workload prefill entry point, "
                          f"float64, {smp['seconds']:.1f} s",
                "extrapolated_full_seconds": smp["seconds"], "_sample": smp}
    return {"value": smp["tflops"], "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the first {smp['rows']} query rows of the first {smp['heads']} head(s) of "
                      f"{PREFILL} (of {smp['of_row_heads']} (row, head) pairs), each against all "
                      f"{smp['keys']} keys, "
                      f"through the oracle's whole-workload prefill entry point, float64, "
                      f"{smp['seconds']:.1f} s",
            "extrapolated_full_seconds": smp["extrapolated_full_seconds"],
            "_sample": smp}


def oracle_per_config(budget_s, known=None):
    """The oracle, as it stands, on each benchmark workload: in full where that
    takes seconds (the 276-token prefill, the decode workload), else on a
    sample (oracle_prefill_sample) with the full-workload time extrapolated as
    seconds x (rows x heads) / n and labelled as such.  `known` holds samples
    already taken (by workload name)."""
    import oracle
    from softmax_attention_flashattention_amd import inputs as gen
    threads = oracle.num_threads()
    res = {}
    for name in PREFILL_CONFIGS:
        if known and name in known:
            res[name] = dict(known[name])
            continue
        inp = gen.workload_inputs(name)
        S, H, D = inp["q"].shape
        if S * S * H <= 1 << 24:
            t0 = time.perf_counter()
            oracle.varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"])
            t = time.perf_counter() - t0
            res[name] = {"mode": "full", "seconds": round(t, 4), "tflops": prefill_flops(inp) / t / 1e12}
            continue
        res[name] = oracle_prefill_sample(name, budget_s)
    inp = gen.workload_inputs(DECODE)
    t0 = time.perf_counter()
    oracle.paged_decode(inp["query"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["seq_lens"])
    t = time.perf_counter() - t0
    res[DECODE] = {"mode": "full", "seconds": round(t, 4), "gbs": decode_bytes(inp) / t / 1e9}
    for v in res.values():
        for key in ("tflops", "gbs"):
            if key in v:
                v[key] = float(f"{v[key]:.4g}")
    return {"cores": threads, "kind": "oracle", "per_config": res}


def copy_reference(torch, dev, args):
    """A plain 1 GiB device-to-device copy (torch's copy kernel): its measured
    bandwidth, and the reference launch for scaling HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "avg_ms": round(ms, 4),
                      "GB/s (read + write)": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def summarize_counters(pmc_dir):
    """Turns four rocprofv3 --pmc runs into profiles/hbm_traffic.json: HBM bytes
    per launch of each kernel, FETCH_SIZE and WRITE_SIZE each scaled by what the
    same counter reads for a plain 1 GiB copy (the --only copy run).

    Expected layout (the -d/-o names of the four runs):
      <pmc_dir>/f/f_counter_collection.csv    FETCH_SIZE, default bench step
      <pmc_dir>/w/w_counter_collection.csv    WRITE_SIZE, default bench step
      <pmc_dir>/cf/cf_counter_collection.csv  FETCH_SIZE, --only copy
      <pmc_dir>/cw/cw_counter_collection.csv  WRITE_SIZE, --only copy
    """
    import csv
    import collections

    def per_kernel(name):
        path = os.path.join(pmc_dir, name, f"{name}_counter_collection.csv")
        vals = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch, write = per_kernel("f"), per_kernel("w")
    cf, cw = per_kernel("cf"), per_kernel("cw")
    copy_kib = (1 << 30) / 1024.0
    copy_kernel = max(cf, key=cf.get)            # the 1 GiB copy dominates
    fetch_scale = copy_kib / cf[copy_kernel]
    write_scale = copy_kib / cw[max(cw, key=cw.get)]
    out = {"_note": ("HBM bytes per launch = FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale "
                     "(KiB -> bytes); scales from a plain 1 GiB device copy"),
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "copy_kernel": copy_kernel}
    for prefix in KERNEL_SOURCES:
        names = [k for k in fetch if prefix in k]
        if not names:
            continue
        k = names[0]
        rd = fetch[k] * fetch_scale * 1024.0
        wr = write.get(k, 0.0) * write_scale * 1024.0
        out[prefix] = {"kernel": k, "source_hash": kernel_source_hash(KERNEL_SOURCES[prefix]),
                       "read_bytes": round(rd),
                       "write_bytes": round(wr), "bytes_per_launch": round(rd + wr)}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def shapes_rows(torch, dev, which):
    """Times every row of one operator page's Shapes table (seeded inputs of
    the row's sizes) and prints one JSON line per row: the per-launch time
    of back-to-back launches, the achieved rate against its roofline and the
    page's production time for context.  Rows under 200 us per launch are
    also timed as 20 calls captured in a HIP graph and replayed (no per-call
    host path): the device-side rate a launch-bound caller can reach."""
    sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))
    import shapes
    from softmax_attention_flashattention_amd import (attn_chunk_delta_out, attn_paged_decode,
                                                      attn_varlen_fwd, attn_varlen_fwd_workspace_size)
    from softmax_attention_flashattention_amd import inputs as gen

    def timed(call, min_ms=30.0):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        n = 1
        while True:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                call()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            if ms >= min_ms or n >= 4096:
                return ms / n
            n *= 4

    def graph_timed(call, per_graph=20, reps=20):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                call()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * per_graph)

    rows = {"prefill": shapes.prefill_rows, "decode": shapes.decode_rows,
            "chunk": shapes.chunk_rows}[which]()
    for r in rows:
        if which == "prefill":
            x = gen.prefill_inputs([r["seq_len"]], r["num_heads"], r["head_dim"], seed=2000 + r["row"])
            d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
            out = torch.empty_like(d["q"])
            ws = torch.empty(attn_varlen_fwd_workspace_size(1, x["max_seqlen_q"], r["num_heads"],
                                                            r["head_dim"]), dtype=torch.uint8,
                             device=dev)
            call = lambda: attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"],
                                           d["cu_seqlens_k"], max_seqlen_q=x["max_seqlen_q"],
                                           out=out, workspace=ws)
            work = prefill_flops(x)
            unit, peak = "TFLOP/s", PEAK_BF16_TFLOPS
        elif which == "decode":
            x = gen.decode_inputs(r["num_seqs"], r["ctx_len"], r["num_query_heads"],
                                  r["num_kv_heads"], r["head_size"], seed=3000 + r["row"],
                                  dtype=r["dtype"])
            d = {k: v.to(dev) for k, v in x.items()}
            out = torch.empty_like(d["query"])
            call = lambda: attn_paged_decode(d["query"], d["k_cache"], d["v_cache"],
                                             d["block_tables"], d["seq_lens"], out=out)
            work = decode_bytes(x)
            unit, peak = "GB/s", PEAK_HBM_GBS
        else:
            x = gen.chunk_inputs(r["batch_size"], r["token_count"], r["num_q_heads"],
                                 r["num_v_heads"], seed=4000 + r["row"])
            d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
            out = torch.empty_like(d["v"])
            call = lambda: attn_chunk_delta_out(d["q"], d["k"], d["v"], d["h"], d["g"], out=out)
            work = chunk_bytes(x)
            unit, peak = "GB/s", PEAK_HBM_GBS
        scale = 1e12 if which == "prefill" else 1e9
        ms = timed(call)
        rate = work / (ms * 1e-3) / scale
        gms = graph_timed(call) if ms < 0.2 else None
        sizes = {k: v for k, v in r.items() if k not in ("t_sol_us", "t_prod_us")}
        line = {"shapes": which, **sizes, "us_per_launch": round(ms * 1e3, 2),
                "achieved": round(rate, 1), "unit": unit, "frac": round(rate / peak, 4),
                "graph_us_per_launch": None if gms is None else round(gms * 1e3, 2),
                "graph_frac": None if gms is None else round(work / (gms * 1e-3) / scale / peak, 4),
                "page_t_prod_us": r["t_prod_us"]}
        print(json.dumps(line), flush=True)
        del x, d, out


def decode_partition_sweep(torch, dev):
    """Every row of the decode Shapes table, plus three shapes with few long
    contexts, timed with the library's own partition choice (partition_size
    0) and with forced 16- to 512-token partitions: per-launch time of 20
    calls captured in a HIP graph, the median of 6 rounds of 10 replays (the
    choices of a shape alternate in order from round to round).  One JSON
    line per shape; `max_abs_diff` compares every forced split with the
    automatic one."""
    sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))
    import shapes
    from softmax_attention_flashattention_amd import attn_paged_decode, attn_paged_decode_num_partitions
    from softmax_attention_flashattention_amd import inputs as gen

    def capture(call, per_graph=20):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                call()
        g.replay()
        torch.cuda.synchronize()
        return g

    def graph_us(graphs, per_graph=20, reps=10, rounds=6):
        # rounds in alternating order, median per graph: no choice is timed
        # only on a GPU that is still ramping up
        ts = {k: [] for k in graphs}
        keys = list(graphs)
        for i in range(rounds):
            for k in (keys if i % 2 == 0 else keys[::-1]):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    graphs[k].replay()
                b.record()
                torch.cuda.synchronize()
                ts[k].append(a.elapsed_time(b) / (reps * per_graph) * 1e3)
        return {k: round(sorted(v)[len(v) // 2], 2) for k, v in ts.items()}

    long_ctx = [dict(row="long-1", num_seqs=1, ctx_len=1024, num_query_heads=16, num_kv_heads=2,
                     head_size=128, dtype="bf16"),
                dict(row="long-2", num_seqs=4, ctx_len=2048, num_query_heads=32, num_kv_heads=8,
                     head_size=128, dtype="bf16"),
                dict(row="long-3", num_seqs=1, ctx_len=4096, num_query_heads=8, num_kv_heads=1,
                     head_size=128, dtype="bf16")]
    for r in list(shapes.decode_rows()) + long_ctx:
        x = gen.decode_inputs(r["num_seqs"], r["ctx_len"], r["num_query_heads"], r["num_kv_heads"],
                              r["head_size"], seed=3000, dtype=r["dtype"])
        d = {k: v.to(dev) for k, v in x.items()}
        maxb = x["block_tables"].shape[1]
        graphs, outs = {}, {}
        for ps in (0, 16, 32, 64, 128, 256, 512):
            if ps >= 2 * max(r["ctx_len"], 16):
                continue
            key = "auto" if ps == 0 else str(ps)
            out = outs[key] = torch.empty_like(d["query"])
            graphs[key] = capture(lambda out=out, ps=ps: attn_paged_decode(
                d["query"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], out=out,
                partition_size=ps))
        times = graph_us(graphs)
        auto = outs["auto"].float()
        diff = max((o.float() - auto).abs().max().item() for o in outs.values())
        print(json.dumps({"decode_partitions": r["row"], "num_seqs": r["num_seqs"],
                          "ctx_len": r["ctx_len"], "num_query_heads": r["num_query_heads"],
                          "num_kv_heads": r["num_kv_heads"], "head_size": r["head_size"],
                          "dtype": r["dtype"],
                          "auto_partitions": attn_paged_decode_num_partitions(
                              r["num_seqs"], r["num_kv_heads"], maxb, 16),
                          "graph_us_by_partition_tokens": times, "max_abs_diff": diff}), flush=True)
        del x, d


# device-filling decode shapes with grouped query heads (sequences, context,
# query heads, KV heads, head_size): where the library runs the score and
# value products on MFMAs, and the one-query-head-per-KV-head cases beside
GROUPED_DECODE_SHAPES = [
    (64, 2048, 8, 8, 128), (64, 2048, 16, 8, 128), (64, 2048, 32, 8, 128), (64, 2048, 64, 8, 128),
    (64, 2048, 128, 8, 128), (256, 512, 32, 8, 128), (256, 128, 64, 8, 128), (256, 64, 128, 8, 128),
    (128, 1024, 16, 16, 256), (128, 512, 64, 8, 256), (32, 2048, 64, 4, 256), (64, 256, 128, 8, 256),
]


def decode_grouped(torch, dev):
    """Paged decode on device-filling grids with 1-16 query heads per KV head:
    per-launch time of 20 calls captured in a HIP graph (median of 6 rounds of
    5 replays), the K/V bytes read per second, and which kernel the library
    chose.  One JSON line per shape."""
    from softmax_attention_flashattention_amd import attn_paged_decode
    from softmax_attention_flashattention_amd import inputs as gen
    for (S, ctx, hq, hkv, d) in GROUPED_DECODE_SHAPES:
        x = gen.decode_inputs(S, ctx, hq, hkv, d, seed=4242)
        t = {k: v.to(dev) for k, v in x.items()}
        out = torch.empty_like(t["query"])
        call = lambda: attn_paged_decode(t["query"], t["k_cache"], t["v_cache"], t["block_tables"],
                                         t["seq_lens"], out=out)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                call()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(5):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 100 * 1e3)
        us = sorted(ts)[len(ts) // 2]
        kv = 2 * S * ctx * hkv * d * 2
        G = hq // hkv
        print(json.dumps({"decode_grouped": f"{S}x{ctx}", "num_seqs": S, "ctx_len": ctx, "num_query_heads": hq,
                          "num_kv_heads": hkv, "head_size": d, "query_heads_per_kv_head": G,
                          "graph_us_per_launch": round(us, 2), "kv_bytes": kv,
                          "gbs": round(kv / us / 1e3, 1), "frac": round(kv / us / 1e3 / PEAK_HBM_GBS, 4)}),
              flush=True)
        del x, t, out, g


def page_context(p_host):
    """The pages' own times for the timed workloads (Shapes tables stored under
    tests/golden): T_SOL on hardware the pages label only "XPU-A", T_Prod on
    unstated hardware.  Context, never a target."""
    sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))
    import shapes
    S, H, D = int(p_host["max_seqlen_q"]), int(p_host["q"].shape[1]), int(p_host["q"].shape[2])
    pre = [r for r in shapes.prefill_rows()
           if (r["seq_len"], r["num_heads"], r["head_dim"]) == (S, H, D)]
    dec = [r for r in shapes.decode_rows()
           if (r["num_seqs"], r["ctx_len"], r["num_query_heads"], r["num_kv_heads"],
               r["head_size"]) == (256, 64, 16, 16, 128)]
    chk = [r for r in shapes.chunk_rows()
           if (r["token_count"], r["num_v_heads"], r["num_q_heads"]) == (14807, 32, 16)]
    ctx = {"hardware": "XPU-A (name missing from the pages); T_Prod hardware unstated",
           "note": "context only, not a target"}
    for key, rows in (("prefill", pre), ("decode", dec), ("chunk", chk)):
        if rows:
            ctx[key] = {"page_row": rows[0]["row"], "t_sol_us": rows[0]["t_sol_us"],
                        "t_prod_us": rows[0]["t_prod_us"]}
    return ctx


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (the shader clock settles over the first few launches)")
    ap.add_argument("--rotate", type=int, default=8,
                    help="decode input copies cycled through (8 x 138 MB > 256 MB cache)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU work for the oracle baseline (0 skips it)")
    ap.add_argument("--only", choices=["prefill", "decode", "chunk", "copy"], default=None,
                    help="time one part alone (for profiling); 'copy' times a plain 1 GiB "
                         "device-to-device copy, the reference for HBM counter scaling")
    ap.add_argument("--prefill-workload", default=PREFILL,
                    choices=[k for k in ("prefill_s276_h4_d72", "prefill_s8136_h16_d72",
                                         "prefill_s16742_h32_d128", "prefill_s65556_h16_d72")],
                    help="prefill workload of the step (default: the head_dim-128 roofline case)")
    ap.add_argument("--shapes", choices=["prefill", "decode", "chunk"], default=None,
                    help="time every row of that operator page's Shapes table (one JSON line "
                         "per row) and exit")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads after the step (counter runs use this "
                         "so that each kernel name in their output is one workload)")
    ap.add_argument("--decode-partitions", action="store_true",
                    help="time the decode Shapes rows and three few-long-context shapes with the "
                         "automatic and with forced context partitions (one JSON line each) and exit")
    ap.add_argument("--decode-grouped", action="store_true",
                    help="time device-filling decode shapes with 1-16 query heads per KV head "
                         "(one JSON line each) and exit")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR", default=None,
                    help="write profiles/hbm_traffic.json from rocprofv3 counter runs and exit "
                         "(no GPU needed)")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single GPU and no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from softmax_attention_flashattention_amd import (attn_chunk_delta_out, attn_paged_decode,
                                                      attn_varlen_fwd)
    from softmax_attention_flashattention_amd import inputs as gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if args.only == "copy":
        return copy_reference(torch, dev, args)
    if args.shapes:
        return shapes_rows(torch, dev, args.shapes)
    if args.decode_partitions:
        return decode_partition_sweep(torch, dev)
    if args.decode_grouped:
        return decode_grouped(torch, dev)

    p_name = args.prefill_workload
    p_host = gen.workload_inputs(p_name)
    p = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p_host.items()}
    p_out = torch.empty_like(p["q"])
    from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
    p_ws = torch.empty(attn_varlen_fwd_workspace_size(p_host["cu_seqlens_q"].numel() - 1,
                                                      p_host["max_seqlen_q"], p_host["q"].shape[1],
                                                      p_host["q"].shape[2]),
                       dtype=torch.uint8, device=dev)
    flops = prefill_flops(p_host)

    d_host = gen.workload_inputs(DECODE)
    d_copies = []
    for _ in range(max(1, args.rotate)):
        d_copies.append({k: v.to(dev) for k, v in d_host.items()})
    d_out = [torch.empty_like(c["query"]) for c in d_copies]
    dbytes = decode_bytes(d_host)

    def prefill_call():
        attn_varlen_fwd(p["q"], p["k"], p["v"], p["cu_seqlens_q"], p["cu_seqlens_k"],
                        max_seqlen_q=p["max_seqlen_q"], out=p_out, workspace=p_ws)

    def decode_call(i):
        c = d_copies[i % len(d_copies)]
        attn_paged_decode(c["query"], c["k_cache"], c["v_cache"], c["block_tables"],
                          c["seq_lens"], out=d_out[i % len(d_copies)])

    c_host = gen.workload_inputs(CHUNK)
    ck = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in c_host.items()}
    c_out = torch.empty_like(ck["v"])
    cbytes = chunk_bytes(c_host)

    def chunk_call():
        attn_chunk_delta_out(ck["q"], ck["k"], ck["v"], ck["h"], ck["g"],
                             chunk_size=ck["chunk_size"], out=c_out)

    do_prefill = args.only in (None, "prefill")
    do_decode = args.only in (None, "decode")
    do_chunk = args.only in (None, "chunk")
    for i in range(args.warmup):
        if do_prefill:
            prefill_call()
        if do_decode:
            decode_call(i)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    clock = ClockSampler()
    with clock:
        t0 = time.perf_counter()
        for i in range(args.steps):
            a, b, c, d = ev[i]
            a.record()
            if do_prefill:
                prefill_call()
            b.record()
            c.record()
            if do_decode:
                decode_call(args.warmup + i)
            d.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    pre_ms = sorted(a.elapsed_time(b) for a, b, _, _ in ev)
    dec_ms = sorted(c.elapsed_time(d) for _, _, c, d in ev)
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_step_avg = sum(dec_ms) / len(dec_ms)
    # Decode calls are short enough (tens of microseconds) that a lone call's
    # event pair also times its dispatch; its per-launch figure comes from the
    # same calls issued back to back (still rotating the input copies).
    dec_avg = dec_step_avg
    if do_decode:
        reps = 4 * args.steps
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            decode_call(i)
        b.record()
        torch.cuda.synchronize()
        dec_avg = a.elapsed_time(b) / reps
    # The chunked delta-rule output (a further operator, not part of the
    # step): its own back-to-back launches.  One call streams 608 MB, beyond
    # the 256 MB Infinity Cache, so no input rotation is needed.
    chunk_avg = 0.0
    if do_chunk:
        for _ in range(args.warmup):
            chunk_call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            chunk_call()
        b.record()
        torch.cuda.synchronize()
        chunk_avg = a.elapsed_time(b) / args.steps
    tflops = flops / (pre_avg * 1e-3) / 1e12 if do_prefill else 0.0
    gbs = dbytes / (dec_avg * 1e-3) / 1e9 if do_decode else 0.0

    # The other benchmark workloads (page rows 11, 4 and 8 of the prefill
    # Shapes table), each timed on its own: back-to-back launches bracketed by
    # one event pair; the 276-token one, a few microseconds of work, also as
    # 20 calls captured in a HIP graph and replayed (no per-call host path).
    configs = {}
    if args.only is None and p_name == PREFILL and not args.no_configs:
        from softmax_attention_flashattention_amd import attn_varlen_fwd_workspace_size
        for name in PREFILL_CONFIGS:
            if name == PREFILL:
                continue
            x_host = gen.workload_inputs(name)
            x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x_host.items()}
            S, H, D = x_host["q"].shape
            x_out = torch.empty_like(x["q"])
            x_ws = torch.empty(attn_varlen_fwd_workspace_size(1, S, H, D), dtype=torch.uint8, device=dev)

            def call(x=x, x_out=x_out, x_ws=x_ws):
                attn_varlen_fwd(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["cu_seqlens_k"],
                                max_seqlen_q=x["max_seqlen_q"], out=x_out, workspace=x_ws)

            xf = prefill_flops(x_host)
            reps = max(10, min(2000, int(5e13 / xf)))   # 25 ms or more of launches
            for _ in range(3):
                call()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            rate = xf / (ms * 1e-3) / 1e12
            entry = {"head_dim": D, "kernel": prefill_kernel(D, S, H)[1], "flops_per_launch": xf,
                     "launches": reps, "avg_launch_us": round(ms * 1e3, 2), "achieved": round(rate, 1),
                     "unit": "TFLOP/s", "frac": round(rate / PEAK_BF16_TFLOPS, 4)}
            if ms < 0.2:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(20):
                        call()
                g.replay()
                torch.cuda.synchronize()
                a.record()
                for _ in range(20):
                    g.replay()
                b.record()
                torch.cuda.synchronize()
                gms = a.elapsed_time(b) / 400
                entry["graph_us_per_launch"] = round(gms * 1e3, 2)
                entry["graph_frac"] = round(xf / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            configs[name] = entry
            del x, x_out, x_ws

    def traffic(prefix):
        return profiled_traffic(prefix, kernel_source_hash(KERNEL_SOURCES[prefix]))

    src_hash = kernel_source_hash(ALL_SOURCES)
    pre_prefix, pre_label = prefill_kernel(int(p_host["q"].shape[2]), int(p_host["max_seqlen_q"]),
                                           int(p_host["q"].shape[1]))
    pre_traffic = traffic(pre_prefix) if p_name == PREFILL else None
    dec_traffic = traffic("decode_partition_kernel")
    chunk_traffic = traffic("chunk_delta_out_kernel")
    cgbs = cbytes / (chunk_avg * 1e-3) / 1e9 if do_chunk else 0.0

    result = {
        "metric": "prefill attn TFLOP/s & % MFMA peak; paged-decode GB/s & % HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{p_name} + {DECODE}",
            "prefill": {"seq_lens": [int(p_host["max_seqlen_q"])],
                        "num_heads": int(p_host["q"].shape[1]),
                        "head_dim": int(p_host["q"].shape[2]),
                        "scale": "head_dim^-0.5", "causal": False},
            "decode": {"num_seqs": 256, "ctx_len": 64, "num_query_heads": 16,
                       "num_kv_heads": 16, "head_size": 128, "block_size": 16,
                       "input_copies_rotated": len(d_copies)},
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": pre_traffic,
            "kernel": pre_label,
            "flops_per_launch": flops, "avg_launch_ms": round(pre_avg, 4),
            "min_launch_ms": round(pre_ms[0], 4),
            "median_launch_ms": round(pre_ms[len(pre_ms) // 2], 4),
            "shader_clock": clock.summary(),
        },
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {
                "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": dec_traffic,
                "kernel": "decode_partition_kernel<bf16, 1>",
                "bytes_per_launch": dbytes, "avg_launch_us": round(dec_avg * 1e3, 3),
                "avg_in_step_us": round(dec_step_avg * 1e3, 3),
                "min_in_step_us": round(dec_ms[0] * 1e3, 3),
            },
        },
        "chunk": {
            "workload": CHUNK, "value": round(cgbs, 1), "unit": "GB/s",
            "roofline": {
                "bound": "hbm", "achieved": round(cgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(cgbs / PEAK_HBM_GBS, 4), "traffic": chunk_traffic,
                "kernel": "chunk_delta_out_kernel<bf16>", "bytes_per_launch": cbytes,
                "avg_launch_us": round(chunk_avg * 1e3, 3),
            },
        },
        "configs": configs,
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
        "kernel_source_hash": src_hash,
        "page_context": page_context(p_host),
    }
    for name, entry in configs.items():
        row = WORKLOAD_PAGE_ROWS.get(name)
        entry["page_row"] = row
    # this run's per-launch times beside the pages' (context only)
    for key, us, on in (("prefill", pre_avg * 1e3, do_prefill), ("decode", dec_avg * 1e3, do_decode),
                        ("chunk", chunk_avg * 1e3, do_chunk)):
        if on and key in result["page_context"]:
            result["page_context"][key]["this_run_us"] = round(us, 2)
    if args.only is not None:
        result["only"] = args.only
    if args.cpu_budget > 0 and args.only is None:
        cb = cpu_baseline(args.cpu_budget)
        smp = cb.pop("_sample")
        if p_name == PREFILL and tflops > 0:
            cb["gpu_over_cpu"] = round(tflops / cb["value"], 1)
        cb["workloads"] = oracle_per_config(max(1.0, args.cpu_budget / 5),
                                            known={PREFILL: smp})["per_config"]
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
