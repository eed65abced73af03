"""Throughput of the MSA sparse-layer decode step on one MI355X.

A step is one pass of the whole hot path over one batch: block scores over the
FP8 index cache, top-k block selection, and sparse attention over the selected
FP8 K/V pages with its split-K merge.  The timed step is msa_decode_step: the
score launch, then msa_select_sparse_decode's attention launch, which selects
each token's blocks itself, and the split merge.  Each public call on its own
and the step as the three separate calls are timed too.
Workload: 16 request rows x 4 query tokens (1 + 3 speculative), 16384-token
context per row (128 blocks of 128), 16 query heads / 1 KV head, head dim 128,
index dim 128, top-k 16, a 4096-page pool with random non-overlapping block
tables (synthetic seeded data).

Timing: M independent copies of the pools (192 MiB each) are rotated so that
each step reads cold data rather than the 256 MB Infinity Cache; M steps are
captured into one HIP graph, replayed after warm-up, and bracketed by HIP
events on the stream the kernels run on.  The roofline figure is for the
attention launch of the step (msa_select_sparse_decode timed on its own the
same way): its algorithmic bytes over its duration.  The CPU baseline is the
oracle (plain C, fp64) running full steps of the same batch on the host cores.

Also in the line: the same step on one pool copy (cache-resident, not an HBM
figure), the streaming rates of library kernels on the same GPU, the step at
top-k 8, 32 and 128 and at 1, 4, 8 and 16 rows, the prefill score sheet and the ragged prefill call
(MFMA rooflines), and the attention variants (dense bf16 caches, one
selection per request, one per KV head).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the launch msa_select_sparse_decode makes at this shape
ROOFLINE_KERNEL = "attn_token_select_kernel<128, 2>"
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--k", type=int, default=16)
    ap.add_argument("--copies", type=int, default=0,
                    help="pool copies rotated per graph (0: the largest count in 5..16 that divides "
                         "both --steps and --warmup, preferring 8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill block-score measurement")
    ap.add_argument("--kernels", default="score,select,decode,select_decode,calls",
                    help="extra timing graphs to build (per call, and the three-call step)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain fp32 streaming kernel (out = in * 1) over this many MiB, "
                         "8 times, as the reference for HBM byte counters")
    ap.add_argument("--calib-out", default=".",
                    help="directory for calib.json (the copy size and the calls' algorithmic bytes)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the dense bf16 K/V attention variant")
    ap.add_argument("--ktrace-summary", nargs=3, metavar=("DIR", "NAME", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace --stats --output-format csv run in DIR "
                         "(made by COMMAND) into profiles/NAME_kernels.md and the kernel durations "
                         "bench.py reports beside its event timings (profiles/kernel_durations.json); "
                         "needs no GPU")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script made with --calib-copy-mib, write profiles/traffic.json, print a "
                         "table; needs no GPU")
    return ap.parse_args()


def plan_copies(steps: int, warmup: int, copies: int = 0) -> tuple[int, int, int]:
    """Pool copies M per step graph, and the steps and warmup steps actually run
    (multiples of M).  M >= 5 copies x the step's 62 MB exceed the 256 MB
    Infinity Cache, so every step reads cold data; when some M in 5..16 divides
    both counts they are run exactly."""
    steps, warmup = max(1, steps), max(0, warmup)
    if copies > 0:
        m = copies
    else:
        divs = lambda x: [c for c in range(16, 4, -1) if x % c == 0]
        both = [c for c in divs(steps) if warmup % c == 0]
        pick = lambda cs: (8 if 8 in cs else cs[0]) if cs else None
        m = pick(both) or pick(divs(steps)) or 8
    return m, -(-steps // m) * m, -(-warmup // m) * m


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_paged_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case, topk: np.ndarray) -> dict:
    """Bytes each call must move at minimum: every page a row touches once per
    row, each small input once, each output once."""
    R, T, N, MB, B = case.R, case.T, case.N, case.MB, case.B
    lens = case.seq_lens.numpy().astype(np.int64)
    Di, D, Hq, Hkv, k = case.Di, case.D, case.Hq, case.Hkv, topk.shape[1]
    index = int(lens.sum()) * Di * 1
    kv_tokens = 0
    for r in range(R):
        ids = np.unique(topk[r * T:(r + 1) * T])
        ids = ids[ids >= 0]
        kv_tokens += int(sum(min(B, lens[r] - j * B) for j in ids if j * B < lens[r]))
    kv = kv_tokens * Hkv * D * 1 * 2
    paging = R * MB * 4 + R * 4                 # block table + seq_lens
    score_sheet = N * MB * 4
    sel = N * k * 4
    qo = N * Hq * D * 2 * 2                     # bf16 queries in, bf16 output out
    score = index + N * Di * 2 + score_sheet + paging
    select = score_sheet + sel
    attend = kv + qo + sel + paging
    select_decode = kv + qo + score_sheet + sel + paging
    return dict(score=score, select=select, decode=attend, select_decode=select_decode,
                step=score + select_decode, calls=score + select + attend, index=index, kv=kv)


# kernels whose counters the PMC summary reports, by the call that launches them
PMC_KERNELS = {"select_decode": "attn_token_select_kernel", "score": "score_mfma_decode_kernel"}
CALIB_KERNEL = "MulFunctor"          # the reference streaming kernel of --calib-copy-mib


def short_kernel_name(name: str) -> str:
    """A kernel's name without its return type, namespaces and argument list,
    e.g. 'attn_token_select_kernel<128, 2>' for rocprofv3's full
    'void msa::(anonymous namespace)::attn_token_select_kernel<128, 2>(msa::AttnParams)'."""
    depth = 0
    for i in range(len(name) - 1, -1, -1):            # the trailing argument list
        if name[i] == ")":
            depth += 1
        elif name[i] == "(":
            depth -= 1
            if depth == 0:
                name = name[:i]
                break
    cut, tdepth, pdepth = 0, 0, 0
    for i, c in enumerate(name):
        if c == "<":
            tdepth += 1
        elif c == ">":
            tdepth -= 1
        elif c == "(":
            pdepth += 1
        elif c == ")":
            pdepth -= 1
        elif tdepth == 0 and pdepth == 0:
            if c == " ":
                cut = i + 1
            elif c == ":" and name[i + 1:i + 2] == ":":
                cut = i + 2
    return name[cut:]


def ktrace_summary(run_dir: str, name: str, command: str) -> None:
    """profiles/<name>_kernels.md from a rocprofv3 kernel_stats.csv, and the average
    duration of each kernel, keyed by the kernel sources' digest, into
    profiles/kernel_durations.json."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# Kernel durations: {name}", "",
             "Command (run from the repository root on an MI355X host):", "", f"    {command}", "",
             f"rocprofv3 --kernel-trace --stats, all dispatches of the run; kernel sources digest "
             f"`{kernel_source_digest()}`.", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    avg = {}
    for r in rows[:14]:
        short = short_kernel_name(r["Name"])
        short = short if len(short) <= 90 else short[:90]
        a_us = float(r["AverageNs"]) / 1e3
        avg[short_kernel_name(r["Name"])] = round(a_us, 3)
        lines.append(f"| `{short}` | {r['Calls']} | {a_us:.3f} | {float(r['MinNs']) / 1e3:.3f} | "
                     f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f}% |")
    with open(os.path.join(ROOT, "profiles", f"{name}_kernels.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    jf = os.path.join(ROOT, "profiles", "kernel_durations.json")
    data = json.load(open(jf)) if os.path.exists(jf) else {}
    if data.get("source_digest") != kernel_source_digest():
        data = {"source_digest": kernel_source_digest(), "kernels": {}}
    data["kernels"].update(avg)
    with open(jf, "w") as fh:
        json.dump(data, fh, indent=1)
    print("\n".join(lines))


def rocprof_duration_us(kernel: str):
    """Average duration of `kernel` (name up to its argument list) in the committed
    rocprofv3 summary, or None when the summary was taken of other kernel sources."""
    jf = os.path.join(ROOT, "profiles", "kernel_durations.json")
    try:
        data = json.load(open(jf))
    except Exception:
        return None
    if data.get("source_digest") != kernel_source_digest():
        return None
    return data.get("kernels", {}).get(kernel)


def pmc_means(run_dir: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch for each kernel name in a rocprofv3 CSV run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def pmc_summary(fetch_dir: str, write_dir: str) -> None:
    """HBM traffic per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the counter reads for the reference copy of known size."""
    fetch, write = pmc_means(fetch_dir, "FETCH_SIZE"), pmc_means(write_dir, "WRITE_SIZE")

    def pick(d, key):
        hits = [v for k, v in d.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}")
        return sum(hits) / len(hits)

    meta = json.load(open(os.path.join(fetch_dir, "calib.json")))
    copy_bytes = meta["copy_bytes"]
    f_factor = pick(fetch, CALIB_KERNEL) * 1024 / copy_bytes
    w_factor = pick(write, CALIB_KERNEL) * 1024 / copy_bytes
    calls, raw = {}, {}
    for call, key in PMC_KERNELS.items():
        fk, wk = pick(fetch, key), pick(write, key)
        raw[call] = {"FETCH_SIZE_KiB": round(fk, 1), "WRITE_SIZE_KiB": round(wk, 1)}
        calls[call] = int(fk * 1024 / f_factor + wk * 1024 / w_factor)
    out = {"source_digest": kernel_source_digest(), "copy_bytes": copy_bytes,
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "calls": calls, "raw": raw, "algorithmic_bytes": meta.get("algorithmic_bytes")}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"reference copy: {copy_bytes} B read + written; FETCH_SIZE reads {f_factor:.3f} x the "
          f"bytes, WRITE_SIZE {w_factor:.3f} x\n")
    print("| call (kernel) | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | algorithmic bytes |")
    print("|---|---|---|---|---|")
    for call, key in PMC_KERNELS.items():
        alg = (meta.get("algorithmic_bytes") or {}).get(call)
        print(f"| {call} (`{key}`) | {raw[call]['FETCH_SIZE_KiB']} | {raw[call]['WRITE_SIZE_KiB']} | "
              f"{calls[call]} | {alg} |")


def prefill_score(torch, msa, synth, copies: int = 4, reps: int = 50) -> dict:
    """The prefill variant of the block score (4 rows x 2048 new tokens over an
    8192-token prefix, FP8 index, Di = 128), an MFMA-bound contraction, and the
    top-k over its [8192, 80] sheet, each timed alone like the decode calls."""
    c = synth.prefill()
    dev = "cuda"
    q_idx, bt, sl = c.q_idx.to(dev), c.block_table.to(dev), c.seq_lens.to(dev)
    idx0 = c.index_k.view(torch.float8_e4m3fn).to(dev)
    pools = [idx0] + [idx0.clone() for _ in range(copies - 1)]
    scores = [torch.full((c.N, c.MB), float("nan"), device=dev) for _ in range(copies)]
    topk = [torch.full((c.N, c.k), -1, dtype=torch.int32, device=dev) for _ in range(copies)]
    stream = torch.cuda.Stream()

    def graph(fn):
        with torch.cuda.stream(stream):
            for i in range(copies):
                fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(copies):
                fn(i)
        with torch.cuda.stream(stream):
            for _ in range(5):
                g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0 / (reps * copies)

    t_score = graph(lambda i: msa.msa_block_score(q_idx, pools[i], bt, sl, c.T, c.B, c.idx_scale,
                                                  scores[i]))
    t_sel = graph(lambda i: msa.msa_select_topk(scores[i], c.k, topk[i]))
    lens = c.seq_lens.numpy().astype(np.int64)
    # dot products over the visible keys: token t of a row sees L - (T - 1 - t) keys
    dots = int(sum(int(L) * c.T - c.T * (c.T - 1) // 2 for L in lens))
    flops = 2 * dots * c.Di
    tflops = flops / t_score / 1e12
    return {"workload": "prefill block score: 4 rows x 2048 new tokens over an 8192-token prefix "
                        "(seq_len 10240, 80 blocks), FP8 index, Di=128, top-k 16 over [8192, 80]",
            "score_us": round(t_score * 1e6, 3), "select_us": round(t_sel * 1e6, 3),
            "algorithmic_gflop": round(flops / 1e9, 3),
            "roofline": {"bound": "mfma", "kernel": "score_prefill_kernel<128, 4>", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def prefill_select_ragged(torch, msa, synth, copies: int = 4, reps: int = 50) -> dict:
    """msa_prefill_block_score on the ragged prefill batch (4 requests with
    2048/1536/1024/512 new tokens over 8192/4096/12288/2048 cached, 4 index
    heads, Di = 128, 64-token query blocks, top-16 with 1 initial and 2 local
    blocks): plan, scoring and selection launches, timed together on cold
    index-pool copies."""
    pb = synth.prefill_ragged()
    dev = "cuda"
    q = pb.q.to(dev)
    idx0 = pb.index_k.view(torch.float8_e4m3fn).to(dev)
    pools = [idx0] + [idx0.clone() for _ in range(copies - 1)]
    ints = {n: getattr(pb, n).to(dev) for n in ("block_table", "slot_ids", "cu_seqlens", "seq_lens",
                                               "prefix_lens", "cu_seqblocks_q")}
    out = [torch.full((pb.Hq, pb.all_qb, pb.topk), -1, dtype=torch.int32, device=dev)
           for _ in range(copies)]
    nbytes = msa.msa_prefill_block_score_workspace_bytes(pb.batch, pb.Hq, pb.all_qb, pb.MB,
                                                         pb.block_size_q)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def body():
        for i in range(copies):
            msa.msa_prefill_block_score(q, pools[i], ints["block_table"], ints["slot_ids"],
                                        ints["cu_seqlens"], ints["seq_lens"], ints["prefix_lens"],
                                        pb.block_size_q, pb.B, pb.topk, pb.init_blocks,
                                        pb.local_blocks, pb.scale, ints["cu_seqblocks_q"], out[i], ws)
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    with torch.cuda.stream(stream):
        for _ in range(5):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1000.0 / (reps * copies)
    # dot products: every (head, query-block token, visible key) triple
    cu = pb.cu_seqlens.numpy().astype(np.int64)
    dots = 0
    for b in range(pb.batch):
        nq = int(cu[b + 1] - cu[b])
        for qb in range(-(-nq // pb.block_size_q)):
            ntok = min(pb.block_size_q, nq - qb * pb.block_size_q)
            V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + qb * pb.block_size_q)
            dots += ntok * V
    flops = 2 * dots * pb.Di * pb.Hq
    tflops = flops / t / 1e12
    return {"workload": "ragged prefill score-to-selection: 4 requests, 2048/1536/1024/512 new tokens "
                        "over 8192/4096/12288/2048 cached, 4 heads, Di=128, 64-token query blocks, "
                        "top-16 (1 initial + 2 local blocks)",
            "call_us": round(t * 1e6, 3), "algorithmic_gflop": round(flops / 1e9, 3),
            "roofline": {"bound": "mfma", "kernel": "msa_prefill_block_score (plan + scoring + select)",
                         "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def bf16_kv_attention(torch, msa, case, topk, copies: int = 4, reps: int = 50) -> dict:
    """msa_sparse_decode over the same selection with the caches held as dense
    bf16 (attention.decode's commissioned cache; the FP8 values widened
    exactly), timed alone on cold pool copies like the decode calls."""
    dev = "cuda"
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    k0 = f8(case.k_cache).to(dev).to(torch.bfloat16)
    v0 = f8(case.v_cache).to(dev).to(torch.bfloat16)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    q, bt, sl = case.q.to(dev), case.block_table.to(dev), case.seq_lens.to(dev)
    tk = torch.from_numpy(topk).to(dev)
    out = torch.empty((case.N, case.Hq, case.D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(msa.msa_sparse_decode_workspace_bytes(case.R, case.T, case.Hq, case.Hkv, case.D,
                                                           case.k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def body():
        for kc, vc in pools:
            msa.msa_sparse_decode(q, kc, vc, bt, sl, tk, case.T, out, case.sm_scale, case.k_scale,
                                  case.v_scale, case.B, ws)
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    with torch.cuda.stream(stream):
        for _ in range(5):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1000.0 / (reps * copies)
    ab = algorithmic_bytes(case, topk)
    nbytes = ab["decode"] + ab["kv"]            # the K/V rows count twice at 2 bytes per element
    gbs = nbytes / t / 1e9
    return {"workload": "msa_sparse_decode, 16 rows x 4 tokens, 16384 ctx, top-k 16, dense bf16 K/V caches",
            "us": round(t * 1e6, 3), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "kernel": "attn_token_kernel<128, 1>", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def graph_seconds(torch, stream, body, calls: int, reps: int, warm: int = 5) -> float:
    """Seconds per call of `body` (which makes `calls` calls) captured into one
    HIP graph on `stream`, replayed `warm` times, then `reps` times between HIP
    events recorded on that stream."""
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1000.0 / (reps * calls)


def time_sparse_decode(torch, msa, case, pools, tk, out_dtype, copies: int, reps: int) -> float:
    """Seconds per msa_sparse_decode over `pools` [(k_cache, v_cache)] rotated in
    a graph (cold copies), selection tensor `tk` on the device."""
    dev = "cuda"
    q, bt, sl = case.q.to(dev), case.block_table.to(dev), case.seq_lens.to(dev)
    out = torch.empty((case.N, case.Hq, case.D), dtype=out_dtype, device=dev)
    ws = torch.zeros(msa.msa_sparse_decode_workspace_bytes(case.R, case.T, case.Hq, case.Hkv, case.D,
                                                           tk.shape[-1]), dtype=torch.uint8, device=dev)

    def body():
        for kc, vc in pools:
            msa.msa_sparse_decode(q, kc, vc, bt, sl, tk, case.T, out, case.sm_scale, case.k_scale,
                                  case.v_scale, case.B, ws)
    return graph_seconds(torch, torch.cuda.Stream(), body, len(pools), reps)


def time_step(torch, msa, case, copies: int = 8, reps: int = 25):
    """Seconds per msa_decode_step on `case` over `copies` cold pool copies in a
    graph, and the selection it made (host array)."""
    dev = "cuda"
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    k = case.k
    q_idx, q = case.q_idx.to(dev), case.q.to(dev)
    bt, sl = case.block_table.to(dev), case.seq_lens.to(dev)
    base = (f8(case.index_k).to(dev), f8(case.k_cache).to(dev), f8(case.v_cache).to(dev))
    pools = [base] + [tuple(x.clone() for x in base) for _ in range(copies - 1)]
    sc = torch.empty((case.N, case.MB), device=dev)
    tk = torch.empty((case.N, k), dtype=torch.int32, device=dev)
    out = torch.empty((case.N, case.Hq, case.D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(msa.msa_decode_step_workspace_bytes(case.R, case.T, case.Hq, case.Hkv, case.D, k),
                     dtype=torch.uint8, device=dev)

    def body():
        for idx, kc, vc in pools:
            msa.msa_decode_step(q_idx, idx, q, kc, vc, bt, sl, case.T, k, case.B, case.idx_scale,
                                case.sm_scale, case.k_scale, case.v_scale, sc, tk, out, ws)
    t = graph_seconds(torch, torch.cuda.Stream(), body, len(pools), reps)
    return t, tk.cpu().numpy()


def step_entry(case, t: float, tk) -> dict:
    ab = algorithmic_bytes(case, tk)
    gbs = ab["step"] / t / 1e9
    return {"us": round(t * 1e6, 3), "steps_per_s": round(1.0 / t, 1), "algorithmic_bytes": ab["step"],
            "achieved_hbm_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}


def topk_sweep(torch, msa, synth, ks=(8, 32, 128)) -> dict:
    """The whole step (msa_decode_step: score launch, then selection + attention
    + split merge) on the same workload at the other top-k sizes, 8, 32 and all
    128 blocks (attention over the whole context), each on its own seeded data
    and 8 cold pool copies."""
    res = {"workload": "msa_decode_step, 16 rows x 4 tokens, 16384 ctx, 16q/1kv heads, D=Di=128, FP8 "
                       "caches, top-k 8 / 32 / 128 (all blocks)"}
    for k in ks:
        case = synth.hbm_decode(k)
        res[f"k{k}"] = step_entry(case, *time_step(torch, msa, case))
    return res


def bucket_sweep(torch, msa, synth, rows=(1, 4, 8, 16)) -> dict:
    """The whole step at the decode buckets: R rows x 4 tokens with per-row
    context lengths uniform in [2048, 16384], top-k 16, 8 cold pool copies
    (small batches are bound by the launches' latency, not by HBM)."""
    res = {"workload": "msa_decode_step, R rows x 4 tokens, context uniform in [2048, 16384], 16q/1kv "
                       "heads, D=Di=128, FP8 caches, top-k 16"}
    for R in rows:
        case = synth.bucket_sweep(R)
        res[f"r{R}"] = step_entry(case, *time_step(torch, msa, case))
    return res


def kv_bytes(case, sel_rows) -> int:
    """K/V bytes of one KV head's selection: every visible token of the union of
    the selected blocks of each row, K and V, D bytes each (FP8)."""
    lens = case.seq_lens.numpy().astype(np.int64)
    tokens = 0
    for r in range(case.R):
        ids = np.unique(sel_rows[r])
        ids = ids[ids >= 0]
        tokens += int(sum(min(case.B, lens[r] - j * case.B) for j in ids if j * case.B < lens[r]))
    return tokens * case.D * 2


def per_request_selection(torch, msa, case, copies: int = 4, reps: int = 50) -> dict:
    """msa_sparse_decode with one selection per request ([R, k], shared by the
    request's 4 tokens), made on the device from the per-request score sheet
    (msa_block_score into [R, MB] + msa_select_topk), on cold pool copies."""
    dev = "cuda"
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    sheet = torch.empty((case.R, case.MB), device=dev)
    msa.msa_block_score(case.q_idx.to(dev), f8(case.index_k).to(dev), case.block_table.to(dev),
                        case.seq_lens.to(dev), case.T, case.B, case.idx_scale, sheet)
    tk = torch.empty((case.R, case.k), dtype=torch.int32, device=dev)
    msa.msa_select_topk(sheet, case.k, tk)
    k0, v0 = f8(case.k_cache).to(dev), f8(case.v_cache).to(dev)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    t = time_sparse_decode(torch, msa, case, pools, tk, torch.bfloat16, copies, reps)
    tkh = tk.cpu().numpy()
    nbytes = (kv_bytes(case, tkh) * case.Hkv + case.N * case.Hq * case.D * 2 * 2 + case.R * case.k * 4
              + case.R * case.MB * 4 + case.R * 4)
    gbs = nbytes / t / 1e9
    return {"workload": "msa_sparse_decode, 16 rows x 4 tokens, 16384 ctx, top-k 16, one selection per "
                        "request ([16, 16], from the per-request sheet)",
            "us": round(t * 1e6, 3), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "kernel": "attn_token_kernel<128, 2>", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def per_kv_head_selection(torch, msa, synth, case, copies: int = 4, reps: int = 50) -> dict:
    """msa_sparse_decode with 32 query / 2 KV heads and one selection per KV
    head ([2, 64, 16], random visible blocks), 16 rows x 4 tokens at 16384
    context, on cold pool copies.  The second KV head's pages are the bench
    pool's pages shifted by one page, and its 16 query heads the bench queries
    shifted by one token (built on the device)."""
    import dataclasses
    dev = "cuda"
    u8 = lambda t: t.view(torch.uint8).to(dev)
    two = lambda t: torch.stack([t[:, :, 0], t.roll(1, dims=0)[:, :, 0]], dim=2).view(torch.float8_e4m3fn)
    k0, v0 = two(u8(case.k_cache)), two(u8(case.v_cache))
    c2 = dataclasses.replace(case, name="hbm_hkv2", Hq=32, Hkv=2,
                             q=torch.cat([case.q, case.q.roll(1, dims=0)], dim=1))
    tkh = np.stack([synth.random_topk(c2, seed=5101 + g).numpy() for g in range(c2.Hkv)])
    tk = torch.from_numpy(tkh).to(dev)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    t = time_sparse_decode(torch, msa, c2, pools, tk, torch.bfloat16, copies, reps)
    rows = lambda g: [tkh[g][r * c2.T:(r + 1) * c2.T] for r in range(c2.R)]
    nbytes = (sum(kv_bytes(c2, rows(g)) for g in range(c2.Hkv)) + c2.N * c2.Hq * c2.D * 2 * 2
              + tkh.size * 4 + c2.R * c2.MB * 4 + c2.R * 4)
    gbs = nbytes / t / 1e9
    return {"workload": "msa_sparse_decode, 16 rows x 4 tokens, 16384 ctx, 32 q / 2 KV heads, top-k 16 "
                        "per KV head ([2, 64, 16], random visible blocks)",
            "us": round(t * 1e6, 3), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "kernel": "attn_token_kernel<128, 2>", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def _bench_lib():
    """libmsa_bench.so: the measurement kernels (built beside libmsa by build())."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_paged_amd", "libmsa_bench.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.msab_stream_read.restype = ctypes.c_int
    lib.msab_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.msab_empty.restype = ctypes.c_int
    lib.msab_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    return lib


def hbm_calibration(torch, step_bytes: int, reps: int = 20) -> dict:
    """What this GPU's HBM gives a plain streaming read (a hand-written kernel of
    non-temporal 16-byte loads, 8 in flight per lane): a 1 GiB read (steady state)
    and one launch reading the step's algorithmic bytes (ramp and tail included),
    on cold copies; and the cost of one launch boundary (graph-replayed empty
    launches)."""
    lib = _bench_lib()
    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    grid = 1024
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    res = {}

    def graph_time(body, calls, n_reps):
        with torch.cuda.stream(stream):
            body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            body()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(n_reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0 / (n_reps * calls)

    def read(bufs, nbytes):
        def body():
            for b in bufs:
                rc = lib.msab_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), grid, h)
                if rc != 0:
                    raise RuntimeError(f"stream read launch failed: {rc}")
        return body

    big = 1 << 30
    bufs = [torch.ones(big // 4, dtype=torch.float32, device="cuda") for _ in range(2)]
    t = graph_time(read(bufs, big), len(bufs), reps)
    res["read_1gib_gbs"] = round(big / t / 1e9, 1)
    del bufs
    n = (step_bytes + 4095) // 4096 * 4096
    bufs = [torch.ones(n // 4, dtype=torch.float32, device="cuda") for _ in range(8)]
    t = graph_time(read(bufs, n), len(bufs), reps)
    res["read_one_launch_step_bytes"] = {"bytes": n, "us": round(t * 1e6, 3), "gbs": round(n / t / 1e9, 1)}
    del bufs

    def empties():
        for _ in range(64):
            lib.msab_empty(256, h)
    res["launch_boundary_us"] = round(graph_time(empties, 64, 20) * 1e6, 3)
    res["note"] = ("hand-written streaming read (non-temporal 16-byte loads, 1024 workgroups of 256 "
                   "lanes, 8 loads in flight per lane) over cold buffers; launch_boundary_us: one "
                   "graph-replayed empty launch of 256 one-wave workgroups")
    return res


def host_cores() -> tuple[int, int, int]:
    """(threads the oracle runs on, cores in this process's affinity mask, the
    host's hardware concurrency).  Worker pools stay within 16 threads, the CPU
    share of one GPU of an 8-GPU host, whatever the host has."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    hw = os.cpu_count() or aff
    return min(16, aff), aff, hw


def oracle_step(case, threads: int) -> float:
    """Seconds of one full oracle step (score, select, attend) on `threads` threads."""
    import oracle
    t0 = time.perf_counter()
    s = oracle.block_score(case.q_idx, case.index_k, case.block_table, case.seq_lens, case.T,
                           case.idx_scale, threads=threads)
    tk = oracle.select_topk(s, case.k)
    oracle.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                         tk, case.T, case.sm_scale, case.k_scale, case.v_scale, threads=threads)
    return time.perf_counter() - t0


def cpu_baseline(case, small_case, min_wall: float = 1.0) -> dict:
    """The oracle's full step on the host cores: the bench workload (16 rows) and
    the 4-row decode bucket, each on every thread of the pool and on one thread.
    Whole steps are timed (the sample is the step itself, repeated for at least
    min_wall seconds on the pool)."""
    threads, aff, hw = host_cores()

    def rate(c, nthreads, wall):
        steps, spent = 0, 0.0
        while True:
            spent += oracle_step(c, nthreads)
            steps += 1
            if spent >= wall:
                return steps / spent, steps, spent
    v, n16, w16 = rate(case, threads, min_wall)
    v1, _, w1 = rate(case, 1, 0.0)
    s, ns, ws = rate(small_case, threads, min_wall / 2)
    s1, _, ws1 = rate(small_case, 1, 0.0)
    return {"value": round(v, 4), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "affinity_cores": aff, "hardware_concurrency": hw,
            "one_thread_steps_per_s": round(v1, 4),
            "decode_bucket4": {"workload": "4 rows x 4 tokens, 16384 ctx, top-k 16 (msa decode step)",
                               "steps_per_s": round(s, 4), "one_thread_steps_per_s": round(s1, 4)},
            "sample": f"whole steps of the same batches: {n16} of the 16-row batch on {threads} threads "
                      f"({w16:.2f} s), one on 1 thread ({w1:.2f} s); {ns} of the 4-row batch on {threads} "
                      f"threads ({ws:.2f} s), one on 1 thread ({ws1:.2f} s)",
            "note": f"{threads} threads: the pool stays within the 16-core CPU share of one GPU "
                    f"({aff} cores in the affinity mask, hardware concurrency {hw})"}


def prefill_cpu_baseline(synth, rows_per_request: int = 2) -> dict:
    """The oracle's ragged prefill score-to-selection on a bounded sample of the
    workload's rows (head 0, the first and the last query block of every
    request), extrapolated to the whole call by the count of dot products."""
    import oracle
    pb = synth.prefill_ragged()
    cu = pb.cu_seqblocks_q.numpy()
    cus = pb.cu_seqlens.numpy()
    rows = np.zeros((pb.Hq, pb.all_qb), dtype=bool)

    def dots(b, qb):
        nq = int(cus[b + 1] - cus[b])
        ntok = min(pb.block_size_q, nq - qb * pb.block_size_q)
        return ntok * min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + qb * pb.block_size_q)
    sample = total = 0
    for b in range(pb.batch):
        n = int(cu[b + 1] - cu[b])
        for qb in range(n):
            total += dots(b, qb) * pb.Hq
        for qb in sorted({0, n - 1})[:rows_per_request]:
            rows[0, cu[b] + qb] = True
            sample += dots(b, qb)
    t0 = time.perf_counter()
    oracle.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens, pb.seq_lens,
                          pb.prefix_lens, pb.block_size_q, pb.topk, pb.init_blocks, pb.local_blocks,
                          pb.scale, pb.cu_seqblocks_q, pb.all_qb, threads=1, rows=rows)
    dt = time.perf_counter() - t0
    per_call = dt * total / sample
    return {"value": round(1.0 / per_call, 6), "unit": "calls/s", "cores": 1, "kind": "oracle",
            "sample": f"{int(rows.sum())} of {pb.Hq * pb.all_qb} (head, query-block) rows (head 0, first and "
                      f"last query block of each request), {dt:.2f} s wall on one thread, scaled by "
                      f"dot products ({sample} of {total}) to {per_call:.1f} s per call"}


def main():
    a = parse()
    if a.ktrace_summary:
        ktrace_summary(*a.ktrace_summary)
        return
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the sharded path is described, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_paged_amd as msa
    import synth

    case = synth.hbm_decode(a.k)
    M, steps, warm_steps = plan_copies(a.steps, a.warmup, a.copies)
    reps, reps_w = steps // M, warm_steps // M
    dev = "cuda"
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    q_idx = case.q_idx.to(dev)
    q = case.q.to(dev)
    bt = case.block_table.to(dev)
    sl = case.seq_lens.to(dev)
    pools = []
    idx0, k0, v0 = f8(case.index_k).to(dev), f8(case.k_cache).to(dev), f8(case.v_cache).to(dev)
    for i in range(M):
        pools.append((idx0.clone(), k0.clone(), v0.clone()) if i else (idx0, k0, v0))
    scores = [torch.full((case.N, case.MB), float("nan"), device=dev) for _ in range(M)]
    topk = [torch.full((case.N, case.k), -1, dtype=torch.int32, device=dev) for _ in range(M)]
    out = [torch.full((case.N, case.Hq, case.D), float("nan"), dtype=torch.bfloat16, device=dev)
           for _ in range(M)]
    wsb = msa.msa_decode_step_workspace_bytes(case.R, case.T, case.Hq, case.Hkv, case.D, case.k)
    ws = [torch.zeros(wsb, dtype=torch.uint8, device=dev) for _ in range(M)]   # zero-filled once

    def call(name, i):
        idx, kc, vc = pools[i]
        if name == "step":
            msa.msa_decode_step(q_idx, idx, q, kc, vc, bt, sl, case.T, case.k, case.B,
                                case.idx_scale, case.sm_scale, case.k_scale, case.v_scale,
                                scores[i], topk[i], out[i], ws[i])
        elif name == "score":
            msa.msa_block_score(q_idx, idx, bt, sl, case.T, case.B, case.idx_scale, scores[i])
        elif name == "select":
            msa.msa_select_topk(scores[i], case.k, topk[i])
        elif name == "select_decode":
            msa.msa_select_sparse_decode(scores[i], case.k, topk[i], q, kc, vc, bt, sl, case.T,
                                         out[i], case.sm_scale, case.k_scale, case.v_scale,
                                         case.B, ws[i])
        else:
            msa.msa_sparse_decode(q, kc, vc, bt, sl, topk[i], case.T, out[i], case.sm_scale,
                                  case.k_scale, case.v_scale, case.B, ws[i])

    stream = torch.cuda.Stream()
    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib << 18                      # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def capture(names):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(M):
                for name in names:
                    call(name, i)
        return g

    def timed(g, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(n):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0   # seconds

    # W warmup steps (reps_w replays of the M-step graph), then exactly `steps`
    # timed steps (reps replays) between HIP events on the kernels' stream
    step_graph = capture(("step",))
    with torch.cuda.stream(stream):
        for _ in range(reps_w):
            step_graph.replay()
    torch.cuda.synchronize()
    t_step = timed(step_graph, reps) / steps
    # the same graph over at least 400 steps, for a figure less exposed to noise
    long_reps = max(reps, -(-400 // M))
    t_long = timed(step_graph, long_reps) / (long_reps * M)

    # the same M steps all on pool copy 0: its 62 MB stay in the 256 MB Infinity
    # Cache, so this is a warm (cache-resident) figure, not an HBM one
    def capture_warm():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(M):
                call("step", 0)
        return g
    warm_graph = capture_warm()
    with torch.cuda.stream(stream):
        warm_graph.replay()
    t_warm = timed(warm_graph, long_reps) / (long_reps * M)
    del warm_graph

    # each call on its own, timed over as many replays as the long step figure
    per_call = {}
    names = [n for n in a.kernels.split(",") if n]
    if "select_decode" not in names:          # the roofline launch is always timed
        names.append("select_decode")
    for name in names:
        g = capture(("score", "select", "decode") if name == "calls" else (name,))
        with torch.cuda.stream(stream):
            g.replay()
        per_call[name] = timed(g, long_reps) / (long_reps * M)
        del g

    tk_host = topk[0].cpu().numpy()
    ab = algorithmic_bytes(case, tk_host)
    eff_gbs = ab["step"] / t_step / 1e9
    # dominant launch: the step's attention launch, timed on its own
    dom = "select_decode"
    t_dom = per_call.get(dom)
    dom_gbs = ab[dom] / t_dom / 1e9 if t_dom else None
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            if tj.get("source_digest") == kernel_source_digest() and dom in tj.get("calls", {}):
                traffic = tj["calls"][dom]
        except Exception:
            traffic = None
    prof_us = rocprof_duration_us(ROOFLINE_KERNEL)

    res = {
        "metric": "sparse decode steps/s + achieved HBM GB/s (% of peak), 16 rows x 16K ctx",
        "value": round(1.0 / t_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm_steps,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-in/bf16-mfma/fp32-acc",
        "data": "synthetic (seeded N(0,1), per-tensor E4M3 quantised, random page tables)",
        "config": {"workload": "msa sparse decode step, 16 rows x 4 tokens, 16384 ctx, "
                               "16q/1kv heads, D=Di=128, FP8 caches, top-k 16",
                   "rows": case.R, "tokens_per_row": case.T, "context": int(case.seq_lens[0]),
                   "top_k": case.k, "pool_pages": case.P, "pool_copies": M},
        "achieved_hbm_gbs": round(eff_gbs, 1),
        "pct_of_hbm_peak": round(100.0 * eff_gbs / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_step": ab["step"],
        "long_run": {"steps": long_reps * M, "us_per_step": round(t_long * 1e6, 3),
                     "steps_per_s": round(1.0 / t_long, 1),
                     "pct_of_hbm_peak": round(100.0 * ab["step"] / t_long / 1e9 / HBM_PEAK_GBS, 2)},
        "per_call_us": {k: round(v * 1e6, 3) for k, v in per_call.items()},
        "warm_cache_resident": {"us_per_step": round(t_warm * 1e6, 3), "steps_per_s": round(1.0 / t_warm, 1),
                                "note": "one pool copy replayed: the step's bytes stay in the Infinity "
                                        "Cache; not an HBM figure"},
        "roofline": {"bound": "hbm", "kernel": ROOFLINE_KERNEL, "achieved": round(dom_gbs, 1) if dom_gbs else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4) if dom_gbs else None, "traffic": traffic,
                     "algorithmic_bytes": ab[dom],
                     "duration_us": round(t_dom * 1e6, 3) if t_dom else None,
                     "duration_note": "HIP events over graph-replayed launches: kernel time plus the "
                                      "launch boundary",
                     "rocprof_duration_us": prof_us,
                     "rocprof_frac": (round(ab[dom] / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if prof_us else None)},
    }
    res["hbm_calibration"] = hbm_calibration(torch, step_bytes=ab["step"])
    if not a.no_prefill:
        res["prefill_score"] = prefill_score(torch, msa, synth)
        res["prefill_select_ragged"] = prefill_select_ragged(torch, msa, synth)
        if not a.no_cpu_baseline:
            res["prefill_select_ragged"]["cpu_baseline"] = prefill_cpu_baseline(synth)
    if not a.no_variants:
        del pools, scores, out, ws
        res["bf16_kv_attention"] = bf16_kv_attention(torch, msa, case, tk_host)
        res["per_request_selection"] = per_request_selection(torch, msa, case)
        res["per_kv_head_selection"] = per_kv_head_selection(torch, msa, synth, case)
        res["topk_sweep"] = topk_sweep(torch, msa, synth)
        res["bucket_sweep"] = bucket_sweep(torch, msa, synth)
    if a.calib_copy_mib > 0:
        # the reference copy's size and the calls' algorithmic bytes, for --pmc-summary
        os.makedirs(a.calib_out, exist_ok=True)
        with open(os.path.join(a.calib_out, "calib.json"), "w") as fh:
            json.dump({"copy_bytes": a.calib_copy_mib << 20,
                       "algorithmic_bytes": {c: ab[c] for c in PMC_KERNELS}}, fh)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, synth.decode_bucket4())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
