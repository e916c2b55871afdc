"""Throughput of the TriAttention pruning path on one MI355X.

One step = tri_score + tri_select_compact over the whole batch of the
long-reasoning compression workload (28 layers, 4 KV heads, 28 query heads,
head_dim 128, batch 8, 32768 keys per head pruned to 2048, K and V bf16),
inputs resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
  python bench.py --workload {smallest,decode_window,ragged,stress_ties}
                                        # other workloads; those that fit in the
                                        # Infinity Cache are also timed cold
  python bench.py --offsets linear --reduce max   # offset-set variant (tri_score_offsets)
  python bench.py --compare-reductions  # kept-set overlap of the mean and max readings
  python bench.py --copy-probe          # 1 GiB device copy, for counter scaling
  python bench.py --stream-probe        # 4 GiB streaming read: the practical read ceiling
  python bench.py --summarize DIR --out FILE --cmd "..."   # rocprofv3 CSV -> text
  python bench.py --traffic DIR --out FILE   # counter runs (DIR/fetch, write, copy_fetch,
                                             # copy_write) -> HBM bytes per tri_score call
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "keys scored+compacted/sec and achieved HBM GB/s (% of peak), 1 MI355X"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
COPY_PROBE_BYTES = 1 << 30
STREAM_PROBE_BYTES = 4 << 30  # well past the 256 MB Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_tri_score_long_reasoning_32k_to_2048.json")
# The fused score kernel, its preparation kernel and launch shape
# (score_mfma.hip), the prologue of the other paths (calib.hip) and the
# shared device helpers (tri_internal.hpp): the kernels one tri_score call
# runs on the 32K->2048 workload.
KERNEL_SOURCES = ["score_mfma.hip", "calib.hip", "tri_internal.hpp"]


def kernel_source_hash():
    """Hash of the sources that define the tri_score kernels: counter
    readings taken on other sources do not describe this build."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rope_aware_key_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per tri_score call from the committed counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_call")


def device_copy_gbps(reps=10):
    """Read+write rate of a plain 1 GiB device-to-device copy on the current
    stream (HIP events), the practical ceiling of a gather."""
    import torch
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * COPY_PROBE_BYTES / t / 1e9


def stream_probe_gbps(reps=10):
    """Rate of a plain streaming read (tri_stream_probe: 16-byte
    non-temporal loads over every CU) of STREAM_PROBE_BYTES, timed with HIP
    events on the stream it runs on: the practical ceiling of the score
    kernel's K stream."""
    import torch
    import rope_aware_key_amd as R
    a = torch.empty(STREAM_PROBE_BYTES, dtype=torch.uint8, device="cuda:0")
    a.fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    R.tri_stream_probe(a, sink, stream=st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        R.tri_stream_probe(a, sink, stream=st)
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del a
    torch.cuda.empty_cache()
    return STREAM_PROBE_BYTES / t / 1e9


def copy_probe(reps=10):
    """A plain device copy of COPY_PROBE_BYTES, for scaling FETCH_SIZE and
    WRITE_SIZE (each copy reads and writes exactly that many bytes)."""
    import torch
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "reps": reps}))


def summarize(prof_dir, out, cmd):
    """Turn a rocprofv3 --stats / --pmc CSV directory into a short text summary."""
    import csv
    lines = [f"# rocprofv3 summary: {os.path.basename(out)}", "", f"command: `{cmd}`", "",
             f"kernel_source_hash: `{kernel_source_hash()}` (score_mfma.hip, calib.hip, "
             f"tri_internal.hpp as built for this run)", ""]
    for path in sorted(glob.glob(os.path.join(prof_dir, "**", "*kernel_stats.csv"), recursive=True)):
        lines += ["kernel stats (durations in microseconds):", "",
                  "| kernel | calls | avg | min | max |", "|---|---|---|---|---|"]
        rows = list(csv.DictReader(open(path)))
        ours = any(r["Name"].replace("void ", "").startswith("tri::") for r in rows)
        for r in rows:
            name = r["Name"].split("(")[0].replace("void ", "")
            if ours and not name.startswith("tri::"):
                continue
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        lines.append("")
    for path in sorted(glob.glob(os.path.join(prof_dir, "**", "*counter_collection.csv"), recursive=True)):
        per = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"].split("(")[0].replace("void ", ""), r["Counter_Name"])
            per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        lines += ["counters (mean per dispatch over the dispatches seen):", "",
                  "| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
        ours = any(kn.startswith("tri::") for kn, _ in per)
        for (kname, cname), d in sorted(per.items()):
            if ours and not kname.startswith("tri::"):
                continue
            vals = list(d.values())
            lines.append(f"| {kname[:60]} | {cname} | {len(vals)} | {sum(vals) / len(vals):.6g} |")
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)

TRAFFIC_RUNS = {
    # subdirectory of --traffic: (counter, command that fills it; OUT = that subdirectory)
    "fetch": ("FETCH_SIZE", "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- "
                            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline"),
    "write": ("WRITE_SIZE", "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o run -- "
                            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline"),
    "copy_fetch": ("FETCH_SIZE", "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- "
                                 "python3 bench.py --copy-probe"),
    "copy_write": ("WRITE_SIZE", "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o run -- "
                                 "python3 bench.py --copy-probe"),
    "probe_fetch": ("FETCH_SIZE", "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- "
                                  "python3 bench.py --stream-probe"),
}
# kernels of one tri_score call on the 32K->2048 workload (its plan travels
# in the preparation kernel's arguments)
SCORE_KERNELS = ("tri::prep_fused_kernel", "tri::score_fused_kernel")
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_long_reasoning_32k_to_2048.md")


def trace_avg_us(kernel_prefix):
    """Average duration (us) of a kernel in the committed rocprofv3 trace of
    the 32K->2048 bench run, if that trace was taken on the current kernel
    sources; else None."""
    try:
        text = open(TRACE_FILE).read()
    except OSError:
        return None
    if f"kernel_source_hash: `{kernel_source_hash()}`" not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[0].startswith(kernel_prefix):
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def counter_means(run_dir, counter):
    """Mean per dispatch (KiB) of one counter, per kernel name, over a run."""
    import csv
    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            d = per.setdefault(name, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def write_traffic(run_root, out):
    """HBM bytes per tri_score call from the counter runs of TRAFFIC_RUNS
    under run_root.  FETCH_SIZE is scaled by what it reads for the stream
    probe, which reads exactly STREAM_PROBE_BYTES per dispatch with the
    score kernel's load pattern (16-byte non-temporal loads covering whole
    128-byte lines); WRITE_SIZE by what it reads for the copy probe, which
    writes exactly COPY_PROBE_BYTES per dispatch.  The copy probe's fetch
    factor is kept beside it as a cross-check."""
    means = {sub: counter_means(os.path.join(run_root, sub), c) for sub, (c, _) in TRAFFIC_RUNS.items()}
    true_kib = COPY_PROBE_BYTES / 1024.0
    # the probes' own kernels are the dispatches with the largest reading
    copy_fetch_scale = true_kib / max(means["copy_fetch"].values())
    fetch_scale = (STREAM_PROBE_BYTES / 1024.0) / max(means["probe_fetch"].values())
    write_scale = true_kib / max(means["copy_write"].values())
    raw = {}
    fetch = write = 0.0
    for name in set(means["fetch"]) | set(means["write"]):
        if name.startswith(SCORE_KERNELS):
            f, w = means["fetch"].get(name, 0.0), means["write"].get(name, 0.0)
            raw[name] = {"FETCH_SIZE": f, "WRITE_SIZE": w}
            fetch += f * 1024.0 * fetch_scale
            write += w * 1024.0 * write_scale
    cfg = synth_config_bytes("long_reasoning")
    t = {
        "what": "HBM bytes per tri_score call on the 32K->2048 long-reasoning workload (28 layers, "
                "4 KV heads, 28 q heads, d 128, batch 8): preparation kernel + fused score kernel",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_scale": fetch_scale,
        "fetch_scale_from": "stream probe (read-only, the score kernel's load pattern)",
        "copy_fetch_scale": copy_fetch_scale,
        "write_scale": write_scale,
        "stream_probe_kib": {"FETCH_SIZE": max(means["probe_fetch"].values()),
                             "true": STREAM_PROBE_BYTES / 1024.0},
        "copy_probe_kib": {"FETCH_SIZE": max(means["copy_fetch"].values()),
                           "WRITE_SIZE": max(means["copy_write"].values()), "true_each": true_kib},
        "raw_kib_per_dispatch": raw,
        "fetch_bytes_per_call": fetch,
        "write_bytes_per_call": write,
        "bytes_per_call": fetch + write,
        "algorithmic_bytes_per_call": cfg,
        "ratio_to_algorithmic": (fetch + write) / cfg,
        "commands": [cmd for _, cmd in TRAFFIC_RUNS.values()],
    }
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
    print(out)


def synth_config_bytes(name):
    """Algorithmic tri_score bytes of a fixed-length workload, from its sizes
    alone (no tensors): units * n * (d*2 + 4)."""
    sizes = {"long_reasoning": dict(S=8, L=28, Hkv=4, n=32768, d=128)}[name]
    return sizes["S"] * sizes["L"] * sizes["Hkv"] * sizes["n"] * (sizes["d"] * 2 + 4)


WORKLOADS = {
    # name: (overrides, label)
    "long_reasoning": ({}, "long_reasoning_32k_to_2048"),
    "smallest": ({}, "smallest_4096_to_512"),
    "decode_window": ({}, "decode_window_3200_to_3072"),
    "ragged": ({}, "ragged_256seq_one_layer"),
    "stress_ties": ({}, "stress_ties_131072_to_4096"),
}


INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level cache

OFFSET_SETS = {
    "default": [2.0 ** j for j in range(17)],           # {2^0..2^16}
    "linear": [float(x) for x in range(1, 129, 8)],     # 16 offsets, spacing 8
    "short": [2.0 ** j for j in range(9)],              # {2^0..2^8}
}


def max_mode_flops(case, n_offsets):
    """Per-key MFMA work of the max-over-offsets kernel: the method's dot
    products (2*G*|D|*d flops, fp32-equivalent) and the bf16 MFMA flops the
    kernel issues for them.  Issued work follows the library's plan: per 16
    keys and pass, tiles*d/32*2 trig MFMAs (two bf16 terms per
    coefficient) and d/32*3 norm MFMAs, 16*16*32*2 flops each; tiles hold the
    (head, offset) rows with each head's rows rounded up to 4 (one lane
    slot) or, when one head exceeds the LDS budget, to 16 (all four).  The
    LDS budget holds the norm operands (three terms per step) and the tiles."""
    G, d = case.shape.group, case.shape.head_dim
    steps = d // 32
    max_tiles = (160 * 1024 - steps * 3 * 64 * 16) // (steps * 2 * 64 * 16)
    tph = (n_offsets + 3) // 4
    if tph <= max_tiles:
        hp_max = min(G, 4 * (max_tiles // tph))
        npass = -(-G // hp_max)
        hp = -(-G // npass)
        tiles = -(-hp // 4) * tph
    else:
        tph = (n_offsets + 15) // 16
        hp_max = min(G, max_tiles // tph)
        npass = -(-G // hp_max)
        hp = -(-G // npass)
        tiles = hp * tph
    mfma_per_16_keys = npass * (tiles * steps * 2 + steps * 3)
    return 2 * G * n_offsets * d, mfma_per_16_keys * 16 * 16 * 32 * 2 // 16


def algorithmic_bytes(case, budgets=None):
    """Bytes the method must move (no design intermediates):
    score:   n*d*2 (K read) + n*4 (score write)
    select:  n*4 (score read) + b*4 (index write)
    compact: 2*b*d*2 (K, V rows read) + 2*b*d*2 (rows written) + 2*b*4 (positions).
    budgets: optional [S][L] per-layer budgets (else the sequence's budget)."""
    d = case.shape.head_dim
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    score = sel = 0
    keys = 0
    for s in range(case.num_seqs):
        n = case.seq_len(s)
        for l in range(L):
            b = case.kept(s) if budgets is None else max(0, min(int(budgets[s][l]), n))
            keys += H * n
            score += H * (n * d * 2 + n * 4)
            sel += H * (n * 4 + b * 4 + 4 * b * d * 2 + 2 * b * 4)
    return keys, score, sel


def _oracle_unit_job(job):
    """One unit through the oracle as it stands (fp64 score, z-score, max,
    top-B, gather), on one thread; runs in a worker process of cpu_baseline.
    Returns (keys, seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    (kbits, vrows, pos, p_q, centre, absmean, Rr, d, theta, budget, reduce, layout, factored,
     offsets) = job
    om = O.rope_omega(d, theta)
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        score = O.unit_scores(O.bf16_bits_to_f64(kbits), pos, p_q, centre, absmean, Rr, om,
                              reduce=reduce, layout=layout, factored=factored,
                              **({} if offsets is None else {"offsets": offsets}))[0]
        kept = O.select_topb(score.astype(np.float32), budget)
        O.compact_rows(kbits, kept)
        O.compact_rows(vrows, kept)
        O.compact_rows(pos, kept)
    return kbits.shape[0], time.perf_counter() - t0


def oracle_workers():
    """Worker processes for the oracle baseline: the host cores this process
    may run on, at most 16 (one GPU's CPU share on a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(case, max_seconds=30.0, offsets=None, reduce="mean", layout="interleaved",
                 factored=False):
    """The oracle as it stands (fp64) on whole units of the same workload, in
    (sequence, layer, KV head) order, one unit per worker process at a time
    over oracle_workers() processes (one thread each), with the same offset
    set and reduction as the GPU line, until max_seconds of wall time.
    Returns the aggregate keys/s over that wall time and the time the whole
    workload would take at that rate.  factored=False: the term-by-term
    definition (the baseline); factored=True: the oracle's factored form of
    the same score (one dot product per head), the faster CPU reference."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    G = case.shape.group
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    order = [(s, l, g) for s in range(case.num_seqs) for l in range(L) for g in range(H)]
    nw = oracle_workers()

    def job(s, l, g):
        start, n = case.unit_rows(s, l, g)
        hs = slice(g * G, (g + 1) * G)
        qc = case.q_centre[l, hs].cpu().double().numpy()
        return (case.k[start:start + n].cpu().numpy().view(np.uint16),
                case.v[start:start + n].cpu().numpy(),
                case.k_pos[start:start + n].cpu().numpy().astype(np.float64),
                float(case.cur_pos[s]), qc[..., 0] + 1j * qc[..., 1],
                case.q_absmean[l, hs].cpu().double().numpy(),
                case.q_R[l, hs].cpu().double().numpy(), case.shape.head_dim,
                case.shape.rope_theta, int(case.budget[s]), reduce, layout, factored,
                None if offsets is None else np.asarray(offsets, np.float64))

    keys = units = 0
    nxt = 0
    with cf.ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn")) as ex:
        ex.submit(time.sleep, 0).result()    # workers up before the clock starts
        t0 = time.perf_counter()
        pending = set()
        while nxt < len(order) and len(pending) < 2 * nw:
            pending.add(ex.submit(_oracle_unit_job, job(*order[nxt])))
            nxt += 1
        while pending:
            done, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for f in done:
                k, _ = f.result()
                keys += k
                units += 1
            if time.perf_counter() - t0 < max_seconds:
                while nxt < len(order) and len(pending) < 2 * nw:
                    pending.add(ex.submit(_oracle_unit_job, job(*order[nxt])))
                    nxt += 1
            elif pending:
                # past the budget: count only what is already running, drop the rest
                for f in pending:
                    f.cancel()
                pending = {f for f in pending if not f.cancelled()}
        dt = time.perf_counter() - t0
    rate = keys / dt
    total_keys = case.total_rows()
    how = ("factored fp64 score (one dot product per head)" if factored
           else "term-by-term fp64 score")
    return {"value": rate, "unit": "keys/s", "cores": nw,
            "kind": "oracle (factored)" if factored else "oracle",
            "extrapolated_s": total_keys / rate,
            "sample": f"{units} whole unit(s) in (sequence, layer, KV head) order on {nw} worker "
                      f"processes, one thread each ({len(os.sched_getaffinity(0))} host cores "
                      f"visible), G={G}: {how} ({reduce} over "
                      f"{len(offsets) if offsets is not None else 17} offsets), z-score, max, "
                      f"top-B, gather; {dt:.1f} s wall; extrapolated_s = the whole workload "
                      f"({total_keys} keys) at this rate"}


def decode_cpu_baseline(case, tokens_k, tokens_v, B, interval, sink, recent, max_seconds=30.0):
    """The oracle's decode loop (term by term, one host thread) on whole units
    of the same run: each unit starts from its pruned prompt and takes
    `interval` appends, the last of which prunes.  Returns ms of host time
    per generated token for the whole batch (per-unit time x units)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    sh = case.shape
    LH, G = sh.num_layers * sh.num_kv_heads, sh.group
    om = O.rope_omega(sh.head_dim, sh.rope_theta)
    done, t_sum = 0, 0.0
    with threadpool_limits(limits=1):
        for g in range(sh.num_kv_heads):
            start, n = case.unit_rows(0, 0, g)
            qc = case.q_centre[0, g * G:(g + 1) * G].cpu().double().numpy()
            stats = (qc[..., 0] + 1j * qc[..., 1],
                     case.q_absmean[0, g * G:(g + 1) * G].cpu().double().numpy(),
                     case.q_R[0, g * G:(g + 1) * G].cpu().double().numpy())
            u = O.DecodeUnit(case.k[start:start + n].cpu().numpy().view(np.uint16),
                             case.v[start:start + n].cpu().numpy().view(np.uint16),
                             case.k_pos[start:start + n].cpu().numpy())
            sc = u.scores(*stats, om, p_q=int(case.cur_pos[0]))
            u.prune(O.select_protected(sc, B, sink, recent))
            p = int(case.cur_pos[0])
            t0 = time.perf_counter()
            for t in range(interval):
                O.decode_step(u, tokens_k[t, g].cpu().numpy().view(np.uint16),
                              tokens_v[t, g].cpu().numpy().view(np.uint16), p + t, B, interval,
                              sink, recent, lambda unit: unit.scores(*stats, om))
            t_sum += time.perf_counter() - t0
            done += 1
            if t_sum > max_seconds:
                break
    per_unit_token = t_sum / done / interval
    units = case.num_units
    return {"value": per_unit_token * units * 1e3, "unit": "ms/token", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} unit(s) (sequence 0, layer 0, KV heads 0..{done - 1}), each "
                      f"after its prompt prune: {interval} appends and the prune they trigger, "
                      f"term-by-term fp64; per-unit time x {units} units; {t_sum:.1f} s"}


def run_decode(args):
    """Decode-loop driver at the decode-window shape: 64 sequences, 32 layers,
    8 KV heads, G = 4, d = 128; prompts of 3200 keys pruned to 3072 at
    prefill, then one token per sequence per step, a prune every 128."""
    import numpy as np
    import torch

    import rope_aware_key_amd as R
    import synth

    B, interval, sink, recent = 3072, 128, 4, 64
    steps = args.steps if args.steps_given else 256
    warm = args.warmup if args.warmup_given else 0
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print("[bench] building the decode-window prompts", file=sys.stderr, flush=True)
    case = synth.workload_case("decode_window", device=dev)
    sh = case.shape
    S, LH, d = case.num_seqs, sh.num_layers * sh.num_kv_heads, sh.head_dim
    T = warm + steps
    pos_tok = [torch.arange(T, device=dev, dtype=torch.int64) + int(case.cur_pos[s])
               for s in range(S)]
    tok = synth.build_case("decode_tokens", sh, [T] * S, [1] * S, device=dev, seed=0,
                           positions=pos_tok)
    # [T][S*LH][d]: token t of unit (s, l, g)
    idx = (torch.arange(S * LH, device=dev)[None, :] * T + torch.arange(T, device=dev)[:, None])
    tokens_k, tokens_v = tok.k[idx].contiguous(), tok.v[idx].contiguous()
    del tok
    dec = R.Decode(R.make_shape(d, sh.num_q_heads, sh.num_kv_heads, sh.num_layers, sh.rope_theta),
                   S, B, interval, case.q_centre, case.q_absmean, case.q_R,
                   protect_sink=sink, protect_recent=recent)
    stream = torch.cuda.current_stream()
    cu = torch.as_tensor(case.cu_len).pin_memory().numpy()
    cp = torch.as_tensor(case.cur_pos).pin_memory().numpy()
    dec.prefill(cu, cp, case.k, case.v, case.k_pos, stream=stream)
    pos_host = [torch.as_tensor(case.cur_pos.astype(np.int64) + t, dtype=torch.int32)
                .pin_memory().numpy() for t in range(T)]
    for t in range(warm):
        dec.append(tokens_k[t], tokens_v[t], pos_host[t], stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    prunes0 = dec.view()["prunes"]
    pruning = []
    t0 = time.perf_counter()
    for i in range(steps):
        before = dec.view()["len"][0]
        ev[i][0].record(stream)
        dec.append(tokens_k[warm + i], tokens_v[warm + i], pos_host[warm + i], stream=stream)
        ev[i][1].record(stream)
        pruning.append(dec.view()["len"][0] < before + 1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    pr = np.array(pruning)
    prunes = dec.view()["prunes"] - prunes0
    dec.close()
    total = float(ms.sum())
    prune_ms = float(ms[pr].mean()) if pr.any() else None
    append_ms = float(ms[~pr].mean()) if (~pr).any() else None
    units = S * LH
    # algorithmic bytes of one prune of every sequence: K read by the score,
    # scores written and read, K and V rows of the kept keys read and
    # written, positions read and written, indices written
    C = B + interval
    prune_bytes = units * (C * d * 2 + 2 * C * 4 + 4 * B * d * 2 + 2 * B * 4 + B * 4)
    out = {
        "metric": "decode-loop cache upkeep per generated token (append + amortised prune), 1 MI355X",
        "value": total / steps,
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": total / steps,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (decode-window prompts: steady-state positions; generated keys drawn "
                "at the following positions)",
        "config": {"workload": "decode_loop_3072_plus_128", "batch": S, "layers": sh.num_layers,
                   "kv_heads": sh.num_kv_heads, "q_heads": sh.num_q_heads, "head_dim": d,
                   "budget": B, "interval": interval, "protect_sink": sink,
                   "protect_recent": recent, "units": units},
        "wall_ms_per_step": wall / steps * 1e3,
        "breakdown_ms": {"append_step": append_ms, "pruning_step": prune_ms,
                         "prunes_in_timed_steps": int(prunes)},
        "roofline": {"bound": "hbm", "kernel": "pruning step (score + protect + select + gather)",
                     "achieved": prune_bytes / (prune_ms * 1e-3) / 1e9 if prune_ms else None,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": prune_bytes / (prune_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS
                     if prune_ms else None,
                     "traffic": None, "algorithmic_bytes_per_launch": prune_bytes},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle decode loop)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = decode_cpu_baseline(case, tokens_k[:, :LH], tokens_v[:, :LH], B,
                                                  interval, sink, recent)
    print(json.dumps(out), flush=True)


def run_compare_reductions(args):
    """How far the two offset readings disagree: the averaged score (the talk
    page's formula) against the maximum over offsets (the blog review's
    reading), each z-scored, maxed over the group and cut to the top B, on
    the long-reasoning synthetic cache.  Per unit: the fraction of the B
    kept keys the two readings share, for the pages' budgets."""
    import numpy as np
    import torch

    import rope_aware_key_amd as R
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    case = synth.workload_case("long_reasoning", device=dev)
    sh = R.make_shape(case.shape.head_dim, case.shape.num_q_heads, case.shape.num_kv_heads,
                      case.shape.num_layers, case.shape.rope_theta)
    cu = torch.as_tensor(case.cu_len).pin_memory().numpy()
    cp = torch.as_tensor(case.cur_pos).pin_memory().numpy()
    offs = torch.as_tensor(OFFSET_SETS["default"], dtype=torch.float64).pin_memory().numpy()
    rows, n = case.total_rows(), case.seq_len(0)
    units = case.num_units
    ws = torch.empty(max(R.tri_workspace_bytes(sh, cu),
                         R.tri_workspace_bytes_offsets(sh, cu, len(offs), "max")),
                     dtype=torch.uint8, device=dev)
    sc = {}
    for red in ("mean", "max"):
        sc[red] = torch.empty(rows, dtype=torch.float32, device=dev)
        R.tri_score_offsets(sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean,
                            case.q_R, offs, red, sc[red], workspace=ws)
    corr = []
    for u in range(units):
        a = sc["mean"][u * n:(u + 1) * n].double()
        b = sc["max"][u * n:(u + 1) * n].double()
        corr.append(float(torch.corrcoef(torch.stack([a, b]))[0, 1]))
    by_budget = {}
    for B in (512, 1024, 2048, 4096):
        bu = torch.full((case.num_seqs,), B, dtype=torch.int32).pin_memory().numpy()
        masks = {}
        for red in ("mean", "max"):
            kept = torch.empty(units * B, dtype=torch.int32, device=dev)
            R.tri_select_compact(sh, cu, bu, sc[red], None, None, None, kept, None, None, None,
                                 workspace=ws)
            m = torch.zeros(rows, dtype=torch.bool, device=dev)
            base = torch.arange(units, device=dev, dtype=torch.int64).repeat_interleave(B) * n
            m[base + kept.long()] = True
            masks[red] = m
        both = (masks["mean"] & masks["max"]).view(units, n).sum(dim=1).double() / B
        q = both.cpu().numpy()
        by_budget[str(B)] = {"mean": float(q.mean()), "min": float(q.min()),
                             "p10": float(np.percentile(q, 10)), "max": float(q.max())}
    torch.cuda.synchronize()
    corr = np.array(corr)
    out = {
        "metric": "kept-set overlap between the mean and the max over the 17 offsets",
        "value": by_budget["2048"]["mean"], "unit": "fraction of B shared (B = 2048)",
        "n_gpus": 1, "higher_is_better": True, "vs_baseline": None,
        "data": "synthetic (seeded concentrated bf16 K cache, synthesised query statistics)",
        "config": {"workload": "long_reasoning_32k_to_2048", "units": units,
                   "keys_per_head": n, "offsets": "2^0..2^16"},
        "overlap_by_budget": by_budget,
        "score_pearson_per_unit": {"mean": float(corr.mean()), "min": float(corr.min())},
    }
    print(json.dumps(out), flush=True)


def run_calib(args):
    """Calibration at scale and the reconstruction diagnostic at the
    long-reasoning model shape (28 layers, 28 query heads, 4 KV heads,
    d = 128): tri_calibrate on 10240 sample queries (the blog review's ~10K
    calibration tokens), tri_trig_correlation on 1024 of them against one
    sequence of 4096 keys per KV head, and a sweep of the synthetic query
    concentration R_Q with the per-head r and R distributions."""
    import numpy as np
    import torch

    import rope_aware_key_amd as R
    import synth
    from synth.cases import _calibration_queries

    dev = "cuda:0"
    torch.cuda.set_device(0)
    shape = synth.Shape(128, 28, 4, 28)
    L, Hq, Hkv, d = 28, 28, 4, 128
    N, n_q, n_k = 10240, 1024, 4096
    reps = args.steps if args.steps_given else 5
    sh = R.make_shape(d, Hq, Hkv, L, shape.rope_theta)
    stream = torch.cuda.current_stream()
    keys = synth.build_case("diag_keys", shape, (n_k,), (1,), device=dev, seed=7, with_values=False)
    qc = torch.empty(L, Hq, d // 2, 2, device=dev)
    qa = torch.empty(L, Hq, d // 2, device=dev)
    qr = torch.empty(L, Hq, d // 2, device=dev)
    ws = torch.empty(R.tri_trig_correlation_workspace_bytes(sh, n_q), dtype=torch.uint8, device=dev)
    r = torch.empty(L, Hq, dtype=torch.float64, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    sweep = []
    timing = None
    for R_Q in (0.99, 0.95, 0.9, 0.8, 0.6):
        print(f"[bench] R_Q = {R_Q}", file=sys.stderr, flush=True)
        q, q_pos = _calibration_queries(shape, N, dev, seed=3, R_Q=R_Q)
        qd = q[:, :n_q].contiguous()
        t_cal = timed(lambda: R.tri_calibrate(sh, q, q_pos, N, qc, qa, qr, stream=stream))
        t_diag = timed(lambda: R.tri_trig_correlation(sh, qd, q_pos, n_q, keys.k, keys.k_pos, n_k,
                                                      qc, r, workspace=ws, stream=stream))
        rr = r.cpu().numpy().ravel()
        head_R = qr.mean(dim=2).cpu().numpy().ravel()
        bins = [0.0, 0.5, 0.7, 0.8, 0.9, 0.95, 1.0001]
        sweep.append({"R_Q": R_Q, "r_mean": float(rr.mean()), "r_min": float(rr.min()),
                      "r_frac_above_0.7": float((rr > 0.7).mean()),
                      "head_R_mean": float(head_R.mean()),
                      "head_R_hist": {f"{bins[i]:.2f}-{min(bins[i + 1], 1.0):.2f}":
                                      int(((head_R >= bins[i]) & (head_R < bins[i + 1])).sum())
                                      for i in range(len(bins) - 1)}})
        if R_Q == 0.95:
            timing = (t_cal, t_diag)
        del q, qd
    t_cal, t_diag = timing
    q_bytes = L * N * Hq * d * 2
    pairs = L * Hq * n_q * n_k
    out = {
        "metric": "tri_calibrate sample queries per second (10240 queries, 28 layers x 28 heads)",
        "value": N / (t_cal * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 1,
        "ms_per_step": t_cal,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic post-RoPE queries concentrated at R_Q around per-(layer, head, band) "
                "centres; keys of the long-reasoning synthetic cache",
        "config": {"workload": "calibration_10240_queries_28x28_d128", "layers": L, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "samples": N},
        "roofline": {"bound": "hbm", "kernel": "calibrate_kernel", "achieved": q_bytes / (t_cal * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": q_bytes / (t_cal * 1e-3) / 1e9 / PEAK_HBM_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": q_bytes},
        "diagnostic": {"call": "tri_trig_correlation", "queries": n_q, "keys": n_k,
                       "ms": t_diag, "pairs_per_s": pairs / (t_diag * 1e-3),
                       "issued_bf16_tflops": pairs * d * 2 * 4 / (t_diag * 1e-3) / 1e12},
        "concentration_sweep": sweep,
    }
    print(json.dumps(out), flush=True)


def phase_profile(args, label, score, scores, stream):
    """tri_score calls with the phase-counting copy of the fused kernel
    (tri_debug_set_phase_buffer): cycles of wave 0 of a work-group per pass
    and phase, averaged over every pass of every work-group; the scores are
    checked bit for bit against a plain call."""
    import torch
    import rope_aware_key_amd as R
    plain = scores.clone()
    buf = torch.zeros(8, dtype=torch.int64, device=scores.device)
    R.tri_debug_set_phase_buffer(buf)
    try:
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            score()
        ev1.record(stream)
        torch.cuda.synchronize()
    finally:
        R.tri_debug_set_phase_buffer(None)
    same = bool(torch.equal(scores.view(torch.int32), plain.view(torch.int32)))
    c = buf.cpu().tolist()
    passes = c[7]
    cyc = {name: c[i] / passes for i, name in enumerate(R.PHASE_NAMES)}
    total = sum(cyc.values())
    print(json.dumps({"phase_profile": label, "calls": args.steps, "passes_per_call": passes / args.steps,
                      "cycles_per_pass": {k: round(v, 1) for k, v in cyc.items()},
                      "share": {k: round(v / total, 4) for k, v in cyc.items()},
                      "tri_score_ms_with_counters": ev0.elapsed_time(ev1) / args.steps,
                      "scores_bit_identical": same,
                      "clock": "s_memtime (core clock) on wave 0 of every work-group"}))
    if not same:
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--decode", action="store_true",
                    help="time the decode-loop driver at the decode-window shape")
    ap.add_argument("--calib", action="store_true",
                    help="calibration at scale and the reconstruction diagnostic")
    ap.add_argument("--compare-reductions", action="store_true",
                    help="kept-set overlap of the mean and the max over offsets")
    ap.add_argument("--workload", default="long_reasoning", choices=list(WORKLOADS))
    ap.add_argument("--offsets", default="default", choices=list(OFFSET_SETS))
    ap.add_argument("--reduce", default="mean", choices=["mean", "max"])
    ap.add_argument("--rope-layout", default="interleaved", choices=["interleaved", "half"],
                    help="store the keys half split (band f = x[f], x[f + d/2])")
    ap.add_argument("--paged", type=int, default=None, metavar="PAGE_SIZE",
                    help="K, V and positions in a paged pool (token-major pages of PAGE_SIZE "
                         "tokens, random page order); compaction into a second pool")
    ap.add_argument("--page-order", default="token", choices=["token", "head"],
                    help="token-major pages [page][slot][head] or head-major [page][head][slot]")
    ap.add_argument("--pyramid", type=float, default=None, metavar="RATIO",
                    help="per-layer pyramid budgets (last/first = RATIO, mean = the "
                         "sequence's budget), selected by tri_select_compact_layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--stream-probe", action="store_true",
                    help="time the read-bandwidth probe alone (4 GiB, 20 reads) and print its rate")
    ap.add_argument("--phase-profile", action="store_true",
                    help="cycles per phase of the fused score kernel's passes (tri_score only)")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--out", default=None)
    ap.add_argument("--cmd", default="")
    ap.add_argument("--traffic", default=None, metavar="DIR",
                    help="write the tri_score traffic JSON (--out) from the counter runs under DIR")
    args = ap.parse_args()
    args.steps_given, args.warmup_given = args.steps is not None, args.warmup is not None
    args.steps = 20 if args.steps is None else args.steps
    args.warmup = 3 if args.warmup is None else args.warmup
    if args.traffic:
        write_traffic(args.traffic, args.out)
        return
    if args.summarize:
        summarize(args.summarize, args.out, args.cmd)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.stream_probe:
        g = stream_probe_gbps(reps=20)
        print(json.dumps({"stream_probe_bytes": STREAM_PROBE_BYTES, "reps": 20,
                          "stream_probe_gbps": g, "frac_of_peak": g / PEAK_HBM_GBPS}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path shards over (sequence, layer, KV head) "
              "units with no exchange, so N GPUs run N independent copies of this step.",
              file=sys.stderr)
        sys.exit(2)

    if args.decode:
        run_decode(args)
        return
    if args.calib:
        run_calib(args)
        return
    if args.compare_reductions:
        run_compare_reductions(args)
        return

    import numpy as np
    import torch

    import rope_aware_key_amd as R
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    over, label = WORKLOADS[args.workload]
    print(f"[bench] building workload {label}", file=sys.stderr, flush=True)
    case = synth.workload_case(args.workload, device=dev, **over)
    if args.rope_layout == "half":
        # the same keys with their columns permuted to the half-split layout
        d = case.shape.head_dim
        perm = torch.as_tensor(np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)]),
                               device=dev)
        case.k = case.k[:, perm].contiguous()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        label = f"{label}+half_split_rope"
    sh = R.make_shape(case.shape.head_dim, case.shape.num_q_heads, case.shape.num_kv_heads,
                      case.shape.num_layers, case.shape.rope_theta, rope_layout=args.rope_layout)
    if case.calib_q is not None:
        # statistics from the workload's own calibration queries (not timed)
        if args.rope_layout == "half":
            print("--rope-layout half runs on workloads with synthesised statistics",
                  file=sys.stderr)
            sys.exit(2)
        R.tri_calibrate(sh, case.calib_q, case.calib_pos, case.calib_q.shape[1], case.q_centre,
                        case.q_absmean, case.q_R)
        torch.cuda.synchronize()
    rows, out_rows, d = case.total_rows(), case.total_out_rows(), case.shape.head_dim
    cu = torch.as_tensor(case.cu_len).pin_memory().numpy()
    cp = torch.as_tensor(case.cur_pos).pin_memory().numpy()
    bu = torch.as_tensor(case.budget).pin_memory().numpy()
    variant = args.offsets != "default" or args.reduce != "mean"
    budgets = None
    if args.pyramid is not None:
        L = case.shape.num_layers
        budgets = np.stack([R.tri_pyramid_budgets(L, float(b), args.pyramid)
                            for b in case.budget]).astype(np.int32)
        out_rows = int(sum(case.shape.num_kv_heads * min(int(budgets[s][l]), case.seq_len(s))
                           for s in range(case.num_seqs) for l in range(L)))
        bu = torch.as_tensor(budgets.reshape(-1)).pin_memory().numpy()
        label = f"{label}+pyramid_ratio_{args.pyramid:g}"
    offs = torch.as_tensor(OFFSET_SETS[args.offsets], dtype=torch.float64).pin_memory().numpy()
    if variant:
        label = f"{label}+{args.reduce}_over_{args.offsets}_offsets"
        wsb = R.tri_workspace_bytes_offsets(sh, cu, len(offs), args.reduce)
    else:
        wsb = R.tri_workspace_bytes(sh, cu)
    if budgets is not None:
        wsb = max(wsb, R.tri_workspace_bytes_layers(sh, cu))
    ws = torch.empty(max(1, wsb), dtype=torch.uint8, device=dev)
    pool = out_pool = None
    if args.paged is not None:
        if budgets is not None or variant:
            print("--paged runs with the default offsets and one budget per sequence",
                  file=sys.stderr)
            sys.exit(2)
        P = args.paged
        print(f"[bench] scattering the cache into {P}-token pages", file=sys.stderr, flush=True)
        hm = args.page_order == "head"
        pool = synth.paged_from_case(case, P, head_major=hm, seed=1)
        need = [(case.kept(s) + P - 1) // P for s in range(case.num_seqs)]
        out_pool = synth.empty_pool(case.num_seqs, case.shape.num_layers, case.shape.num_kv_heads,
                                    d, P, need, head_major=hm, spare=0, seed=2, device=dev)
        pg_in = R.make_pages(pool.table, P, pool.num_pages, *pool.strides())
        pg_out = R.make_pages(out_pool.table, P, out_pool.num_pages, *out_pool.strides())
        torch.cuda.synchronize()
        label = f"{label}+paged_{P}_{args.page_order}_major"
    scores = torch.empty(rows, dtype=torch.float32, device=dev)
    kept = torch.empty(max(1, out_rows), dtype=torch.int32, device=dev)
    k_out = torch.empty(max(1, out_rows), d, dtype=torch.int16, device=dev)
    v_out = torch.empty(max(1, out_rows), d, dtype=torch.int16, device=dev)
    pos_out = torch.empty(max(1, out_rows), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def score():
        if pool is not None:
            R.tri_score_paged(sh, cu, cp, pg_in, pool.k, case.q_centre, case.q_absmean, case.q_R,
                              scores, workspace=ws, stream=stream)
        elif variant:
            R.tri_score_offsets(sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean,
                                case.q_R, offs, args.reduce, scores, workspace=ws, stream=stream)
        else:
            R.tri_score(sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean, case.q_R,
                        scores, workspace=ws, stream=stream)

    def select():
        if pool is not None:
            R.tri_select_compact_paged(sh, cu, bu, scores, pg_in, pool.k, pool.v, pool.pos, kept,
                                       pg_out, out_pool.k, out_pool.v, out_pool.pos, workspace=ws,
                                       stream=stream)
        elif budgets is not None:
            R.tri_select_compact_layers(sh, cu, bu, scores, case.k, case.v, case.k_pos, kept,
                                        k_out, v_out, pos_out, workspace=ws, stream=stream)
        else:
            R.tri_select_compact(sh, cu, bu, scores, case.k, case.v, case.k_pos, kept, k_out,
                                 v_out, pos_out, workspace=ws, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        score()
        select()
    torch.cuda.synchronize()
    if args.phase_profile:
        phase_profile(args, label, score, scores, stream)
        return

    # The timed steps run back to back between one pair of events: an event
    # recorded between two kernels costs about 5 us of GPU time on this
    # chip (the queue drains and the caches write back before its
    # timestamp), which per-call events would add to every step.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        score()
        select()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: wall {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)
    # The split: as many calls of each kind, back to back, one event pair
    # around each run (a repeated call recomputes the same outputs).
    ea, eb, ec = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    ea.record(stream)
    for _ in range(args.steps):
        score()
    eb.record(stream)
    for _ in range(args.steps):
        select()
    ec.record(stream)
    torch.cuda.synchronize()
    t_score = np.array([ea.elapsed_time(eb) * 1e-3 / args.steps])
    t_sel = np.array([eb.elapsed_time(ec) * 1e-3 / args.steps])

    keys, b_score, b_sel = algorithmic_bytes(case, budgets)
    value = keys / step
    gbps = (b_score + b_sel) / step / 1e9
    score_gbps = b_score / float(t_score.mean()) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded concentrated bf16 K cache, N(0,1) V)",
        "config": {"workload": label, "batch": case.num_seqs, "layers": case.shape.num_layers,
                   "kv_heads": case.shape.num_kv_heads, "q_heads": case.shape.num_q_heads,
                   "head_dim": d, "keys_per_head": int(case.seq_len(0)),
                   "budget": int(case.budget[0]), "units": case.num_units},
        "hbm_gbps": gbps,
        "hbm_frac_of_peak": gbps / PEAK_HBM_GBPS,
        "wall_ms_per_step": wall / args.steps * 1e3,
        "breakdown_ms": {"tri_score": float(t_score.mean()) * 1e3,
                         ("tri_select_compact_layers" if budgets is not None
                          else "tri_select_compact"): float(t_sel.mean()) * 1e3},
        "select_hbm_gbps": b_sel / float(t_sel.mean()) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "tri_score",
                     "achieved": score_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": score_gbps / PEAK_HBM_GBPS,
                     "traffic": measured_traffic() if args.workload == "long_reasoning"
                     and not variant
                     and args.rope_layout == "interleaved" else None,
                     "algorithmic_bytes_per_launch": b_score,
                     "launch": "tri_score call: preparation kernel (plan, resets, operand "
                               "pack), fused score kernel",
                     "timing": "achieved: HIP events around as many back-to-back tri_score "
                               "calls as timed steps, right after them, on the stream the "
                               "kernels run on"},
    }
    if args.workload == "long_reasoning" and not variant and args.rope_layout == "interleaved":
        out["roofline"]["timing"] += ("; frac_trace: the fused kernel's average duration in the "
                                      "committed rocprofv3 trace of this build (profiles/), null "
                                      "if that trace is of other sources")
        t_us = trace_avg_us("tri::score_fused_kernel")
        out["roofline"]["trace_avg_us"] = t_us
        out["roofline"]["frac_trace"] = (b_score / (t_us * 1e-6) / 1e9 / PEAK_HBM_GBPS
                                         if t_us else None)
    copy_gbps = device_copy_gbps()
    out["device_copy_gbps"] = copy_gbps
    out["hbm_frac_of_device_copy"] = gbps / copy_gbps
    probe_gbps = stream_probe_gbps()
    out["stream_probe_gbps"] = probe_gbps
    out["roofline"]["frac_of_stream_probe"] = score_gbps / probe_gbps
    if b_score + b_sel < INFINITY_CACHE_BYTES:
        # The working set fits in the Infinity Cache, so the steps above run
        # warm.  Cold: a 1 GiB scratch write before each step (outside the
        # timed region, ahead of it on the same stream) evicts it.
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                 torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i, (e0, e1, e2) in enumerate(cold):
            scratch.fill_(i & 255)
            e0.record(stream)
            score()
            e1.record(stream)
            select()
            e2.record(stream)
        torch.cuda.synchronize()
        del scratch
        c_score = np.array([a.elapsed_time(b) for a, b, _ in cold])
        c_sel = np.array([b.elapsed_time(c) for _, b, c in cold])
        c_step = np.array([a.elapsed_time(c) for a, _, c in cold])
        out["cold_cache"] = {
            "flush": "1 GiB scratch write before each step, outside the timed region",
            "ms_per_step": float(c_step.mean()), "ms_per_step_median": float(np.median(c_step)),
            "keys_per_s": keys / (float(c_step.mean()) * 1e-3),
            "breakdown_ms": {"tri_score": float(c_score.mean()),
                             "tri_select_compact": float(c_sel.mean())}}
    if budgets is not None:
        out["config"]["budget"] = "pyramid"
        out["config"]["layer_budgets"] = [int(x) for x in budgets[0]]
    if variant:
        out["offsets"] = {"set": args.offsets, "values": OFFSET_SETS[args.offsets],
                          "reduce": args.reduce}
        out["roofline"]["kernel"] = "tri_score_offsets"
        out["roofline"]["launch"] = "tri_score_offsets call: " + (
            "prologue + operand pack + max-over-offsets MFMA kernel + z pass"
            if args.reduce == "max" else "preparation kernel + score kernels")
        if args.reduce == "max":
            # One row per (head, offset): a dense contraction on the bf16
            # MFMA.  `achieved` counts the method's dot products once
            # (2*G*|D|*d per key); the kernel issues more (three bf16 terms
            # per coefficient, padded rows, the norm term).
            f_alg, f_issued = max_mode_flops(case, len(offs))
            t = float(t_score.mean())
            alg, issued = keys * f_alg / t / 1e12, keys * f_issued / t / 1e12
            out["roofline"].update({
                "bound": "mfma", "achieved": alg, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": alg / PEAK_BF16_TFLOPS,
                "algorithmic_flops_per_launch": keys * f_alg,
                "issued_bf16_tflops": issued, "issued_frac": issued / PEAK_BF16_TFLOPS,
                "hbm_gbps": score_gbps})
            out["roofline"].pop("algorithmic_bytes_per_launch", None)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(case, offsets=OFFSET_SETS[args.offsets],
                                           reduce=args.reduce, layout=args.rope_layout)
        if not variant and budgets is None and pool is None:
            print("[bench] cpu factored baseline", file=sys.stderr, flush=True)
            out["cpu_factored_baseline"] = cpu_baseline(case, max_seconds=20.0,
                                                        layout=args.rope_layout, factored=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
