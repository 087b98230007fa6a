"""Benchmark: one decode step of the quantized KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: append one new token per sequence (which
flushes every full BF16 window first, then quantizes the token or copies it into the window), then
single-query decode attention
over every cached token with the K/V codes dequantized in registers.  Inputs are seeded synthetic
tensors generated on the GPU (kvq_inputs); the cache is resident in HBM before timing starts.

Default workload: the paged mixed batch (64 sequences, lengths log-uniform in [1024, 131072],
16-token blocks in shuffled physical order, H_q=32, H_kv=8, head_dim 128, INT4 symmetric group 64
with fp16 scales, 128-token BF16 window).  It is the largest single-GPU configuration and the only
one that exercises every step (flush, append, window, paged addressing, attention, combine).

Output: one JSON line (rank 0, N=1).  `value` is whole-step algorithmic bytes / step time in GB/s;
`roofline` prices the decode-attention call (its split-K kernel plus the combine kernel) against
MI355X's 8 TB/s; `cpu_baseline` times the CPU oracle's fp64 attention on a bounded sample of the
same sequences.  Before the W warmup steps, read-only attention calls over the prefilled cache
run untimed until their per-call time is stable (`settle_calls` in the line): a cold GPU takes
the first few dozen calls at up to twice the steady time.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5|c4|c3|c2x32|c2|c1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
HEAD_DIM = 128


# ------------------------------------------------------------------------------------------
# Algorithmic bytes
# ------------------------------------------------------------------------------------------

def side_token_bytes(side) -> float:
    """Bytes of one (token, kv head) row of one side: codes plus per-token metadata, or the
    per-token share of per-channel metadata."""
    bits, scheme, axis, group = side
    meta = 2 * (2 if scheme == 1 else 1)
    codes = HEAD_DIM * bits / 8
    if bits == 16 or scheme == 2:  # BF16 rows and FP8 (scales per head / tensor): no per-row metadata
        return codes
    if axis == 0:
        return codes + (HEAD_DIM // group) * meta
    return codes + HEAD_DIM * meta / group


def attention_bytes(w, nq, nr) -> float:
    """Codes + metadata of every attended compressed token, the BF16 window rows, q (bf16), the
    output (fp32) and the block-table entries (paged).  Split-K partials are not counted."""
    H, Hq = w.n_kv_heads, w.n_q_heads
    per_tok = side_token_bytes(w.k.astuple()) + side_token_bytes(w.v.astuple())
    total = 0.0
    for a, r in zip(nq, nr):
        total += a * H * per_tok + r * H * HEAD_DIM * 2 * 2
        total += Hq * HEAD_DIM * (2 + 4)
        if w.paged:
            total += -(-a // 16) * 4
    return total


def append_bytes(w, nq_before, nr_before) -> tuple[float, int]:
    """Bytes of one flush-where-due + append-one step, and the number of flushing sequences."""
    H, R = w.n_kv_heads, w.residual
    row_bf16 = H * HEAD_DIM * 2
    per_tok = side_token_bytes(w.k.astuple()) + side_token_bytes(w.v.astuple())
    total, flushes = 0.0, 0
    for a, r in zip(nq_before, nr_before):
        total += 2 * row_bf16  # read the new K and V rows
        if R == 0:
            total += H * per_tok
        else:
            if r == R:
                flushes += 1
                total += R * 2 * row_bf16 + R * H * per_tok
            total += 2 * row_bf16  # window write
    return total, flushes


def advance(w, nq, nr):
    """Host copy of the per-sequence state machine: flush a full window, then append one."""
    R = w.residual
    nq, nr = list(nq), list(nr)
    for b in range(len(nq)):
        if R == 0:
            nq[b] += 1
        else:
            if nr[b] == R:
                nq[b] += R
                nr[b] = 0
            nr[b] += 1
    return nq, nr


# ------------------------------------------------------------------------------------------
# Workload state on the GPU
# ------------------------------------------------------------------------------------------

class State:
    pass


def setup(name: str, extra_steps: int, device="cuda"):
    import torch

    import kvq_inputs as ki
    from quantized_kv_cache_07_amd import kvq

    layers = 1
    base = name
    if name == "c2x32":
        base, layers = "c2", 32
    w = ki.CONFIGS[base]
    lens = ki.lengths(w)
    R = w.residual
    st = State()
    st.name, st.w, st.layers, st.lens = name, w, layers, lens
    k_side, v_side = w.k.astuple(), w.v.astuple()
    st.caches = []
    for layer in range(layers):
        lw = w if layers == 1 else ki.Workload(**{**w.__dict__, "seed": 1000 * w.seed + layer})
        if w.paged:
            table, nblk = ki.block_tables(lw, lens, extra_tokens=R + extra_steps + 32)
            cache = kvq.Cache(k_side, v_side, w.batch, w.n_kv_heads, residual=R,
                              block_table=torch.from_numpy(table), num_blocks=nblk, device=device)
        else:
            gt = w.k.group if w.k.axis == ki.PER_CHANNEL else 16
            cap = -(-(max(lens) + R + extra_steps + 16) // gt) * gt
            cache = kvq.Cache(k_side, v_side, w.batch, w.n_kv_heads, residual=R, capacity=cap,
                              device=device)
        for b in range(w.batch):
            # prefill in pieces of at most 16384 tokens; the window state is carried by the cache
            t0 = 0
            while t0 < lens[b]:
                n = min(16384, lens[b] - t0)
                k, v = ki.prefill_kv(lw, b, n, device=device, t0=t0)
                kvq.quantize_append(cache, k[None].contiguous(), v[None].contiguous(),
                                    desc=cache.sequence(b))
                t0 += n
        st.caches.append((lw, cache))
    torch.cuda.synchronize()
    for _, cache in st.caches:
        if kvq.read_error(cache):
            raise RuntimeError("device error during prefill")
    if R:
        st.nq = [R * ((t - 1) // R) for t in lens]
        st.nr = [t - a for t, a in zip(lens, st.nq)]
    else:
        st.nq, st.nr = list(lens), [0] * w.batch
    got_nq = st.caches[0][1].n_quant.cpu().tolist()
    got_nr = st.caches[0][1].n_res.cpu().tolist()
    assert got_nq == st.nq and got_nr == st.nr, "prefill counters disagree with the state machine"
    st.max_tokens = max(lens) + extra_steps + 1
    st.ws = torch.empty(kvq.workspace_bytes(st.caches[0][1], w.n_q_heads, st.max_tokens),
                        dtype=torch.uint8, device=device)
    st.out = torch.empty((w.batch, w.n_q_heads, HEAD_DIM), dtype=torch.float32, device=device)
    return st


def make_step_inputs(st, n_steps: int, device="cuda"):
    import kvq_inputs as ki
    st.step_in = []
    for s in range(n_steps):
        per_layer = []
        for lw, _ in st.caches:
            k, v = ki.step_kv(lw, s, device)
            q = ki.queries(lw, s + 1, device)
            per_layer.append((k.contiguous(), v.contiguous(), q.contiguous()))
        st.step_in.append(per_layer)


def run_step(st, s: int) -> None:
    from quantized_kv_cache_07_amd import kvq
    w = st.w
    for (lw, cache), (k, v, q) in zip(st.caches, st.step_in[s]):
        if w.step_append or st.layers > 1:
            # the append flushes every full window before adding the token (kvq.h contract);
            # a separate kvq_flush_residual call would only add two launches
            kvq.quantize_append(cache, k, v)
        kvq.decode_attention(cache, q, st.max_tokens, out=st.out, workspace=st.ws)


def attention_only(st, q) -> None:
    from quantized_kv_cache_07_amd import kvq
    for _, cache in st.caches:
        kvq.decode_attention(cache, q, st.max_tokens, out=st.out, workspace=st.ws)


def settle(st, q, window: int = 10, max_windows: int = 30, tol: float = 0.02) -> int:
    """Untimed read-only attention calls until the per-call time of two consecutive windows
    agrees within `tol` (at least three windows).  On a cold start the first calls over the
    prefilled cache run up to 2x slower (clocks ramping, address translations not yet cached);
    the cache state does not change.  Returns the number of calls made."""
    import torch
    prev, calls = None, 0
    for i in range(max_windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(window):
            attention_only(st, q)
        e1.record()
        torch.cuda.synchronize()
        calls += window
        t = e0.elapsed_time(e1)
        if prev is not None and i >= 2 and abs(t - prev) <= tol * prev:
            break
        prev = t
    return calls


# ------------------------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample of the same sequences
# ------------------------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host threads for the N-core leg: the cores this process may run on, at most 16 (one GPU's
    share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(st, gpu_out0, q0, budget_s: float = 15.0):
    """The oracle's fp64 attention, as it stands, over the shortest sequences of the workload
    until about budget_s of single-core work: once on one pinned core, then the same sequences
    on N threads (one sequence per task; the oracle's C calls release the GIL).  Both legs
    compute the same outputs, compared with the GPU's."""
    import concurrent.futures as cf

    import numpy as np

    import kvq_inputs as ki
    from oracle import oracle

    w = st.w
    lw = st.caches[0][0]
    sm = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))
    order = sorted(range(w.batch), key=lambda b: st.lens[b])  # shortest first: bounded sample
    qb = ki.bf16_bits(q0)
    used, seqs, t_attn, nbytes, max_err = [], [], 0.0, 0.0, 0.0
    ok = True
    try:
        aff = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(aff)})  # the single-core leg on one pinned core
    except (AttributeError, OSError):
        aff = None
    try:
        for b in order:
            T = st.lens[b]
            seq = oracle.Sequence(w.k.astuple(), w.v.astuple(), w.n_kv_heads, w.residual,
                                  -(-(T + w.residual + 64) // 64) * 64)
            k, v = ki.prefill_kv(lw, b, T, device="cpu")
            seq.append(ki.bf16_bits(k), ki.bf16_bits(v))
            t0 = time.perf_counter()
            ref = seq.attend(qb[b], sm)
            t_attn += time.perf_counter() - t0
            nbytes += attention_bytes(w, [seq.n_quant], [seq.n_res])
            used.append((b, T))
            seqs.append(seq)
            err = np.abs(gpu_out0[b] - ref)
            max_err = max(max_err, float(err.max()))
            ok = ok and bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ref)))
            if t_attn >= budget_s:
                break
    finally:
        if aff is not None:
            os.sched_setaffinity(0, aff)
    n = cpu_threads()
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        outs = list(ex.map(lambda i: seqs[i].attend(qb[used[i][0]], sm), range(len(seqs))))
    t_n = time.perf_counter() - t0
    same = all(np.array_equal(o, seqs[i].attend(qb[used[i][0]], sm)) for i, o in
               enumerate(outs[:2]))
    model = cpu_model()
    return {
        "value": nbytes / t_n / 1e9,
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "value_1core": nbytes / t_attn / 1e9,
        "seconds_1core": round(t_attn, 3),
        "seconds_ncore": round(t_n, 3),
        "cpu_model": model,
        "sample": (f"fp64 oracle attention (all {w.n_q_heads} query heads) over sequences "
                   f"{[b for b, _ in used]} with {sum(t for _, t in used)} cached tokens: "
                   f"{t_attn:.1f} s on one pinned core, {t_n:.2f} s on {n} threads (one sequence "
                   f"per task) of a {model}; same algorithmic-byte count as the GPU"),
    }, {"sequences": [b for b, _ in used], "max_abs_err": max_err, "within_tolerance": ok,
        "ncore_equals_1core": same}


# ------------------------------------------------------------------------------------------
# Counter-derived traffic committed under profiles/
# ------------------------------------------------------------------------------------------

DECODE_SOURCES = ("kvq_decode.h", "kvq_dev.h", "kvq_host.hip")


def decode_source_hash() -> str:
    """Hash of the sources that decide the decode-attention call's memory traffic: the kernels,
    the unit weights and layout constants, and the host's launch configuration (the counters go
    stale when any of them changes)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_kv_cache_07_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


CALIBRATION_BYTES = 1 << 30  # plain copy of known size, for scaling the byte counters


def _counter_rows(directory: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        rows.extend(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    return rows


def _per_dispatch(rows, counter: str, kernel_substr: str) -> float:
    """Mean over dispatches of a kernel of one counter (summed over its dimensions)."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
            continue
        per[r.get("Dispatch_Id") or r.get("Correlation_Id")] = (
            per.get(r.get("Dispatch_Id") or r.get("Correlation_Id"), 0.0) + float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no {counter} samples for {kernel_substr}")
    return sum(per.values()) / len(per)


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, command: str) -> dict:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one decode-attention call (decode_kernel +
    combine_kernel), each scaled by what the counter reads for a plain copy of known size."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    copy_f = _per_dispatch(fr, "FETCH_SIZE", "measure_copy_kernel") * 1024
    copy_w = _per_dispatch(wr, "WRITE_SIZE", "measure_copy_kernel") * 1024
    kf, kw = CALIBRATION_BYTES / copy_f, CALIBRATION_BYTES / copy_w
    out = {"workload": workload, "command": command,
           "decode_sources": list(DECODE_SOURCES),
           "decode_sources_sha256_16": decode_source_hash(),
           "calibration": {"copy_bytes": CALIBRATION_BYTES, "fetch_counter_bytes": copy_f,
                           "write_counter_bytes": copy_w, "fetch_scale": kf, "write_scale": kw}}
    total = 0.0
    for name in ("decode_kernel", "combine_kernel"):
        f = _per_dispatch(fr, "FETCH_SIZE", name) * 1024 * kf
        w = _per_dispatch(wr, "WRITE_SIZE", name) * 1024 * kw
        out[name] = {"fetch_bytes": round(f), "write_bytes": round(w)}
        total += f + w
    out["bytes_per_launch"] = round(total)
    return out


def summarize_pmc(dirs, kernel_substr: str = "decode_kernel") -> str:
    """Mean per dispatch of every counter in rocprofv3 --pmc output directories (one line per
    directory, one pass each), over the dispatches of kernels whose name holds kernel_substr."""
    out = []
    for d in dirs:
        rows = _counter_rows(d)
        names = sorted({r["Counter_Name"] for r in rows})
        n = len({r.get("Dispatch_Id") or r.get("Correlation_Id") for r in rows
                 if kernel_substr in r["Kernel_Name"]})
        vals = " ".join(f"{c}={_per_dispatch(rows, c, kernel_substr):.4g}" for c in names)
        out.append(f"{os.path.basename(os.path.normpath(d))}: {vals} (dispatches {n})")
    return "\n".join(out) + "\n"


def summarize_stats(stats_csv: str, command: str, title: str) -> str:
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (from the repository root on the GPU box):", "",
             f"    {command}", "",
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in rows:
        if "kvq" not in r["Name"]:
            continue
        lines.append(f"{r['Name'][:58]:58s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_csv: str, bench_json: str, command: str, workload: str) -> str:
    """Per-dispatch durations of the kvq kernels from a rocprofv3 --kernel-trace CSV, split into
    the phases of one bench.py run (its JSON line gives the counts): the untimed calls (the
    prefilled-state call and the settle phase), the warmup and timed steps, and the
    back-to-back attention loop whose average is the line's roofline figure."""
    import csv
    import statistics
    line = None
    for raw in open(bench_json):
        raw = raw.strip()
        if raw.startswith("{"):
            line = json.loads(raw)
    if line is None:
        raise SystemExit(f"no JSON line in {bench_json}")
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    def durs(sub):
        return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
                if sub in r["Kernel_Name"]]
    dec, comb = durs("decode_kernel"), durs("combine_kernel")
    quant, tail = durs("quantize_kernel"), durs("tail_kernel")
    layers = line["config"].get("layers", 1)
    W, K, A = line["warmup"], line["steps"], line["roofline"].get("attn_reps", 50)
    n_loop, n_steps = (A + 3) * layers, (W + K) * layers
    nd = len(dec)
    groups = [("untimed (prefilled-state call + settle phase)", 0, nd - n_loop - n_steps),
              ("warmup steps", nd - n_loop - n_steps, nd - n_loop - K * layers),
              ("timed steps", nd - n_loop - K * layers, nd - n_loop),
              ("attention loop (3 warm + the roofline's calls)", nd - n_loop, nd - n_loop + 3 * layers),
              ("roofline calls", nd - A * layers, nd)]
    out = [f"# Kernel trace: decode attention, workload {workload}", "",
           "Command (from the repository root on the GPU box):", "", f"    {command}", "",
           f"Bench line of the same run: ms_per_step {line['ms_per_step']}, roofline avg_launch_us "
           f"{line['roofline']['avg_launch_us']} (HIP events around {A} back-to-back calls), frac "
           f"{line['roofline']['frac']}, settle_calls {line.get('settle_calls')}.", "",
           "Durations in µs per dispatch (kernel start to end, from the trace).", "",
           "| phase | kernel | calls | mean | median | min | max |", "|---|---|---|---|---|---|---|"]
    for name, lo, hi in groups:
        for kname, xs in (("decode_kernel", dec), ("combine_kernel", comb)):
            sel = xs[max(lo, 0):max(hi, 0)]
            if not sel:
                continue
            out.append(f"| {name} | {kname} | {len(sel)} | {statistics.mean(sel):.2f} | "
                       f"{statistics.median(sel):.2f} | {min(sel):.2f} | {max(sel):.2f} |")
    rl_dec = dec[-A * layers:]
    rl_comb = comb[-A * layers:] if len(comb) >= A * layers else []
    tot = statistics.mean(rl_dec) + (statistics.mean(rl_comb) if rl_comb else 0.0)
    ab = line["roofline"]["algorithmic_bytes_per_launch"]
    out += ["", f"Roofline calls: decode_kernel + combine_kernel mean {tot:.2f} µs per call "
            f"(kernel time only; the bench's {line['roofline']['avg_launch_us']} µs also holds the "
            f"gaps between launches) -> {ab / (tot * 1e-6) / 1e9:.1f} GB/s = "
            f"{ab / (tot * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} of 8 TB/s for {ab} algorithmic bytes."]
    if len(quant) >= K * layers > 0:
        qt, tt = quant[-K * layers:], tail[-K * layers:]
        out += ["", f"Append kernels of the timed steps ({len(qt)} calls): quantize_kernel mean "
                f"{statistics.mean(qt):.2f} µs (median {statistics.median(qt):.2f}), tail_kernel "
                f"mean {statistics.mean(tt):.2f} µs (median {statistics.median(tt):.2f})."]
    return "\n".join(out) + "\n"


def counter_traffic(workload: str):
    """Per-launch HBM bytes of the decode kernel from the committed rocprofv3 counter summary,
    or None when there is none for this workload or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("decode_sources_sha256_16") != decode_source_hash():
        return None
    return d.get("bytes_per_launch")


# ------------------------------------------------------------------------------------------

# ------------------------------------------------------------------------------------------
# Crossover sweep: unquantized BF16 against FP8 / INT8 / INT4 / INT2 decode attention over context
# length and batch [P2, "Why compression may also improve speed": fewer bytes to stream against
# the instructions spent decoding them, with short contexts where decoding can cost more]
# ------------------------------------------------------------------------------------------

SWEEP_FORMATS = {
    "bf16": (16, 0, 0, 128),
    "fp8-head": (8, 2, 3, 0),
    "int8-g128": (8, 0, 0, 128),
    "int4-g64": (4, 0, 0, 64),
    "int2-g32": (2, 0, 0, 32),
}


def sweep_crossover(batches, lengths, calls_per_graph: int = 20, replays: int = 5) -> list[dict]:
    """Device time of one decode-attention call per (batch, context length, format), H_q = 32,
    H_kv = 8, head_dim 128, contiguous caches without a window.  The calls are captured in a HIP
    graph and replayed, so the time is the GPU's, not the host's launch rate; the first replay's
    output is checked bit for bit against an eager call."""
    import torch

    import kvq_inputs as ki
    from quantized_kv_cache_07_amd import kvq

    rows = []
    for B in batches:
        for T in lengths:
            base = None
            for name, side in SWEEP_FORMATS.items():
                w = ki.Workload(f"sweep-{name}", 11, B, 32, 8, T, ki.Side(*side), ki.Side(*side))
                cap = -(-(T + 16) // 16) * 16
                # FP8: per-head scales of the N(0, 1) inputs, amax / 448 with amax ~ 5
                f8 = {"fp8_scales": ([5.0 / 448] * 8, [5.0 / 448] * 8)} if side[1] == 2 else {}
                cache = kvq.Cache(side, side, B, 8, residual=0, capacity=cap, **f8)
                k = torch.empty((B, T, 8, HEAD_DIM), dtype=torch.bfloat16, device="cuda")
                v = torch.empty_like(k)
                for b in range(B):
                    kb, vb = ki.prefill_kv(w, b, T, device="cuda")
                    k[b].copy_(kb)
                    v[b].copy_(vb)
                kvq.quantize_append(cache, k, v)
                del k, v
                q = ki.queries(w, 0, "cuda")
                out = torch.empty((B, 32, HEAD_DIM), dtype=torch.float32, device="cuda")
                ws = torch.empty(kvq.workspace_bytes(cache, 32, T), dtype=torch.uint8, device="cuda")
                kvq.decode_attention(cache, q, T, out=out, workspace=ws)
                torch.cuda.synchronize()
                if kvq.read_error(cache):
                    raise RuntimeError(f"device error in sweep {name} B={B} T={T}")
                ref = out.clone()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(calls_per_graph):
                        kvq.decode_attention(cache, q, T, out=out, workspace=ws)
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(out, ref):
                    raise RuntimeError(f"graph replay differs from the eager call ({name} B={B} T={T})")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(replays):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (replays * calls_per_graph)
                nbytes = attention_bytes(w, [T] * B, [0] * B)
                row = {"batch": B, "tokens": T, "format": name, "us_per_call": round(us, 2),
                       "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "kv_tokens_per_s": round(B * T / (us * 1e-6), 1),
                       "kv_bytes": int(nbytes)}
                if name == "bf16":
                    base = us
                row["speedup_vs_bf16"] = round(base / us, 3)
                rows.append(row)
                print(json.dumps(row), flush=True)
                del g, cache, ws, out
                torch.cuda.empty_cache()
    return rows


# the multi-query sweep adds 2-bit codes in key groups of 64 (a dense-kernel instance of its own)
MQ_FORMATS = dict(SWEEP_FORMATS, **{"int2-g64": (2, 0, 0, 64)})


def sweep_multiquery(batch: int, tokens: int, nqs, calls_per_graph: int = 10,
                     replays: int = 5) -> list[dict]:
    """Device time of one multi-query decode call (n_q query tokens per sequence, causal, the
    last n_q cached tokens) per format, against n_q single-query calls, H_q = 32, H_kv = 8,
    contiguous caches of `tokens` tokens without a window (HIP-graph replay)."""
    import torch

    import kvq_inputs as ki
    from quantized_kv_cache_07_amd import kvq

    rows = []
    for name, side in MQ_FORMATS.items():
        w = ki.Workload(f"mq-{name}", 13, batch, 32, 8, tokens, ki.Side(*side), ki.Side(*side))
        cap = -(-(tokens + 16) // 16) * 16
        f8 = {"fp8_scales": ([5.0 / 448] * 8, [5.0 / 448] * 8)} if side[1] == 2 else {}
        cache = kvq.Cache(side, side, batch, 8, residual=0, capacity=cap, **f8)
        for b in range(batch):
            k, v = ki.prefill_kv(w, b, tokens, device="cuda")
            kvq.quantize_append(cache, k[None].contiguous(), v[None].contiguous(), desc=cache.sequence(b))
        single = None
        for nq in nqs:
            q = torch.stack([ki.queries(w, i, "cuda") for i in range(nq)], dim=1).contiguous()
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            ws = torch.empty(kvq.workspace_bytes_mq(cache, 32, nq, tokens), dtype=torch.uint8,
                             device="cuda")
            kvq.decode_attention_mq(cache, q, tokens, out=out, workspace=ws)
            torch.cuda.synchronize()
            if kvq.read_error(cache):
                raise RuntimeError(f"device error in multi-query sweep {name} n_q={nq}")
            ref = out.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(calls_per_graph):
                    kvq.decode_attention_mq(cache, q, tokens, out=out, workspace=ws)
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError(f"graph replay differs from the eager call ({name} n_q={nq})")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (replays * calls_per_graph)
            if nq == 1:
                single = us
            row = {"format": name, "batch": batch, "tokens": tokens, "n_q": nq,
                   "us_per_call": round(us, 2),
                   "query_tokens_per_s": round(batch * nq / (us * 1e-6), 1),
                   "vs_separate_calls": round(nq * single / us, 3) if single else None,
                   "cache_gbs": round(attention_bytes(w, [tokens] * batch, [0] * batch) / (us * 1e-6) / 1e9, 1)}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del g
        del cache
        torch.cuda.empty_cache()
    return rows


def multiquery_table(rows: list[dict], command: str) -> str:
    fmts = list(MQ_FORMATS)
    B, T = rows[0]["batch"], rows[0]["tokens"]
    out = ["# Multi-query decode over the quantized cache (MI355X, one GPU)", "",
           "Command (from the repository root on the GPU box):", "", f"    {command}", "",
           f"Device time of one causal multi-query `kvq_decode_attention_mq` call (HIP-graph "
           f"replay), batch {B}, {T} cached tokens per sequence, H_q = 32, H_kv = 8, contiguous, "
           f"no window; in parentheses the speed-up over n_q single-query calls.", "",
           "| n_q | " + " | ".join(f"{f} µs" for f in fmts) + " |", "|---|" + "---|" * len(fmts)]
    by = {}
    for r in rows:
        by.setdefault(r["n_q"], {})[r["format"]] = r
    for nq, d in sorted(by.items()):
        cells = []
        for f in fmts:
            r = d.get(f)
            cells.append("—" if r is None else f"{r['us_per_call']:.1f} ({r['vs_separate_calls']:.2f}×)")
        out.append(f"| {nq} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def sweep_table(rows: list[dict], command: str) -> str:
    fmts = list(SWEEP_FORMATS)
    out = ["# Decode attention: BF16 against quantized caches (MI355X, one GPU)", "",
           "Command (from the repository root on the GPU box):", "", f"    {command}", "",
           "Device time of one `kvq_decode_attention` call (HIP-graph replay), H_q = 32, "
           "H_kv = 8, head_dim 128, contiguous caches, no window; speed-up against the BF16 "
           "cache in parentheses. Working sets below ~256 MB fit the Infinity Cache.", "",
           "| batch | tokens | KV bytes (bf16) | " + " | ".join(f"{f} µs" for f in fmts) + " |",
           "|---|---|---|" + "---|" * len(fmts)]
    by = {}
    for r in rows:
        by.setdefault((r["batch"], r["tokens"]), {})[r["format"]] = r
    for (B, T), d in sorted(by.items()):
        cells = []
        for f in fmts:
            r = d.get(f)
            cells.append("—" if r is None else
                         (f"{r['us_per_call']:.1f}" if f == "bf16" else
                          f"{r['us_per_call']:.1f} ({r['speedup_vs_bf16']:.2f}×)"))
        kb = d["bf16"]["kv_bytes"] if "bf16" in d else 0
        out.append(f"| {B} | {T} | {kb / 2**20:.1f} MiB | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c2x32", "c3", "c4", "c4p", "c5"])
    ap.add_argument("--attn-reps", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps and the attention loop in HIP graphs (removes "
                         "the host's launch rate from launch-bound workloads such as c2x32)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_<workload>_traffic.json from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print a text summary of a rocprofv3 --stats kernel table")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_TRACE_CSV", "BENCH_JSON"),
                    help="print per-phase kernel durations of one bench run from its rocprofv3 "
                         "--kernel-trace CSV and its JSON line")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="PMC_DIR",
                    help="print per-dispatch means of the counters of decode_kernel in rocprofv3 "
                         "--pmc output directories")
    ap.add_argument("--command", default="", help="the profiling command, recorded in summaries")
    ap.add_argument("--sweep", choices=["crossover", "multiquery"],
                    help="instead of the step benchmark: BF16 vs quantized decode-attention sweep")
    ap.add_argument("--sweep-batches", default="1,16")
    ap.add_argument("--sweep-lengths", default="512,2048,8192,32768,131072")
    ap.add_argument("--sweep-out", default="", help="write the sweep's markdown table here")
    ap.add_argument("--sweep-nq", default="1,2,4,8,16",
                    help="multi-query sweep: query tokens per sequence (1 is the single-query base)")
    ap.add_argument("--pmc-kernel", default="decode_kernel",
                    help="--summarize-pmc: the kernels (name substring) whose dispatches are averaged")
    a = ap.parse_args()
    if a.summarize_counters:
        d = summarize_counters(*a.summarize_counters, a.workload, a.command)
        out = os.path.join(ROOT, "profiles", f"decode_{a.workload}_traffic.json")
        json.dump(d, open(out, "w"), indent=1)
        print(json.dumps(d, indent=1))
        return 0
    if a.summarize_pmc:
        print(summarize_pmc(a.summarize_pmc, a.pmc_kernel), end="")
        return 0
    if a.summarize_stats:
        print(summarize_stats(a.summarize_stats, a.command, f"kvq kernels, workload {a.workload}"), end="")
        return 0
    if a.summarize_trace:
        print(summarize_trace(*a.summarize_trace, a.command, a.workload), end="")
        return 0
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the path is sharded by sequence or kv head across GPUs, not built here)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import kvq_inputs as ki
    from quantized_kv_cache_07_amd import kvq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if a.sweep == "multiquery":
        nqs = [int(x) for x in a.sweep_nq.split(",")]
        if nqs[0] != 1:
            raise SystemExit("--sweep-nq must start with 1 (the single-query base of the table)")
        rows = sweep_multiquery(16, 32768, nqs)
        if a.sweep_out:
            open(a.sweep_out, "w").write(multiquery_table(rows, a.command or "python bench.py --sweep multiquery"))
        return 0
    if a.sweep == "crossover":
        rows = sweep_crossover([int(x) for x in a.sweep_batches.split(",")],
                               [int(x) for x in a.sweep_lengths.split(",")])
        if a.sweep_out:
            cmd = a.command or "python bench.py --sweep crossover"
            open(a.sweep_out, "w").write(sweep_table(rows, cmd))
        return 0
    dev = "cuda"
    n_total = a.warmup + a.steps
    print(f"[bench] setup {a.workload}", file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    st = setup(a.workload, n_total + 1, dev)
    w = st.w

    # Output of the prefilled state, kept for the parity check of the CPU sample.
    q0 = ki.queries(st.caches[0][0], 0, dev)
    kvq.decode_attention(st.caches[0][1], q0, st.max_tokens, out=st.out, workspace=st.ws)
    torch.cuda.synchronize()
    gpu_out0 = st.out.cpu().numpy().copy()
    make_step_inputs(st, n_total, dev)
    torch.cuda.synchronize()
    print(f"[bench] setup done in {time.perf_counter() - t_setup:.1f} s", file=sys.stderr,
          flush=True)
    settle_calls = settle(st, q0)
    print(f"[bench] settled after {settle_calls} untimed attention calls", file=sys.stderr,
          flush=True)

    # Host copy of the state machine, for the algorithmic bytes of each step.
    appends = w.step_append or st.layers > 1
    nq, nr = st.nq, st.nr
    step_bytes, attn_tokens, flushes = [], 0, 0
    for s in range(n_total):
        ab, fl = (0.0, 0)
        if appends:
            ab, fl = append_bytes(w, nq, nr)
            nq, nr = advance(w, nq, nr)
        if s >= a.warmup:
            step_bytes.append(st.layers * (ab + attention_bytes(w, nq, nr)))
            attn_tokens += st.layers * (sum(nq) + sum(nr))
            flushes += st.layers * fl

    for s in range(a.warmup):
        run_step(st, s)
    torch.cuda.synchronize()
    step_graph = None
    if a.graph:
        # the timed steps captured into one HIP graph (no allocation or memset inside: outputs
        # and workspace are preallocated); replayed once below, so the host's launch rate is
        # out of the timed region
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph):
            for s in range(a.warmup, n_total):
                run_step(st, s)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    if step_graph is not None:
        step_graph.replay()
    else:
        for s in range(a.warmup, n_total):
            run_step(st, s)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_ms = e0.elapsed_time(e1)
    for _, cache in st.caches:
        if kvq.read_error(cache):
            raise RuntimeError("device error during the timed steps")
    assert st.caches[0][1].n_quant.cpu().tolist() == nq, "counter drift"
    assert st.caches[0][1].n_res.cpu().tolist() == nr, "counter drift"
    ms_per_step = t_ms / a.steps
    gbs = sum(step_bytes) / (t_ms * 1e-3) / 1e9
    tok_s = attn_tokens / (t_ms * 1e-3)

    # Decode-attention call alone, on the final state, back to back on the current stream.
    q = st.step_in[-1][0][2]
    if step_graph is not None:
        # the graph's last call (the last layer of the last step) left its output in st.out: an
        # eager call on the same final state must reproduce it bit for bit
        from_graph = st.out.clone()
        lw_last, cache_last = st.caches[-1]
        kvq.decode_attention(cache_last, st.step_in[-1][-1][2], st.max_tokens, out=st.out,
                             workspace=st.ws)
        torch.cuda.synchronize()
        if not torch.equal(from_graph, st.out):
            raise RuntimeError("graph replay differs from the eager call")
    for _ in range(3):
        attention_only(st, q)
    torch.cuda.synchronize()
    attn_graph = None
    if a.graph:
        attn_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(attn_graph):
            for _ in range(a.attn_reps):
                attention_only(st, q)
        attn_graph.replay()  # untimed first replay
        torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    if attn_graph is not None:
        attn_graph.replay()
    else:
        for _ in range(a.attn_reps):
            attention_only(st, q)
    a1.record()
    torch.cuda.synchronize()
    attn_us = a0.elapsed_time(a1) * 1e3 / (a.attn_reps * st.layers)
    attn_b = attention_bytes(w, nq, nr)
    achieved = attn_b / (attn_us * 1e-6) / 1e9
    traffic = counter_traffic(a.workload)

    # Measured read-stream ceiling (128-bit loads over 4 GiB, same stream).
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(kvq.lib.kvq_measure_read_sink_floats(), dtype=torch.float32, device=dev)
    kvq.measure_read(buf, sink)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(10):
        kvq.measure_read(buf, sink)
    r1.record()
    torch.cuda.synchronize()
    stream_gbs = 10 * buf.numel() / (r0.elapsed_time(r1) * 1e-3) / 1e9
    # plain copies of known size: the reference for scaling the hardware byte counters
    half = CALIBRATION_BYTES
    for _ in range(3):
        kvq.measure_copy(buf[half:2 * half], buf[:half])
    torch.cuda.synchronize()
    del buf

    cpu, parity = None, None
    if not a.no_cpu:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu, parity = cpu_baseline(st, gpu_out0, q0, a.cpu_budget)
        cpu["cores_available"] = os.cpu_count()

    desc = w.description if st.layers == 1 else (
        "worked example: 32 layers x " + w.description.split(": ", 1)[1])
    line = {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak), KV tokens/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes, fp16 scales, fp32 accumulate" if w.k.bits == 4 else
                 f"int{w.k.bits} codes, fp16 scales, fp32 accumulate",
        "data": "synthetic (seeded counter-hash generator, generated on the GPU)",
        "config": {"workload": f"{a.workload}: {desc}", "batch": w.batch,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": HEAD_DIM,
                   "layers": st.layers, "tokens_min": min(st.lens), "tokens_max": max(st.lens),
                   "cached_tokens": int(sum(st.lens)), "residual": w.residual,
                   "paged": w.paged, "step": ("flush where due + append 1 + attention"
                                              if appends else "attention"),
                   "launch": "hip graph" if a.graph else "eager"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "kv_tokens_per_s": round(tok_s, 1),
        "flushes_in_timed_steps": flushes,
        "wall_s_timed": round(wall, 4),
        "settle_calls": settle_calls,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode attention call: decode_kernel + combine_kernel",
                     "algorithmic_bytes_per_launch": int(attn_b),
                     "avg_launch_us": round(attn_us, 3), "attn_reps": a.attn_reps},
        "stream_read_ceiling_gbs": round(stream_gbs, 1),
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
