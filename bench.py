"""Decode-step benchmark on one MI355X.

Default workload: the Llama-3.2-1B-shaped decoder (16 layers, hidden 2048,
32/8 heads of 64, SwiGLU 8192, vocab 128256, tied), batch 1, seeded KV
prefill of 512 positions, greedy decode (positions 512, 513, ...), seeded
random weights (synthetic data).  A step is one full decode step: every
layer and the LM head with greedy argmax, inputs resident in HBM.

Prints one JSON line: decode tokens/s (value), the roofline of the dominant
kernel (algorithmic HBM bytes per launch / its measured duration, against
8 TB/s), the HBM traffic the hardware counters saw for that kernel (from the
committed counter summary, when it was taken on the current kernel sources)
and the CPU oracle's rate on a bounded sample.

--copy-calibration instead copies a 1 GiB device buffer three times: the
plain copy whose FETCH_SIZE / WRITE_SIZE counters scale the kernel's.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak (no sparsity)
MFMA_MIN_BATCH = 16  # from this many rows the projections run on the MFMA engine
CSRC = os.path.join(ROOT, "overlap_decode_step_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_mega_llama1b_b1_hbm_traffic.md")


def algorithmic_bytes(shape, batch, positions):
    """HBM bytes one decode step must move: bf16 weights once (norm gains
    included), each sequence's embedding row, bf16 K/V read over 0..p plus the
    new row written, and the fp32 logits written."""
    H, V, I, L = shape["hidden"], shape["vocab"], shape["intermediate"], shape["n_layers"]
    qd, kvd = shape["n_q_heads"] * shape["head_dim"], shape["n_kv_heads"] * shape["head_dim"]
    weights = 2 * (V * H * (1 if shape["tied"] else 2) + H
                   + L * (2 * H + (qd + 2 * kvd) * H + H * qd + 3 * I * H))
    kv_row = 2 * L * kvd * 2  # K and V, bf16, all layers, one position
    per_seq = [2 * H + kv_row * (p + 1) + kv_row + 4 * V for p in positions]
    return weights + sum(per_seq)


def algorithmic_flops(shape, batch, positions):
    """Floating-point operations of one decode step (a multiply-add counts
    two): every projection row once per sequence (QKV, O, gate, up, Down, LM
    head), then attention's q.K and p.V over positions 0..p of every query
    head.  Returns (projections, attention); from 16 rows the projections run
    on the MFMA engine and attention on the vector units."""
    H, V, I, L = shape["hidden"], shape["vocab"], shape["intermediate"], shape["n_layers"]
    qd, kvd = shape["n_q_heads"] * shape["head_dim"], shape["n_kv_heads"] * shape["head_dim"]
    proj = 2 * batch * (L * (H * (qd + 2 * kvd) + qd * H + 3 * H * I) + V * H)
    attn = sum(4 * L * qd * (p + 1) for p in positions)
    return proj, attn


def kernel_source_digest():
    """Digest of the HIP/C++ sources the decode kernels are built from."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(mode, batch):
    """HBM bytes per launch of the persistent kernel from the committed counter
    summary, or None when there is none for this launch or the kernel sources
    have changed since the counters were taken."""
    if mode != "mega" or batch != 1 or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu():
    """The host the oracle ran on: CPU model, logical CPUs (nproc) and the CPUs
    this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(shape, prefill, steps):
    """The oracle (single-threaded C, fp32 over bf16 weights) decoding `steps`
    greedy steps of sequence 0 from position `prefill`; weights and KV are
    generated first and not timed."""
    from oracle.lo import Oracle
    from synth import workloads as W
    orc = Oracle("f32")
    om = orc.model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
    okv = orc.kv(shape, 1, prefill + steps + 1, seed=W.SEED_KV, kv_std=1.0, prefill=[prefill])
    tok = W.first_tokens(1, shape["vocab"])[0]
    w0, c0 = time.perf_counter(), time.process_time()
    for s in range(steps):
        _, tok = orc.decode_one(om, okv, 0, tok, prefill + s)
    wall, cpu = time.perf_counter() - w0, time.process_time() - c0
    return {"value": steps / wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": f"{steps} greedy steps of one sequence, positions {prefill}..{prefill + steps - 1}, "
                      f"same shape and seeds; {wall:.1f} s wall, {cpu:.1f} s CPU (one thread)"}


def batch_sweep(runs=4, steps=64, batches=(1, 4, 16, 64)):
    """Short-context batch sweep of the Llama-1B shape: per-sequence KV length
    drawn from U[256, 1024] (seeded), `steps` greedy steps, every mode; each
    configuration timed `runs` times (median, min, max of tokens/s)."""
    import statistics
    import torch
    from overlap_decode_step_amd import ld
    from synth import workloads as W
    shape = W.LLAMA_1B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
    maxb = max(batches)
    m.alloc_kv(maxb, 1024 + steps + 8)
    stream = torch.cuda.current_stream()
    table = {}
    for B in batches:
        prefill = W.kv_lengths(B, 256, 1024)
        logits = torch.empty((B, shape["vocab"]), dtype=torch.float32, device=dev)
        toks = torch.tensor(W.first_tokens(B, shape["vocab"]), dtype=torch.int32, device=dev)
        pos_all = [torch.tensor([p + i for p in prefill], dtype=torch.int32, device=dev)
                   for i in range(steps)]
        pbuf = torch.empty_like(pos_all[0])
        tbuf = [toks.clone(), torch.empty_like(toks)]

        def step(mode, i):
            if mode == "graph":
                # a captured step replays fixed addresses: the positions are
                # updated in place (timed with the step)
                pbuf.copy_(pos_all[i])
                m.step(tbuf[i & 1], pbuf, logits, tbuf[(i + 1) & 1])
            else:
                m.step(tbuf[i & 1], pos_all[i], logits, tbuf[(i + 1) & 1])

        row = {}
        for mode in ("wait", "flags", "mega", "graph"):
            m.set_mode(mode)
            rates = []
            fill = prefill + [0] * (maxb - B)  # one length per cache slot
            for _ in range(runs):
                m.fill_kv(W.SEED_KV, 1.0, fill)
                tbuf[0].copy_(toks)
                for i in range(3):  # warm-up, then the cache is refilled
                    step(mode, i)
                m.fill_kv(W.SEED_KV, 1.0, fill)
                tbuf[0].copy_(toks)
                torch.cuda.synchronize()
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for i in range(steps):
                    step(mode, i)
                ev1.record(stream)
                torch.cuda.synchronize()
                if m.device_error() != 0:
                    raise RuntimeError(f"device error at batch {B} mode {mode}")
                rates.append(B * steps * 1000.0 / ev0.elapsed_time(ev1))
            row[mode] = {"median": statistics.median(rates), "min": min(rates), "max": max(rates)}
            print(f"# sweep batch={B} mode={mode} tok/s median={row[mode]['median']:.1f} "
                  f"min={row[mode]['min']:.1f} max={row[mode]['max']:.1f}", file=sys.stderr, flush=True)
        table[B] = row
    m.free()
    return table


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def multi_token_bench(shape_name, B, M, steps, warmup, modes):
    """Several tokens per sequence per step (ld_decode_step_tokens): B
    sequences x M consecutive tokens (teacher forced: seeded tokens), KV
    prefill 512 (1024 for the 8B and 70B shapes), positions advancing by M
    per step.  Returns {mode: ms per step}; tokens/s = B * M / step time."""
    import torch
    from overlap_decode_step_amd import ld
    from synth import workloads as W
    shape = W.SHAPES[shape_name]
    w_std = W.WORKLOADS["llama70b"]["w_std"] if shape_name.startswith("llama70b") else 0.02
    prefill = 512 if shape_name == "llama1b" else 1024
    rows = B * M
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=w_std)
    m.alloc_kv(rows, prefill + (steps + warmup) * M + 8)
    logits = torch.empty((rows, shape["vocab"]), dtype=torch.float32, device=dev)
    nxt = torch.empty(rows, dtype=torch.int32, device=dev)
    toks = torch.tensor(W.first_tokens(rows, shape["vocab"]), dtype=torch.int32, device=dev)
    pos_all = [torch.tensor([prefill + i * M + j for b in range(B) for j in range(M)],
                            dtype=torch.int32, device=dev) for i in range(max(steps, warmup))]
    pbuf = torch.empty_like(pos_all[0])
    stream = torch.cuda.current_stream()
    out = {}
    for mode in modes:
        try:
            m.set_mode(mode)
        except ld.LdError as e:
            print(f"# tokens_per_seq={M} mode={mode} refused: {e}", file=sys.stderr, flush=True)
            continue
        ms = None
        for n, timed in ((warmup, False), (steps, True)):
            m.fill_kv(W.SEED_KV, 1.0, [prefill] * B + [1] * (rows - B))
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(n):
                pbuf.copy_(pos_all[i])
                m.step_tokens(toks, M, pbuf, logits, nxt)
            ev1.record(stream)
            torch.cuda.synchronize()
            if m.device_error() != 0:
                raise RuntimeError(f"device error with {M} tokens per sequence, mode {mode}")
            if timed:
                ms = ev0.elapsed_time(ev1) / n
        out[mode] = ms
        print(f"# tokens_per_seq={M} sequences={B} mode={mode} ms/step={ms:.4f} "
              f"tok/s={rows * 1000.0 / ms:.1f}", file=sys.stderr, flush=True)
    m.free()
    return out


def tune_tables(shape_name, batches, modes):
    """The offline SwiGLU tiling choice (ld_tune) at one shape: for each mode,
    whole decode steps with each tiling at every batch size (KV length 1024,
    or 512 at the Llama-1B shape); returns {mode: table} as ld_tune writes it."""
    import tempfile
    import torch
    from overlap_decode_step_amd import ld
    from synth import workloads as W
    shape = W.SHAPES[shape_name]
    w_std = W.WORKLOADS["llama70b"]["w_std"] if shape_name.startswith("llama70b") else 0.02
    prefill = 512 if shape_name == "llama1b" else 1024
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=w_std)
    m.alloc_kv(max(batches), prefill + 1)
    m.fill_kv(W.SEED_KV, 1.0, [prefill] * max(batches))
    out = {}
    for mode in modes:
        try:
            m.set_mode(mode)
        except ld.LdError as e:
            print(f"# tune mode={mode} refused: {e}", file=sys.stderr, flush=True)
            continue
        with tempfile.NamedTemporaryFile("r", suffix=".json") as f:
            ld.ld_tune(m.h, list(batches), f.name)
            out[mode] = json.loads(open(f.name).read())
        print(f"# tune {shape_name} mode={mode}: {json.dumps(out[mode])}", file=sys.stderr, flush=True)
    m.free()
    return out


def long_generation(batches=(1, 4, 16), prefills=(1024, 16384), modes=("wait", "flags", "mega"),
                    steps=4, warmup=2):
    """Long generation at the Llama-70B shape (80 layers, about 141 GB of
    bf16 weights, N(0, 0.01)) on one GPU: every sequence of the batch at KV
    length p, `steps` greedy steps timed after `warmup`, for each batch size,
    KV length and mode.  Returns rows of (batch, prefill, mode, ms per step,
    tokens/s, algorithmic bytes per step, fraction of 8 TB/s)."""
    import torch
    from overlap_decode_step_amd import ld
    from synth import workloads as W
    shape = W.LLAMA_70B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    maxb, maxs = max(batches), max(prefills) + steps + warmup + 8
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=W.WORKLOADS["llama70b"]["w_std"])
    m.alloc_kv(maxb, maxs)
    stream = torch.cuda.current_stream()
    rows = []
    for B in batches:
        logits = torch.empty((B, shape["vocab"]), dtype=torch.float32, device=dev)
        toks = torch.tensor(W.first_tokens(B, shape["vocab"]), dtype=torch.int32, device=dev)
        tbuf = [toks.clone(), torch.empty_like(toks)]
        for p in prefills:
            pos = [torch.full((B,), p + i, dtype=torch.int32, device=dev)
                   for i in range(steps + warmup)]
            for mode in modes:
                m.set_mode(mode)
                m.fill_kv(W.SEED_KV, 1.0, [p] * B + [0] * (maxb - B))
                tbuf[0].copy_(toks)
                for i in range(warmup):
                    m.step(tbuf[i & 1], pos[i], logits, tbuf[(i + 1) & 1])
                torch.cuda.synchronize()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for i in range(warmup, warmup + steps):
                    m.step(tbuf[i & 1], pos[i], logits, tbuf[(i + 1) & 1])
                ev1.record(stream)
                torch.cuda.synchronize()
                if m.device_error() != 0:
                    raise RuntimeError(f"device error at batch {B} KV {p} mode {mode}")
                ms = ev0.elapsed_time(ev1) / steps
                nbytes = sum(algorithmic_bytes(shape, B, [p + i] * B)
                             for i in range(warmup, warmup + steps)) / steps
                row = {"batch": B, "kv": p, "mode": mode, "ms_per_step": ms,
                       "tokens_per_s": B * 1000.0 / ms, "bytes_per_step": nbytes,
                       "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
                rows.append(row)
                print(f"# long-gen batch={B} kv={p} mode={mode} ms/step={ms:.3f} "
                      f"tok/s={row['tokens_per_s']:.1f} frac={row['hbm_frac']:.3f}",
                      file=sys.stderr, flush=True)
    m.free()
    return rows


def stage_trace(shape_name, B, prefill, modes, reps=3):
    """Per-stage timeline of one decode step (ld_set_trace): per layer, the time
    from the end of one stage (its last workgroup) to the end of the next,
    averaged over layers 1..L-1; the LM head; and the spread over workgroups
    of the attention items' events and of the SwiGLU stage's end.  Printed as
    text lines and returned as a dict."""
    import numpy as np
    import torch
    from overlap_decode_step_amd import ld
    from synth import workloads as W
    shape = W.SHAPES[shape_name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=0.01 if shape_name.startswith("llama70b") else 0.02)
    m.alloc_kv(B, prefill + reps + 8)
    m.fill_kv(W.SEED_KV, 1.0, [prefill] * B)
    L = shape["n_layers"]
    nbytes = ld.ld_trace_bytes(shape)
    tr = torch.zeros(nbytes // 8, dtype=torch.int64, device=dev)
    lg = torch.empty((B, shape["vocab"]), dtype=torch.float32, device=dev)
    nx = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.tensor(W.first_tokens(B, shape["vocab"]), dtype=torch.int32, device=dev)
    names = ["qkv", "attention", "o", "swiglu", "down"]
    out = {}
    for mode in modes:
        m.set_mode(mode)
        acc = []
        for rep in range(reps):
            pos = torch.full((B,), prefill + rep, dtype=torch.int32, device=dev)
            for _ in range(3):
                m.step(toks, pos, lg, nx)
            torch.cuda.synchronize()
            tr.zero_()
            ld.ld_set_trace(m.h, tr.data_ptr(), nbytes)
            m.step(toks, pos, lg, nx)
            torch.cuda.synchronize()
            ld.ld_set_trace(m.h, None, 0)
            if m.device_error() != 0:
                raise RuntimeError(f"device error in the traced step ({mode})")
            t = tr.cpu().numpy().reshape(L + 1, 8, 4, 1024).astype(np.float64)
            t0 = t[t > 0].min()
            t = np.where(t > 0, (t - t0) / 100.0, np.nan)  # microseconds (100 MHz clock)
            per = {k: [] for k in names}
            items = []
            gu_end = []
            for l in range(1, L):
                prev = np.nanmax(t[l - 1, 5, 3])
                for s_, k in enumerate(names, start=1):
                    end = np.nanmax(t[l, s_, 3])
                    per[k].append(end - prev)
                    prev = end
                qkv_end = np.nanmax(t[l, 1, 3])
                ev = [t[l, 6, 0], t[l, 7, 0], t[l, 7, 1], t[l, 7, 2], t[l, 7, 3], t[l, 2, 3]]
                items.append([np.nanmedian(e - qkv_end) if np.isfinite(e).any() else np.nan for e in ev]
                             + [np.nanmax(t[l, 2, 3]) - qkv_end])
                o_end = np.nanmax(t[l, 3, 3])
                ge = t[l, 4, 3] - o_end
                gu_end.append((np.nanmedian(ge), np.nanmax(ge)))
            lm = np.nanmax(t[L, 6, 3]) - np.nanmax(t[L - 1, 5, 3])
            acc.append((per, np.nanmean(items, axis=0), np.mean(gu_end, axis=0), lm))
        row = {k: float(np.mean([np.mean(a[0][k]) for a in acc])) for k in names}
        it = np.mean([a[1] for a in acc], axis=0)
        ge = np.mean([a[2] for a in acc], axis=0)
        lm = float(np.mean([a[3] for a in acc]))
        row["layer"] = sum(row[k] for k in names)
        row["lm_head"] = lm
        row["attention_items_us_after_qkv_end"] = {
            "item_start": float(it[0]), "tiles_ready": float(it[1]), "scores_done": float(it[2]),
            "outputs_stored": float(it[3]), "split_counter": float(it[4]),
            "stage_end_median": float(it[5]), "stage_end_last": float(it[6])}
        row["swiglu_end_after_o_us"] = {"median": float(ge[0]), "last": float(ge[1])}
        out[mode] = row
        print(f"# stage-trace {shape_name} batch={B} mode={mode} per-layer us: "
              + " ".join(f"{k}={row[k]:.2f}" for k in names)
              + f" layer={row['layer']:.2f} lm_head={lm:.1f}", file=sys.stderr, flush=True)
        print(f"#   attention (us after QKV's end, medians): item start {it[0]:.2f}, tiles "
              f"{it[1]:.2f}, scores {it[2]:.2f}, outputs stored {it[3]:.2f}, split counter "
              f"{it[4]:.2f}; stage end median {it[5]:.2f}, last {it[6]:.2f}", file=sys.stderr,
              flush=True)
        print(f"#   swiglu end after O's end: median {ge[0]:.2f} us, last {ge[1]:.2f} us",
              file=sys.stderr, flush=True)
    m.free()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="mega", choices=["wait", "flags", "mega", "graph"])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--all-modes", action="store_true", help="also time the other modes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=4, help="oracle steps in the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="also run the batch sweep (1, 4, 16, 64; KV ~U[256,1024]; every mode)")
    ap.add_argument("--shape", default="llama1b", choices=["llama1b", "llama8b", "llama70b", "llama70b_tp8"],
                    help="decoder shape (the 8B and 70B shapes skip the CPU baseline; "
                         "llama70b_tp8 is one GPU's 8-way tensor-parallel share of the 70B "
                         "shape, without the exchanges)")
    ap.add_argument("--tokens-per-seq", type=int, default=1,
                    help="several consecutive tokens per sequence per step (a prefill chunk): "
                         "times ld_decode_step_tokens in every mode instead of the decode step")
    ap.add_argument("--mlp-ablation", action="store_true",
                    help="also time the whole-kernel-wait step with the fused SwiGLU stage "
                         "against its two- and four-kernel unfused forms")
    ap.add_argument("--sync", default="auto", choices=["auto", "tile", "stage"],
                    help="readiness granularity of the tile-flag and persistent modes")
    ap.add_argument("--prefill", type=int, default=None,
                    help="KV prefill per sequence (default 512 for llama1b, else 1024)")
    ap.add_argument("--no-free", action="store_true",
                    help="leave the model to be freed at interpreter exit")
    ap.add_argument("--long-gen", action="store_true",
                    help="only run long generation at the Llama-70B shape (batch 1, 4, 16; "
                         "KV 1024 and 16384; whole-kernel-wait and persistent modes)")
    ap.add_argument("--tune", default=None,
                    help="only run the offline SwiGLU tiling choice at this shape for the "
                         "comma-separated batch sizes of --tune-batches, in every mode")
    ap.add_argument("--tune-batches", default="1,2,16,64")
    ap.add_argument("--stage-trace", action="store_true",
                    help="only trace one step per stage (ld_set_trace) at --shape/--batch "
                         "and print the per-layer breakdown, in each of --trace-modes")
    ap.add_argument("--trace-modes", default="mega,wait,flags")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stage_trace:
        prefill = args.prefill or (512 if args.shape == "llama1b" else 1024)
        rows = stage_trace(args.shape, args.batch, prefill, args.trace_modes.split(","))
        print(json.dumps({"stage_trace": args.shape, "batch": args.batch, "prefill": prefill,
                          "modes": rows}), flush=True)
        return
    if args.long_gen:
        rows = long_generation()
        print(json.dumps({"long_generation": "llama70b", "rows": rows}), flush=True)
        return
    if args.tune:
        batches = [int(b) for b in args.tune_batches.split(",")]
        tables = tune_tables(args.tune, batches, ["wait", "flags", "mega", "graph"])
        print(json.dumps({"swiglu_tuning": args.tune, "batches": batches, "tables": tables}),
              flush=True)
        return
    if args.tokens_per_seq > 1:
        M, B = args.tokens_per_seq, args.batch
        # (the persistent kernel is built for decode steps only)
        res = multi_token_bench(args.shape, B, M, args.steps, args.warmup,
                                ["wait", "flags", "graph"])
        best = min(v for v in res.values() if v is not None)
        print(json.dumps({
            "metric": f"prefill-chunk tokens/s, {args.shape} shape, {B} sequences x {M} tokens",
            "value": B * M * 1000.0 / best, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": best, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{args.shape}-shape, {B} sequences x {M} consecutive tokens "
                                   f"per step (teacher forced)", "tokens_per_seq": M, "batch": B},
            "modes_ms_per_step": res}), flush=True)
        return

    import torch

    from overlap_decode_step_amd import ld
    from synth import workloads as W

    shape = W.SHAPES[args.shape]
    w_std = W.WORKLOADS["llama70b"]["w_std"] if args.shape.startswith("llama70b") else 0.02
    headline = args.shape == "llama1b"
    B = args.batch
    prefill = args.prefill if args.prefill is not None else (512 if headline else 1024)
    steps, warmup = args.steps, args.warmup
    max_seq = prefill + max(steps, warmup) + 8
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=w_std)
    m.alloc_kv(B, max_seq)
    m.fill_kv(W.SEED_KV, 1.0, [prefill] * B)
    m.set_sync(args.sync)
    torch.cuda.synchronize()
    logits = torch.empty((B, shape["vocab"]), dtype=torch.float32, device=dev)
    toks = torch.tensor(W.first_tokens(B, shape["vocab"]), dtype=torch.int32, device=dev)
    pos_all = [torch.full((B,), prefill + i, dtype=torch.int32, device=dev)
               for i in range(max(steps, warmup))]
    # every kernel of a step is enqueued on this stream (the persistent kernel
    # and the whole-kernel-wait kernels; the tile-flag mode forks a second
    # stream and joins it back before the step returns)
    stream = torch.cuda.current_stream()

    # token buffers (ping-ponged) and, for graph mode, one position buffer:
    # fixed addresses, so that a captured step replays
    tbuf = [toks.clone(), torch.empty_like(toks)]
    pbuf = torch.empty_like(pos_all[0])

    def run(mode, n, timed):
        # greedy decode: the next tokens of step i are the inputs of step i + 1
        m.set_mode(mode)
        m.fill_kv(W.SEED_KV, 1.0, [prefill] * B)
        tbuf[0].copy_(toks)
        torch.cuda.synchronize()
        if timed:
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
        for i in range(n):
            if mode == "graph":
                pbuf.copy_(pos_all[i])  # in place, timed with the step
                m.step(tbuf[i & 1], pbuf, logits, tbuf[(i + 1) & 1])
            else:
                m.step(tbuf[i & 1], pos_all[i], logits, tbuf[(i + 1) & 1])
        if timed:
            ev1.record(stream)
        torch.cuda.synchronize()
        st = m.device_error()
        if st != 0:
            raise RuntimeError(f"device error {st} in mode {mode}")
        return ev0.elapsed_time(ev1) / n if timed else None

    results = {}
    modes = ["wait", "flags", "mega", "graph"] if args.all_modes else [args.mode]
    for mode in modes:
        if mode != args.mode:
            try:
                m.set_mode(mode)
            except ld.LdError as e:  # e.g. the tile-flag mode at the 70B width
                print(f"# mode={mode} batch={B} refused: {e}", file=sys.stderr, flush=True)
                continue
        run(mode, warmup, False)
        ms = run(mode, steps, True)
        results[mode] = ms
        print(f"# mode={mode} batch={B} ms/step={ms:.4f} tok/s={B * 1000.0 / ms:.1f}",
              file=sys.stderr, flush=True)
    ms = results[args.mode]
    ablation = None
    if args.mlp_ablation:
        ablation = {}
        for variant in ("fused", "two", "four"):
            m.set_mlp_variant(variant)
            run("wait", warmup, False)
            ablation[variant] = run("wait", steps, True)
            print(f"# mlp={variant} mode=wait batch={B} ms/step={ablation[variant]:.4f}",
                  file=sys.stderr, flush=True)
        m.set_mlp_variant("fused")
    if not args.no_free:
        m.free()
        del m
    torch.cuda.synchronize()
    positions = [prefill + i for i in range(steps)]
    bytes_avg = sum(algorithmic_bytes(shape, B, [p] * B) for p in positions) / steps
    # In the persistent mode one launch is one whole step, so the per-launch
    # duration is the timed region over the number of steps.
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    print(f"# kernel_source_digest={digest} algorithmic_bytes_per_step={bytes_avg:.0f}",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu and headline:
        cpu = cpu_baseline(shape, prefill, args.cpu_steps)
        print(f"# cpu_baseline {cpu}", file=sys.stderr, flush=True)
    sweep = batch_sweep() if args.sweep else None
    kernel = {"mega": "k_mega (persistent, one launch per step)",
              "wait": "all stage kernels of one step", "flags": "all stage kernels of one step",
              "graph": "all stage kernels of one step (graph replay)"}
    metric = "decode tokens/s + achieved HBM GB/s vs peak, Llama-1B shape, batch 1"
    if not (headline and B == 1):
        metric = f"decode tokens/s + achieved HBM GB/s vs peak, {args.shape} shape, batch {B}"
    out = {
        "metric": metric,
        "value": B * 1000.0 / ms,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.shape}-shape decode, batch {B}, KV prefill {prefill}, "
                               f"positions {prefill}..{prefill + steps - 1}",
                   "mode": args.mode, "batch": B, "sync": args.sync},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic(args.mode, B) if headline else None,
                     "kernel": kernel[args.mode], "algorithmic_bytes": bytes_avg},
        "cpu_baseline": cpu,
        "modes_ms_per_step": results,
    }
    if B >= MFMA_MIN_BATCH:
        # MFMA utilisation of the projections: algorithmic FLOPs / (time x
        # dense bf16 peak); the engine issues two MFMAs per product (the
        # activations as split-bf16 hi and lo parts), hence issued = 2 x
        proj = sum(algorithmic_flops(shape, B, [p] * B)[0] for p in positions) / steps
        tf = proj / (ms * 1e-3) / 1e12
        out["mfma"] = {"algorithmic_tflops": tf, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                       "util": tf / MFMA_BF16_PEAK_TFLOPS,
                       "issued_util": 2 * tf / MFMA_BF16_PEAK_TFLOPS,
                       "flops_per_step": proj}
    if sweep is not None:
        out["batch_sweep_tokens_per_s"] = sweep
    if ablation is not None:
        out["mlp_ablation_wait_ms_per_step"] = ablation
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
