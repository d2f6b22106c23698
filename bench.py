"""Decode-step benchmark on one MI355X.

Default workload: the Llama-3.2-1B-shaped decoder (16 layers, hidden 2048,
32/8 heads of 64, SwiGLU 8192, vocab 128256, tied), batch 1, seeded KV
prefill of 512 positions, greedy decode (positions 512, 513, ...), seeded
random weights (synthetic data).  A step is one full decode step: every
layer and the LM head with greedy argmax, inputs resident in HBM.

Prints one JSON line: decode tokens/s (value), the roofline of the dominant
kernel (HBM bytes the step must move / its measured duration, against
8 TB/s), and the CPU oracle's rate on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="mega", choices=["wait", "flags", "mega"])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--all-modes", action="store_true", help="also time the other modes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from overlap_decode_step_amd import ld
    from synth import workloads as W

    shape = W.LLAMA_1B
    B = args.batch
    prefill = 512
    steps, warmup = args.steps, args.warmup
    max_seq = prefill + max(steps, warmup) + 8
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
    m.alloc_kv(B, max_seq)
    m.fill_kv(W.SEED_KV, 1.0, [prefill] * B)
    torch.cuda.synchronize()
    logits = torch.empty((B, shape["vocab"]), dtype=torch.float32, device=dev)
    toks = torch.tensor(W.first_tokens(B, shape["vocab"]), dtype=torch.int32, device=dev)
    pos_all = [torch.full((B,), prefill + i, dtype=torch.int32, device=dev)
               for i in range(max(steps, warmup))]
    stream = torch.cuda.current_stream()

    def run(mode, n, timed):
        # greedy decode: the next tokens of step i are the inputs of step i + 1
        m.set_mode(mode)
        tbuf = [toks.clone(), torch.empty_like(toks)]
        if timed:
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
        for i in range(n):
            m.step(tbuf[i & 1], pos_all[i], logits, tbuf[(i + 1) & 1])
        if timed:
            ev1.record(stream)
            torch.cuda.synchronize()
            st = m.device_error()
            if st != 0:
                raise RuntimeError(f"device error {st} in mode {mode}")
            return ev0.elapsed_time(ev1) / n
        torch.cuda.synchronize()
        return None

    results = {}
    modes = ["wait", "flags", "mega"] if args.all_modes else [args.mode]
    for mode in modes:
        run(mode, warmup, False)
        ms = run(mode, steps, True)
        results[mode] = ms
        print(f"# mode={mode} batch={B} ms/step={ms:.4f} tok/s={B * 1000.0 / ms:.1f}",
              file=sys.stderr, flush=True)
    ms = results[args.mode]
    positions = [prefill + i for i in range(steps)]
    bytes_avg = sum(algorithmic_bytes(shape, B, [p] * B) for p in positions) / steps
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode tokens/s + achieved HBM GB/s vs peak, Llama-1B shape, batch 1",
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
        "config": {"workload": f"llama1b-shape decode, batch {B}, KV prefill {prefill}, "
                               f"positions {prefill}..{prefill + steps - 1}",
                   "mode": args.mode, "batch": B},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "modes_ms_per_step": results,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
