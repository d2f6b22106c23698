"""Seeded synthetic workloads for the decode step: model shapes, generator
seeds and standard deviations, KV prefill lengths and first tokens.

This module describes inputs only; it holds none of the decode arithmetic.
It mirrors, in Python integers, the counter-based generator of ld_synth.h
(SplitMix64 output function; Irwin-Hall(4) for approximately normal values;
multiply-shift for uniform integers), so host code can draw the same first
tokens and KV lengths as the C side without linking either library.

Model shapes: a tiny 2-layer decoder for exhaustive checks, and decoders with
the shapes of Llama-3.2-1B (the single-sequence workload of Hazy Research,
"Look Ma, No Bubbles! Designing a Low-Latency Megakernel for Llama-1B",
introduction), Llama-3.1-8B (MegaOps summary, "Small shapes expose a limit")
and Llama-3.1-70B ("Deep Kernel Fusion for Transformers", Key points, "Setup";
MegaOps summary, "A multi-GPU check"), all with seeded random weights.
"""
import math

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

SEED_WEIGHTS, SEED_KV, SEED_TOKENS, SEED_KVLEN = 1, 2, 3, 4
T_EMBED, T_FINAL_NORM, T_LM_HEAD = 1, 2, 3
K_ATTN_NORM, K_WQ, K_WK, K_WV, K_WO, K_MLP_NORM, K_WG, K_WU, K_WD = range(9)
T_TOKENS = 0x200000
T_KVLEN = 0x200001


def t_layer(layer, kind):
    return 0x1000 + 16 * layer + kind


def t_kcache(layer):
    return 0x100000 + 2 * layer


def t_vcache(layer):
    return 0x100000 + 2 * layer + 1


def kv_index(b, n_kv, h, pos, d, i):
    return ((b * n_kv + h) << 32) + pos * d + i


def mix64(z):
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def key(seed, tensor):
    return mix64(seed ^ mix64((tensor * GAMMA + 0x632BE59BD9B4E019) & M64))


def hash64(k, index):
    return mix64((k + ((index + 1) * GAMMA)) & M64)


def uniform_int(k, index, lo, hi):
    h = hash64(k, index)
    span = hi - lo + 1
    return lo + (((h >> 32) * span) >> 32)


def irwin_hall4(h):
    return (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + ((h >> 48) & 0xFFFF) - 131070


def kappa(sigma):
    import numpy as np
    return float(np.float32(float(np.float32(sigma)) / math.sqrt((65536.0 * 65536.0 - 1.0) / 3.0)))


def normal_bf16(k, index, kap):
    """bf16 bits of one approximately-normal element (bit-exact with ld_synth.h)."""
    import numpy as np
    v = np.float32(irwin_hall4(hash64(k, index))) * np.float32(kap)
    u = int(np.array([v], dtype=np.float32).view(np.uint32)[0])
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFFFFFF
    return u >> 16


def first_tokens(batch, vocab, seed=SEED_TOKENS):
    k = key(seed, T_TOKENS)
    return [uniform_int(k, b, 0, vocab - 1) for b in range(batch)]


def kv_lengths(batch, lo, hi, seed=SEED_KVLEN):
    k = key(seed, T_KVLEN)
    return [uniform_int(k, b, lo, hi) for b in range(batch)]


def shape(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, tied,
          rms_eps=1e-5, rope_theta=500000.0):
    return dict(n_layers=n_layers, hidden=hidden, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, intermediate=intermediate, vocab=vocab, tied=tied,
                rms_eps=rms_eps, rope_theta=rope_theta)


# 2 layers, hidden 256, 4 Q / 2 KV heads of 64, SwiGLU 768, vocab 1024, untied.
TINY = shape(2, 256, 4, 2, 64, 768, 1024, 0, 1e-5, 10000.0)
# Llama-3.2-1B shape: tied embeddings, RoPE theta 500000.
LLAMA_1B = shape(16, 2048, 32, 8, 64, 8192, 128256, 1)
# Llama-3.1-8B shape.
LLAMA_8B = shape(32, 4096, 32, 8, 128, 14336, 128256, 0)
# Llama-3.1-70B shape (about 141 GB of bf16 weights on one GPU).
LLAMA_70B = shape(80, 8192, 64, 8, 128, 28672, 128256, 0)
# One GPU's share of the Llama-70B shape under 8-way tensor parallelism:
# 8 Q heads and 1 KV head of 128 (one whole GQA group), SwiGLU 3584 (an eighth
# of 28672), a 16032-row vocabulary shard; the residual stream stays 8192 wide.
LLAMA_70B_TP8 = shape(80, 8192, 8, 1, 128, 3584, 16032, 0)

SHAPES = {"tiny": TINY, "llama1b": LLAMA_1B, "llama8b": LLAMA_8B, "llama70b": LLAMA_70B,
          "llama70b_tp8": LLAMA_70B_TP8}

# Workloads: weights ~N(0, w_std) (norm gains 1.0), KV prefill ~N(0, 1).
WORKLOADS = {
    # tiny decoder: batch 1, KV prefilled for 128 positions, 16 greedy steps
    "tiny": dict(shape="tiny", w_std=0.02, kv_std=1.0, batches=[1], prefill=128, steps=16),
    # Llama-1B shape: batch 1, KV prefill 512, 128 greedy steps (positions 512..639)
    "llama1b_b1": dict(shape="llama1b", w_std=0.02, kv_std=1.0, batches=[1], prefill=512,
                       steps=128),
    # Llama-1B shape, short-context batch sweep: KV length ~U[256, 1024] per sequence, 64 steps
    "llama1b_sweep": dict(shape="llama1b", w_std=0.02, kv_std=1.0, batches=[1, 4, 16, 64],
                          prefill=(256, 1024), steps=64),
    # Llama-8B shape: KV length 1024, batch 1/2/16/64
    "llama8b": dict(shape="llama8b", w_std=0.02, kv_std=1.0, batches=[1, 2, 16, 64],
                    prefill=1024, steps=8),
    # Llama-70B shape on one GPU: KV 1024 -> 16384, batch 1/4/16
    "llama70b": dict(shape="llama70b", w_std=0.01, kv_std=1.0, batches=[1, 4, 16],
                     prefill=1024, steps=4),
    # the same at one GPU's 8-way tensor-parallel share (kernels at the shard's
    # shapes; the exchanges between GPUs are not part of it)
    "llama70b_tp8": dict(shape="llama70b_tp8", w_std=0.01, kv_std=1.0, batches=[1, 4, 16],
                         prefill=1024, steps=4),
}


def prefill_lengths(workload, batch):
    pf = WORKLOADS[workload]["prefill"]
    if isinstance(pf, tuple):
        return kv_lengths(batch, pf[0], pf[1])
    return [pf] * batch
