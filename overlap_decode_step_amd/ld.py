"""Thin ctypes binding of libld.so (include/ld.h, include/ld_ops.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libld.so.  PyTorch supplies device memory and streams.  Importing
this module fails loudly when the library has not been built.
"""
import atexit
import ctypes
import os
import weakref

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libld.so")

LD_OK, LD_EINVAL, LD_ENOMEM, LD_EHIP, LD_ETIMEOUT, LD_ESTATE, LD_EDEVICE, LD_EAUDIT = (
    0, -1, -2, -3, -4, -5, -6, -7)
LD_DEBUG_POISON = 1
LD_MODE_WAIT, LD_MODE_FLAGS, LD_MODE_MEGA, LD_MODE_GRAPH = 0, 1, 2, 3
MODES = {"wait": LD_MODE_WAIT, "flags": LD_MODE_FLAGS, "mega": LD_MODE_MEGA, "graph": LD_MODE_GRAPH}
LD_SWIGLU_COL, LD_SWIGLU_ROW = 0, 1
LD_ACT_X, LD_ACT_QKV, LD_ACT_ATTN, LD_ACT_H = 0, 1, 2, 3
LD_SYNC_STAGE, LD_SYNC_TILE, LD_SYNC_AUTO = 0, 1, 2
SYNC = {"stage": LD_SYNC_STAGE, "tile": LD_SYNC_TILE, "auto": LD_SYNC_AUTO}
LD_MLP_FUSED, LD_MLP_TWO_KERNELS, LD_MLP_FOUR_KERNELS = 0, 1, 2
MLP_VARIANTS = {"fused": LD_MLP_FUSED, "two": LD_MLP_TWO_KERNELS, "four": LD_MLP_FOUR_KERNELS}
(LD_W_EMBED, LD_W_ATTN_NORM, LD_W_Q, LD_W_K, LD_W_V, LD_W_O, LD_W_MLP_NORM, LD_W_GATE, LD_W_UP,
 LD_W_DOWN, LD_W_FINAL_NORM, LD_W_LM_HEAD) = range(12)


class LdConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class LdError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, F, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_float, ctypes.c_double)
    S = ctypes.c_int
    CP = ctypes.POINTER(LdConfig)
    sig = {
        "ld_weights_bytes": (ctypes.c_size_t, [CP]),
        "ld_init_weights": (S, [ctypes.POINTER(P), CP, P, ctypes.c_size_t, U64, F, P]),
        "ld_kv_bytes": (ctypes.c_size_t, [CP, I32, I32]),
        "ld_alloc_kv": (S, [P, P, ctypes.c_size_t, I32, I32]),
        "ld_fill_kv": (S, [P, U64, F, P, P]),
        "ld_fill_kv_static": (S, [P, U64, F, P, P]),
        "ld_set_mode": (S, [P, S]),
        "ld_decode_step": (S, [P, P, I32, P, P, P, P]),
        "ld_decode_step_tokens": (S, [P, P, I32, I32, P, P, P, P]),
        "ld_tune": (S, [P, P, I32, ctypes.c_char_p]),
        "ld_load_tuning": (S, [P, ctypes.c_char_p]),
        "ld_device_error": (S, [P]),
        "ld_last_error": (ctypes.c_char_p, [P]),
        "ld_free": (None, [P]),
        "ld_weight_shape": (S, [P, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "ld_read_weight": (S, [P, I32, I32, P]),
        "ld_write_weight": (S, [P, I32, I32, P]),
        "ld_read_kv": (S, [P, I32, I32, I32, I32, I32, P, P]),
        "ld_set_swiglu_variant": (S, [P, I32, I32]),
        "ld_set_mlp_variant": (S, [P, I32]),
        "ld_get_swiglu_variant": (I32, [P, I32]),
        "ld_set_watchdog": (S, [P, D]),
        "ld_set_sync": (S, [P, I32]),
        "ld_debug_inject_stall": (S, [P]),
        "ld_set_debug": (S, [P, I32]),
        "ld_audit": (S, [P]),
        "ld_launch_info": (S, [P, P, I32]),
        "ld_read_activation": (S, [P, I32, I32, P]),
        "ld_trace_bytes": (ctypes.c_size_t, [CP]),
        "ld_set_trace": (S, [P, P, ctypes.c_size_t]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _check(st, m=None):
    if st != LD_OK:
        raise LdError(st, LIB.ld_last_error(m).decode())
    return st


def _cfg(shape):
    return shape if isinstance(shape, LdConfig) else LdConfig(**shape)


# ---- functions with the ABI's names (pointers are ints: data_ptr() values)

def ld_weights_bytes(shape):
    return int(LIB.ld_weights_bytes(ctypes.byref(_cfg(shape))))


def ld_init_weights(shape, dev_buf, nbytes, seed, w_std, stream=0):
    h = ctypes.c_void_p()
    _check(LIB.ld_init_weights(ctypes.byref(h), ctypes.byref(_cfg(shape)), dev_buf, nbytes, seed,
                               w_std, stream))
    return h.value


def ld_kv_bytes(shape, max_batch, max_seq):
    return int(LIB.ld_kv_bytes(ctypes.byref(_cfg(shape)), max_batch, max_seq))


def ld_alloc_kv(m, dev_buf, nbytes, max_batch, max_seq):
    return _check(LIB.ld_alloc_kv(m, dev_buf, nbytes, max_batch, max_seq), m)


def ld_fill_kv(m, seed, kv_std, prefill_len, stream=0):
    arr = (ctypes.c_int32 * len(prefill_len))(*prefill_len)
    return _check(LIB.ld_fill_kv(m, seed, kv_std, arr, stream), m)


def ld_fill_kv_static(m, seed, kv_std, prefill_len, stream=0):
    arr = (ctypes.c_int32 * len(prefill_len))(*prefill_len)
    return _check(LIB.ld_fill_kv_static(m, seed, kv_std, arr, stream), m)


def ld_set_mode(m, mode):
    return _check(LIB.ld_set_mode(m, MODES.get(mode, mode)), m)


def ld_decode_step(m, tokens, batch, positions, logits, next_tokens, stream=0):
    return _check(LIB.ld_decode_step(m, tokens, batch, positions, logits, next_tokens, stream), m)


def ld_decode_step_tokens(m, tokens, tokens_per_seq, batch, positions, logits, next_tokens,
                          stream=0):
    return _check(LIB.ld_decode_step_tokens(m, tokens, tokens_per_seq, batch, positions, logits,
                                            next_tokens, stream), m)


def ld_tune(m, batches, table_path=None):
    arr = (ctypes.c_int32 * len(batches))(*batches)
    return _check(LIB.ld_tune(m, arr, len(batches),
                              table_path.encode() if table_path else None), m)


def ld_load_tuning(m, table_path):
    return _check(LIB.ld_load_tuning(m, table_path.encode()), m)


def ld_device_error(m):
    """Status code of the device error word (cleared); does not raise."""
    return int(LIB.ld_device_error(m))


def ld_last_error(m=None):
    return LIB.ld_last_error(m).decode()


def ld_free(m):
    LIB.ld_free(m)


def ld_weight_shape(m, kind, layer=0):
    r, c = ctypes.c_int64(), ctypes.c_int64()
    _check(LIB.ld_weight_shape(m, kind, layer, ctypes.byref(r), ctypes.byref(c)), m)
    return r.value, c.value


def ld_read_weight(m, kind, layer, host_ptr):
    return _check(LIB.ld_read_weight(m, kind, layer, host_ptr), m)


def ld_write_weight(m, kind, layer, host_ptr):
    return _check(LIB.ld_write_weight(m, kind, layer, host_ptr), m)


def ld_read_kv(m, layer, seq, kv_head, pos0, npos, k_ptr, v_ptr):
    return _check(LIB.ld_read_kv(m, layer, seq, kv_head, pos0, npos, k_ptr, v_ptr), m)


def ld_set_swiglu_variant(m, batch, variant):
    return _check(LIB.ld_set_swiglu_variant(m, batch, variant), m)


def ld_set_mlp_variant(m, variant):
    return _check(LIB.ld_set_mlp_variant(m, MLP_VARIANTS.get(variant, variant)), m)


def ld_get_swiglu_variant(m, batch):
    return int(LIB.ld_get_swiglu_variant(m, batch))


def ld_set_sync(m, granularity):
    return _check(LIB.ld_set_sync(m, SYNC.get(granularity, granularity)), m)


def ld_set_watchdog(m, seconds):
    return _check(LIB.ld_set_watchdog(m, seconds), m)


def ld_debug_inject_stall(m):
    return _check(LIB.ld_debug_inject_stall(m), m)


def ld_set_debug(m, flags):
    return _check(LIB.ld_set_debug(m, flags), m)


def ld_audit(m):
    """LD_OK or LD_EAUDIT (the mismatches in ld_last_error); does not raise."""
    return int(LIB.ld_audit(m))


def ld_trace_bytes(shape):
    return int(LIB.ld_trace_bytes(ctypes.byref(_cfg(shape))))


def ld_set_trace(m, dev_buf, nbytes):
    return _check(LIB.ld_set_trace(m, dev_buf, nbytes), m)


def ld_read_activation(m, which, rows, host_ptr):
    return _check(LIB.ld_read_activation(m, which, rows, host_ptr), m)


def ld_launch_info(m):
    out = (ctypes.c_int32 * 6)()
    _check(LIB.ld_launch_info(m, out, 6), m)
    keys = ("n_cu", "grid_wait", "grid_flags", "grid_mega_b1", "split_len", "mode")
    return dict(zip(keys, list(out)))


# ---- convenience owner of the device buffers (torch for memory and streams)

# Models still alive when the interpreter exits are freed by an exit hook,
# before Python tears its modules down.  Left to garbage collection during
# that teardown, ld_free (a device synchronisation, stream, event and graph
# destruction) could run after the HIP runtime, or a profiler attached to
# it, had already shut down.  The hook is registered when the first model
# is made, after torch has registered its own, so it runs before them (exit
# hooks run last-in, first-out).
_LIVE = weakref.WeakSet()
_HOOKED = []


def _free_live_models():
    for m in list(_LIVE):
        m.free()

class Model:
    """A model whose weight and KV arenas are torch uint8 buffers on cuda:0."""

    def __init__(self, shape, seed=1, w_std=0.02, device="cuda"):
        import torch
        self.torch = torch
        self.shape = dict(shape) if not isinstance(shape, LdConfig) else shape
        self.device = device
        n = ld_weights_bytes(shape)
        if n == 0:
            raise LdError(LD_EINVAL, "unsupported shape")
        self.wbuf = torch.empty(n, dtype=torch.uint8, device=device)
        self.h = ld_init_weights(shape, self.wbuf.data_ptr(), n, seed, w_std, self.stream())
        if not _HOOKED:
            atexit.register(_free_live_models)
            _HOOKED.append(True)
        _LIVE.add(self)
        self.kbuf = None
        self.max_batch = self.max_seq = 0

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def alloc_kv(self, max_batch, max_seq):
        n = ld_kv_bytes(self.shape, max_batch, max_seq)
        self.kbuf = self.torch.empty(n, dtype=self.torch.uint8, device=self.device)
        self.torch.cuda.synchronize()
        ld_alloc_kv(self.h, self.kbuf.data_ptr(), n, max_batch, max_seq)
        self.max_batch, self.max_seq = max_batch, max_seq

    def fill_kv(self, seed, kv_std, prefill):
        ld_fill_kv(self.h, seed, kv_std, list(prefill), self.stream())

    def set_mode(self, mode):
        ld_set_mode(self.h, mode)

    def set_sync(self, granularity):
        ld_set_sync(self.h, granularity)

    def set_mlp_variant(self, variant):
        ld_set_mlp_variant(self.h, variant)

    def set_debug(self, flags):
        ld_set_debug(self.h, flags)

    def audit(self):
        return ld_audit(self.h)

    def step(self, tokens, positions, logits, next_tokens=None):
        """tokens/positions: cuda int32 [B]; logits: cuda float32 [B, vocab]."""
        B = int(tokens.numel())
        ld_decode_step(self.h, tokens.data_ptr(), B, positions.data_ptr(), logits.data_ptr(),
                       next_tokens.data_ptr() if next_tokens is not None else None, self.stream())

    def step_tokens(self, tokens, tokens_per_seq, positions, logits, next_tokens=None):
        """tokens/positions: cuda int32 [B * M] (row b * M + j: token j of
        sequence b); logits: cuda float32 [B * M, vocab]."""
        rows = int(tokens.numel())
        ld_decode_step_tokens(self.h, tokens.data_ptr(), tokens_per_seq, rows // tokens_per_seq,
                              positions.data_ptr(), logits.data_ptr(),
                              next_tokens.data_ptr() if next_tokens is not None else None,
                              self.stream())

    def device_error(self):
        return ld_device_error(self.h)

    def read_weight(self, kind, layer=0):
        import numpy as np
        r, c = ld_weight_shape(self.h, kind, layer)
        out = np.empty((r, c), dtype=np.uint16)
        ld_read_weight(self.h, kind, layer, out.ctypes.data)
        return out

    def write_weight(self, kind, layer, arr):
        import numpy as np
        r, c = ld_weight_shape(self.h, kind, layer)
        a = np.ascontiguousarray(arr, dtype=np.uint16).reshape(r, c)
        ld_write_weight(self.h, kind, layer, a.ctypes.data)

    def read_kv(self, layer, seq, kv_head, pos0, npos):
        import numpy as np
        d = self.shape["head_dim"]
        k = np.empty((npos, d), dtype=np.uint16)
        v = np.empty((npos, d), dtype=np.uint16)
        ld_read_kv(self.h, layer, seq, kv_head, pos0, npos, k.ctypes.data, v.ctypes.data)
        return k, v

    def read_activation(self, which, rows):
        import numpy as np
        s = self.shape
        qd, kvd = s["n_q_heads"] * s["head_dim"], s["n_kv_heads"] * s["head_dim"]
        width = {LD_ACT_X: s["hidden"], LD_ACT_QKV: qd + 2 * kvd, LD_ACT_ATTN: qd,
                 LD_ACT_H: s["intermediate"]}[which]
        out = np.empty((rows, width), dtype=np.float32)
        ld_read_activation(self.h, which, rows, out.ctypes.data)
        return out

    def free(self):
        if getattr(self, "h", None):
            ld_free(self.h)
            self.h = None

    def __del__(self):
        self.free()
