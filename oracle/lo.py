"""ctypes front end of the CPU oracle (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this.
`Oracle('f32')` is the reference build (float arithmetic over bf16 weights);
`Oracle('f64')` is the same source built with double, used to bound the float
build's own rounding error.
"""
import ctypes
import os

import numpy as np

from . import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))

# weight kinds (ld_oracle.h)
W_EMBED, W_ATTN_NORM, W_Q, W_K, W_V, W_O, W_MLP_NORM, W_GATE, W_UP, W_DOWN, W_FINAL_NORM, \
    W_LM_HEAD = range(12)


class LoConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


def make_config(shape):
    return LoConfig(**shape)


_LIBS = {}


def _load(kind):
    if kind in _LIBS:
        return _LIBS[kind]
    path = _build.LIBS[kind][0]
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    P, I32, I64, U64, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                           ctypes.c_float)
    R = ctypes.c_float if kind == "f32" else ctypes.c_double
    sig = {
        "lo_real_bytes": (I32, []),
        "lo_bf16_round": (ctypes.c_uint16, [F]),
        "lo_bf16_widen": (F, [ctypes.c_uint16]),
        "lo_model_create": (P, [ctypes.POINTER(LoConfig)]),
        "lo_model_free": (None, [P]),
        "lo_model_synth": (ctypes.c_int, [P, U64, F]),
        "lo_weight": (P, [P, ctypes.c_int, ctypes.c_int, ctypes.POINTER(I64),
                          ctypes.POINTER(I64)]),
        "lo_kv_create": (P, [ctypes.POINTER(LoConfig), I32, I32]),
        "lo_kv_free": (None, [P]),
        "lo_kv_synth": (ctypes.c_int, [P, U64, F, P]),
        "lo_kv_synth_from": (ctypes.c_int, [P, U64, F, P, I32]),
        "lo_decode_one": (ctypes.c_int, [P, P, I32, I32, I32, P, P]),
        "lo_kv_k": (P, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "lo_kv_v": (P, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "lo_silu": (R, [R]),
        "lo_rmsnorm": (None, [P, P, I32, F, P]),
        "lo_matvec": (None, [P, I64, I64, P, P]),
        "lo_rope": (None, [P, I32, I32, F]),
        "lo_softmax": (None, [P, I32]),
        "lo_attention_head": (None, [P, P, P, I32, I32, P]),
        "lo_swiglu": (None, [P, P, I64, I64, P, P]),
        "lo_argmax": (I32, [P, I64]),
        "lo_decode_step": (ctypes.c_int, [P, P, P, I32, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIBS[kind] = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class LoTrace(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("layer", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("xn", "q", "k", "v", "o", "x_attn", "xn2", "hh", "x_out")]


class Oracle:
    """One oracle build: op-level functions plus model / KV-cache handles."""

    def __init__(self, kind="f32"):
        self.kind = kind
        self.lib = _load(kind)
        self.real = np.float32 if kind == "f32" else np.float64
        assert self.lib.lo_real_bytes() == np.dtype(self.real).itemsize

    # ---- ops
    def arr(self, a):
        return np.ascontiguousarray(a, dtype=self.real)

    def bf16_round(self, f):
        return int(self.lib.lo_bf16_round(float(f)))

    def bf16_widen(self, b):
        return float(self.lib.lo_bf16_widen(int(b)))

    def silu(self, a):
        return float(self.lib.lo_silu(float(a)))

    def rmsnorm(self, x, g=None, eps=1e-5):
        x = self.arr(x)
        out = np.empty_like(x)
        gbuf = None if g is None else np.ascontiguousarray(g, dtype=np.uint16)
        gp = None if gbuf is None else _ptr(gbuf)
        self.lib.lo_rmsnorm(_ptr(x), gp, x.size, eps, _ptr(out))
        return out

    def matvec(self, W_bf16, x):
        W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
        x = self.arr(x)
        y = np.empty(W.shape[0], dtype=self.real)
        self.lib.lo_matvec(_ptr(W), W.shape[0], W.shape[1], _ptr(x), _ptr(y))
        return y

    def rope(self, h, p, theta):
        h = self.arr(h).copy()
        self.lib.lo_rope(_ptr(h), h.size, int(p), float(theta))
        return h

    def softmax(self, s):
        s = self.arr(s).copy()
        self.lib.lo_softmax(_ptr(s), s.size)
        return s

    def attention_head(self, q, K_bf16, V_bf16):
        q = self.arr(q)
        K = np.ascontiguousarray(K_bf16, dtype=np.uint16)
        V = np.ascontiguousarray(V_bf16, dtype=np.uint16)
        out = np.empty(q.size, dtype=self.real)
        self.lib.lo_attention_head(_ptr(q), _ptr(K), _ptr(V), K.shape[0], q.size, _ptr(out))
        return out

    def swiglu(self, Wg, Wu, xn):
        Wg = np.ascontiguousarray(Wg, dtype=np.uint16)
        Wu = np.ascontiguousarray(Wu, dtype=np.uint16)
        xn = self.arr(xn)
        h = np.empty(Wg.shape[0], dtype=self.real)
        self.lib.lo_swiglu(_ptr(Wg), _ptr(Wu), Wg.shape[0], Wg.shape[1], _ptr(xn), _ptr(h))
        return h

    def argmax(self, v):
        v = self.arr(v)
        return int(self.lib.lo_argmax(_ptr(v), v.size))

    # ---- model
    def model(self, shape, seed=None, w_std=0.02):
        return OracleModel(self, shape, seed, w_std)

    def kv(self, shape, max_batch, max_seq, seed=None, kv_std=1.0, prefill=None, seq0=0):
        return OracleKV(self, shape, max_batch, max_seq, seed, kv_std, prefill, seq0)

    def decode_one(self, model, kv, seq, token, pos):
        """Decode one cache slot only; returns (logits [vocab] float32, next token)."""
        logits = np.empty(model.shape["vocab"], dtype=np.float32)
        nxt = np.empty(1, dtype=np.int32)
        rc = self.lib.lo_decode_one(model.h, kv.h, seq, int(token), int(pos), _ptr(logits),
                                    _ptr(nxt))
        if rc != 0:
            raise ValueError("lo_decode_one rejected its arguments")
        return logits, int(nxt[0])

    def decode_step(self, model, kv, tokens, pos, trace=None):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        B = tokens.size
        logits = np.empty((B, model.shape["vocab"]), dtype=np.float32)
        nxt = np.empty(B, dtype=np.int32)
        tp = None
        if trace is not None:
            tp = ctypes.byref(trace.struct)
        rc = self.lib.lo_decode_step(model.h, kv.h, _ptr(tokens), B, _ptr(pos), _ptr(logits),
                                     _ptr(nxt), tp)
        if rc != 0:
            raise ValueError("lo_decode_step rejected its arguments")
        return logits, nxt

    def trace(self, shape, seq=0, layer=0):
        return Trace(self, shape, seq, layer)


class Trace:
    def __init__(self, orc, shape, seq, layer):
        H, d = shape["hidden"], shape["head_dim"]
        nq, nkv, inter = shape["n_q_heads"], shape["n_kv_heads"], shape["intermediate"]
        sizes = dict(xn=H, q=nq * d, k=nkv * d, v=nkv * d, o=nq * d, x_attn=H, xn2=H, hh=inter,
                     x_out=H)
        self.bufs = {n: np.zeros(s, dtype=orc.real) for n, s in sizes.items()}
        self.struct = LoTrace(seq, layer, *[_ptr(self.bufs[n]).value for n in (
            "xn", "q", "k", "v", "o", "x_attn", "xn2", "hh", "x_out")])

    def __getitem__(self, k):
        return self.bufs[k]


class OracleModel:
    def __init__(self, orc, shape, seed, w_std):
        self.orc, self.shape = orc, dict(shape)
        self.cfg = make_config(shape)
        self.h = orc.lib.lo_model_create(ctypes.byref(self.cfg))
        if not self.h:
            raise MemoryError("lo_model_create failed")
        if seed is not None:
            orc.lib.lo_model_synth(self.h, seed, w_std)

    def weight(self, kind, layer=0):
        r, c = ctypes.c_int64(), ctypes.c_int64()
        p = self.orc.lib.lo_weight(self.h, kind, layer, ctypes.byref(r), ctypes.byref(c))
        if not p:
            raise IndexError("no such weight")
        buf = (ctypes.c_uint16 * (r.value * c.value)).from_address(p)
        return np.ctypeslib.as_array(buf).reshape(r.value, c.value)

    def __del__(self):
        if getattr(self, "h", None):
            self.orc.lib.lo_model_free(self.h)
            self.h = None


class OracleKV:
    def __init__(self, orc, shape, max_batch, max_seq, seed, kv_std, prefill, seq0=0):
        self.orc, self.shape = orc, dict(shape)
        self.max_batch, self.max_seq = max_batch, max_seq
        self.cfg = make_config(shape)
        self.h = orc.lib.lo_kv_create(ctypes.byref(self.cfg), max_batch, max_seq)
        if not self.h:
            raise MemoryError("lo_kv_create failed")
        if seed is not None:
            pf = np.ascontiguousarray(prefill, dtype=np.int32)
            assert pf.size == max_batch
            if orc.lib.lo_kv_synth_from(self.h, seed, kv_std, _ptr(pf), seq0) != 0:
                raise ValueError("lo_kv_synth rejected prefill lengths")

    def _view(self, fn, layer, seq, head):
        p = fn(self.h, layer, seq, head)
        if not p:
            raise IndexError("no such cache slot")
        n = self.max_seq * self.shape["head_dim"]
        buf = (ctypes.c_uint16 * n).from_address(p)
        return np.ctypeslib.as_array(buf).reshape(self.max_seq, self.shape["head_dim"])

    def k(self, layer, seq, head):
        return self._view(self.orc.lib.lo_kv_k, layer, seq, head)

    def v(self, layer, seq, head):
        return self._view(self.orc.lib.lo_kv_v, layer, seq, head)

    def __del__(self):
        if getattr(self, "h", None):
            self.orc.lib.lo_kv_free(self.h)
            self.h = None


def bf16_to_f32(a):
    """Widen bf16 bit patterns (uint16 array) to float32 (numpy, for tests)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
