"""CPU checks of the C ABI: libld.so loads, exports every function that
include/*.h declares, and its host-only helpers (sizes, argument checks)
behave; no GPU work is launched here."""
import ctypes
import os
import re

import pytest

from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "overlap_decode_step_amd", "libld.so")


def declared_functions():
    names = set()
    for h in ("ld.h", "ld_ops.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(ld_\w+)\s*\(", txt, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from overlap_decode_step_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 20, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_abi():
    import overlap_decode_step_amd.ld as b
    missing = [n for n in declared_functions() if not hasattr(b, n)]
    assert not missing, missing


def weights_logical_bytes(s):
    H, V, I, L = s["hidden"], s["vocab"], s["intermediate"], s["n_layers"]
    qd, kvd = s["n_q_heads"] * s["head_dim"], s["n_kv_heads"] * s["head_dim"]
    per_layer = 2 * H + (qd + 2 * kvd) * H + H * qd + 3 * I * H
    return 2 * (V * H * (1 if s["tied"] else 2) + H + L * per_layer)


@pytest.mark.parametrize("name", ["tiny", "llama1b", "llama8b", "llama70b"])
def test_weight_arena_size(name):
    from overlap_decode_step_amd import ld
    s = W.SHAPES[name]
    n = ld.ld_weights_bytes(s)
    logical = weights_logical_bytes(s)
    assert logical <= n <= logical + 256 * (3 + 7 * s["n_layers"])
    if name == "llama1b":
        assert logical == 2_471_628_800  # bf16 weights incl. norm gains


def test_kv_arena_size_and_limits():
    from overlap_decode_step_amd import ld
    s = W.LLAMA_1B
    n = ld.ld_kv_bytes(s, 1, 640)
    cache = 2 * 16 * 1 * 8 * 640 * 64 * 2
    assert cache < n < cache + 64 * 2 ** 20
    assert ld.ld_kv_bytes(s, 65, 640) == 0
    assert ld.ld_kv_bytes(s, 0, 640) == 0
    assert ld.ld_weights_bytes(dict(s, hidden=2047)) == 0
    assert ld.ld_weights_bytes(dict(s, n_kv_heads=7)) == 0


def test_host_rejects_bad_arguments_without_gpu_work():
    from overlap_decode_step_amd import ld
    with pytest.raises(ld.LdError) as e:
        ld.ld_init_weights(dict(W.TINY, head_dim=12), None, 0, 1, 0.02, 0)
    assert e.value.status == ld.LD_EINVAL
    assert "config" in ld.ld_last_error(None)
    assert ld.LIB.ld_decode_step(None, None, 1, None, None, None, None) == ld.LD_EINVAL
    assert ld.LIB.ld_set_mode(None, 0) == ld.LD_EINVAL
    assert ld.LIB.ld_device_error(None) == ld.LD_EINVAL
