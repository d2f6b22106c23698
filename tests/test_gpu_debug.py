"""Debug mechanisms of libld.so through the C ABI: NaN poison before a step,
the post-step counter audit, and the environment overrides of a new model.

A poisoned step fills every activation, partial-result and hand-off buffer,
the logits and next tokens, and the KV-cache rows the step appends with NaN
first; a stage that read a word before its producer wrote it would spread
NaN to the logits.  So each case checks that the poisoned step returns
exactly the logits of the plain one, in every mode, and that the readiness
counters match what the host enqueued.
"""
import numpy as np
import pytest

from gpu_util import GpuRunner
from synth import workloads as W

pytestmark = pytest.mark.gpu

MODES = ("wait", "flags", "mega", "graph")
# hidden 136, n_q d 48 and intermediate 200: no MFMA fragment buffer of this
# shape is poisoned (their K is not a multiple of 32)
RAGGED = W.shape(3, 136, 6, 2, 8, 200, 1000, 0, 1e-5, 10000.0)
SHAPES = {"tiny": W.TINY, "ragged": RAGGED, "llama1b": W.SHAPES["llama1b"]}


@pytest.fixture(scope="module")
def ld():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    from overlap_decode_step_amd import ld as _ld
    return _ld


def _model(ld, shape, B, max_seq, prefill, w_std=0.02):
    m = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=w_std)
    m.alloc_kv(B, max_seq)
    m.fill_kv(W.SEED_KV, 1.0, prefill)
    return m


# batch sizes of both engines, ragged batch tiles, and the ragged shape
POISON_CASES = [("tiny", 1), ("tiny", 5), ("tiny", 16), ("tiny", 45), ("ragged", 3),
                ("llama1b", 1), ("llama1b", 16), ("llama1b", 64),
                ("tiny-long", 1), ("tiny-long", 3), ("tiny-long", 16)]


@pytest.mark.parametrize("name,B", POISON_CASES, ids=[f"{n}-B{b}" for n, b in POISON_CASES])
def test_poison_changes_nothing_and_counters_audit(ld, name, B):
    shape = SHAPES["tiny" if name == "tiny-long" else name]
    if name == "llama1b":
        maxs, prefill = 1040, W.kv_lengths(B, 256, 1024)
    elif name == "tiny-long":
        # 1900..2050 positions: more than 16 splits per head, so the step
        # combines its splits in a phase of its own
        maxs, prefill = 2100, W.kv_lengths(B, 1900, 2050)
    elif name == "ragged":
        maxs, prefill = 1200, [1100, 512, 1][:B]
    else:
        maxs, prefill = 256, W.kv_lengths(B, 1, 200)
    w_std = 0.05 if name == "ragged" else 0.02
    m = _model(ld, shape, B, maxs, prefill, w_std)
    run = GpuRunner(m, shape["vocab"], B)
    toks = W.first_tokens(B, shape["vocab"])
    for mode in MODES:
        m.set_mode(mode)
        m.set_debug(0)
        m.fill_kv(W.SEED_KV, 1.0, prefill)
        lg0, nx0 = run.step(toks, prefill)
        assert m.audit() == ld.LD_OK, f"{name} B={B} mode={mode}: " + ld.ld_last_error(m.h)
        m.set_debug(ld.LD_DEBUG_POISON)
        for rep in range(2):  # twice: the second also follows a poisoned step
            m.fill_kv(W.SEED_KV, 1.0, prefill)
            lg1, nx1 = run.step(toks, prefill)
            assert m.audit() == ld.LD_OK, f"{name} B={B} mode={mode}: " + ld.ld_last_error(m.h)
            assert np.isfinite(lg1).all(), f"{name} B={B} mode={mode}: a stage read poisoned data"
            assert np.array_equal(lg0, lg1), f"{name} B={B} mode={mode}: poison changed the logits"
            assert np.array_equal(nx0, nx1)
        m.set_debug(0)
        print(f"{name} B={B} mode={mode}: poisoned step bitwise equal, audit clean", flush=True)
    m.free()


@pytest.mark.parametrize("mode", ["flags", "mega"])
def test_audit_reports_a_stalled_step(ld, mode):
    # A step whose attention wait the host made unreachable ends at the
    # watchdog: the audit reports it (the error word, and counters off the
    # host's totals) until ld_device_error resets both; then it is clean.
    import torch
    shape = W.TINY
    m = _model(ld, shape, 1, 256, [128])
    m.set_mode(mode)
    ld.ld_set_watchdog(m.h, 0.05)
    run = GpuRunner(m, shape["vocab"], 1)
    run.step([5], [128])
    assert m.audit() == ld.LD_OK, ld.ld_last_error(m.h)
    ld.ld_debug_inject_stall(m.h)
    dev = torch.device("cuda:0")
    lg = torch.empty((1, shape["vocab"]), dtype=torch.float32, device=dev)
    m.step(torch.tensor([5], dtype=torch.int32, device=dev),
           torch.tensor([129], dtype=torch.int32, device=dev), lg)
    torch.cuda.synchronize()
    assert m.audit() == ld.LD_EAUDIT
    assert "expected" in ld.ld_last_error(m.h)
    assert m.device_error() == ld.LD_ETIMEOUT
    m.fill_kv(W.SEED_KV, 1.0, [128])
    run.step([5], [128])
    assert m.audit() == ld.LD_OK, ld.ld_last_error(m.h)
    m.free()


def test_poison_reaches_unwritten_rows(ld):
    # A one-row step on a two-row model writes row 0 of the residual stream
    # only: after a poisoned step row 1 reads back as NaN, after a plain one
    # it keeps its previous (finite) value.
    m = _model(ld, W.TINY, 2, 64, [8, 8])
    run = GpuRunner(m, W.TINY["vocab"], 2)
    run.step([3, 4], [8, 8])
    run.step([3], [8])
    x = m.read_activation(ld.LD_ACT_X, 2)
    assert np.isfinite(x).all()
    m.set_debug(ld.LD_DEBUG_POISON)
    run.step([3], [8])
    x = m.read_activation(ld.LD_ACT_X, 2)
    assert np.isfinite(x[0]).all() and np.isnan(x[1]).all()
    with pytest.raises(ld.LdError):
        ld.ld_set_debug(m.h, 2)
    m.free()


def test_environment_overrides(ld, monkeypatch):
    monkeypatch.setenv("LD_MODE", "wait")
    monkeypatch.setenv("LD_WATCHDOG_US", "50000")
    m = _model(ld, W.TINY, 1, 64, [8])
    assert ld.ld_launch_info(m.h)["mode"] == ld.LD_MODE_WAIT
    run = GpuRunner(m, W.TINY["vocab"], 1)
    run.step([3], [8])
    m.free()
    monkeypatch.setenv("LD_MODE", "graph")
    m = _model(ld, W.TINY, 1, 64, [8])
    assert ld.ld_launch_info(m.h)["mode"] == ld.LD_MODE_GRAPH
    m.free()
    for var, val in (("LD_MODE", "fast"), ("LD_WATCHDOG_US", "abc"), ("LD_WATCHDOG_US", "-5")):
        monkeypatch.setenv("LD_MODE", "mega")
        monkeypatch.setenv("LD_WATCHDOG_US", "50000")
        monkeypatch.setenv(var, val)
        with pytest.raises(ld.LdError):
            ld.Model(W.TINY, seed=W.SEED_WEIGHTS, w_std=0.02)
