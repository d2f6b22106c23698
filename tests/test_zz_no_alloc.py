"""The allocation-free KV fill (ld_fill_kv_static) against ld_fill_kv.

Both fill positions [0, len[b]) of every (layer, sequence, kv head) with the
same seeded values; the allocation-free variant keeps the device copy of the
lengths in the library's static device array instead of a buffer from
hipMalloc.  Two calls in a row, the second with fewer sequences and shorter
lengths, so the shared array still holds the first call's longer list when
the second starts.
"""
import numpy as np
import pytest

from synth import workloads as W

pytestmark = pytest.mark.gpu


def test_fill_kv_static_matches_fill_kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    from overlap_decode_step_amd import ld
    shape = W.TINY
    L, nkv = shape["n_layers"], shape["n_kv_heads"]
    calls = [(8, [150, 3, 77, 160, 0, 1, 99, 128], 2), (3, [40, 0, 17], 5)]
    for max_batch, lens, seed in calls:
        print(f"fill_kv_static: max_batch={max_batch} lens={lens} seed={seed}", flush=True)
        ref = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
        ref.alloc_kv(max_batch, 160)
        new = ld.Model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
        new.alloc_kv(max_batch, 160)
        ld.ld_fill_kv(ref.h, seed, 1.0, lens, ref.stream())
        ld.ld_fill_kv_static(new.h, seed, 1.0, lens, new.stream())
        torch.cuda.synchronize()
        assert new.device_error() == 0
        for layer in range(L):
            for b, n in enumerate(lens):
                for h in range(nkv):
                    ka, va = ref.read_kv(layer, b, h, 0, n)
                    kb, vb = new.read_kv(layer, b, h, 0, n)
                    assert np.array_equal(ka, kb) and np.array_equal(va, vb), (layer, b, h)
        # argument errors are reported before anything is enqueued
        with pytest.raises(ld.LdError) as ei:
            ld.ld_fill_kv_static(new.h, seed, 1.0, [161] + lens[1:], new.stream())
        assert ei.value.status == ld.LD_EINVAL
        ref.free()
        new.free()
