"""The expert store on the CPU: blobs written by the generator come back
byte for byte through pread (buffered and direct I/O), through mmap, at
every queue depth and piece size; bad arguments are refused.  No GPU."""
import ctypes
import os

import numpy as np
import pytest

from synthetic import gen

moe = pytest.importorskip("quantized_mixture_experts_moe_amd.moe")

CFG = gen.CONFIGS["tiny"]
LAYERS = 3


@pytest.fixture(scope="module")
def expert_file(tmp_path_factory):
    d = tmp_path_factory.mktemp("store")
    path = str(d / "experts.bin")
    size = gen.write_expert_file(path, 4, LAYERS, CFG)
    assert os.path.getsize(path) == size
    return path


def _aligned(n_bufs, stride):
    raw = np.zeros(n_bufs * stride + 4096, dtype=np.uint8)
    off = (-raw.ctypes.data) % 4096
    bufs = raw[off:off + n_bufs * stride].reshape(n_bufs, stride)
    return raw, bufs


def test_stride_is_blob_rounded_to_4096():
    assert moe.moe_store_stride(2816, 704) == 3_346_432 == 817 * 4096
    assert moe.moe_store_stride(2816, 704) >= moe.moe_blob_bytes(2816, 704)
    assert moe.moe_store_stride(256, 128) == gen.store_stride(256, 128) == 57_344
    assert moe.moe_store_stride(0, 64) == 0


@pytest.mark.parametrize("flags", [0, moe.MOE_STORE_DIRECT, moe.MOE_STORE_MMAP])
@pytest.mark.parametrize("threads,chunk", [(1, 0), (4, 4096), (16, 8192), (64, 0)])
def test_reads_are_the_generated_blobs(expert_file, flags, threads, chunk):
    st = moe.Store(expert_file, LAYERS, CFG.E, CFG.D, CFG.F, flags=flags, threads=threads)
    nb = moe.moe_blob_bytes(CFG.D, CFG.F)
    rng = np.random.default_rng(threads + flags)
    for layer in range(LAYERS):
        ids = rng.choice(CFG.E, size=5, replace=False)
        _raw, bufs = _aligned(len(ids), st.stride)
        st.read(layer, ids, [bufs[i].ctypes.data for i in range(len(ids))], chunk)
        for i, e in enumerate(ids):
            want = gen.expert_blob(4, layer, int(e), CFG.D, CFG.F)
            assert np.array_equal(bufs[i, :nb], want), (layer, e)
    s = st.stats()
    assert s["blobs"] == 5 * LAYERS and s["bytes"] == 5 * LAYERS * nb
    st.close()


def test_bad_arguments(expert_file, tmp_path):
    h = ctypes.c_void_p()
    lib = moe.lib
    # missing file, file too short for the shapes, bad thread count, both flags
    assert lib.moe_store_open(ctypes.byref(h), str(tmp_path / "none").encode(), 1, CFG.E, CFG.D,
                              CFG.F, 0, 4) == moe.MOE_E_INVALID
    assert lib.moe_store_open(ctypes.byref(h), expert_file.encode(), LAYERS + 1, CFG.E, CFG.D,
                              CFG.F, 0, 4) == moe.MOE_E_INVALID
    assert lib.moe_store_open(ctypes.byref(h), expert_file.encode(), LAYERS, CFG.E, CFG.D, CFG.F,
                              0, 0) == moe.MOE_E_INVALID
    assert lib.moe_store_open(ctypes.byref(h), expert_file.encode(), LAYERS, CFG.E, CFG.D, CFG.F,
                              3, 4) == moe.MOE_E_INVALID
    st = moe.Store(expert_file, LAYERS, CFG.E, CFG.D, CFG.F, flags=moe.MOE_STORE_DIRECT)
    _raw, bufs = _aligned(1, st.stride)
    with pytest.raises(moe.MoEError):
        st.read(LAYERS, [0], [bufs[0].ctypes.data])       # layer out of range
    with pytest.raises(moe.MoEError):
        st.read(0, [CFG.E], [bufs[0].ctypes.data])        # expert out of range
    st.close()
