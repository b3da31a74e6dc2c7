"""The benchmark's read-ceiling probe (libmaxsim_probe.so): exports, host-side argument
checks (CPU), and on the GPU that each mode reads exactly the bytes it should -- the
register mode's per-lane xor against the same fold computed on the host, over a buffer
with a partial last tile and more waves than tiles."""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "late_interaction_reranking_amd", "libmaxsim_probe.so")
TILE, WAVE, WAVES = 4096, 64, 4


def _lib():
    # torch first: it brings its own HIP runtime under the same soname, and the probe
    # library must bind to that one (as it does in the benchmark, where torch is loaded
    # first); loaded the other way round, the process would hold two runtimes.
    import torch  # noqa: F401

    lib = ctypes.CDLL(PROBE)
    lib.maxsim_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_exports():
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})
    assert exported == ["maxsim_probe_blocks", "maxsim_probe_read"]


@pytest.mark.parametrize("buf,nbytes,mode,blocks,sink", [
    (0, 4096, 0, 1, 16),          # null buffer
    (16, 4096, 0, 1, 0),          # null sink
    (16, 0, 0, 1, 16),            # nothing to read
    (16, 4100, 0, 1, 16),         # not a multiple of 16 bytes
    (8, 4096, 0, 1, 16),          # buffer not 16-byte aligned
    (16, 4096, 0, 0, 16),         # no workgroups
    (16, 4096, 0, 65536, 16),     # too many workgroups
    (16, 4096, 2, 1, 16),         # unknown mode
])
def test_rejects_bad_arguments_on_the_host(buf, nbytes, mode, blocks, sink):
    # Rejected before any HIP call, so the pointers are never dereferenced.
    assert _lib().maxsim_probe_read(buf, nbytes, mode, blocks, sink, None) == 1


def expected_register_sink(data: np.ndarray, blocks: int) -> np.ndarray:
    """Per lane of every wave: the xor of the four words of every 16-byte chunk the
    register mode gives it (wave w: tiles [T c(w) / c(W), T c(w + 1) / c(W)), c the
    running sum of wave weights: 12 for a wave of an even block and 11 for one of an odd
    block when the grid is a multiple of 8 blocks, else 1; lane l: the chunks at
    l + 64 s, s < 4, of each tile that lie inside the buffer)."""
    nbytes = data.size
    words = data.view(np.uint32).reshape(-1, 4)
    chunk_fold = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    W = blocks * WAVES
    T = (nbytes + TILE - 1) // TILE
    if blocks % 8 == 0:
        weight = np.where((np.arange(W) // WAVES) % 2 == 0, 12, 11).astype(np.int64)
    else:
        weight = np.ones(W, dtype=np.int64)
    cum = np.concatenate([[0], np.cumsum(weight)])
    starts = T * cum // cum[-1]
    c = np.arange(chunk_fold.size, dtype=np.int64)
    tile = c * 16 // TILE
    e = c % (TILE // 16)
    wave = np.searchsorted(starts, tile, side="right") - 1  # the wave whose range holds the tile
    out = np.zeros(W * WAVE, dtype=np.uint32)
    np.bitwise_xor.at(out, wave * WAVE + e % WAVE, chunk_fold)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("tiles,tail", [(257, 48), (3 * 3072 + 5, 0)])
def test_modes_read_every_byte_once(tiles, tail):
    torch = pytest.importorskip("torch")
    print(f"[read probe] tiles {tiles} tail {tail}", flush=True)
    nbytes = tiles * TILE + tail
    data = np.random.default_rng(tiles).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32).view(np.uint8)
    buf = torch.from_numpy(data).cuda()
    torch.cuda.synchronize()
    lib = _lib()
    blocks = int(lib.maxsim_probe_blocks())
    assert blocks >= 1
    sink = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.maxsim_probe_read(buf.data_ptr(), nbytes, 1, blocks, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, expected_register_sink(data, blocks))
    # LDS-DMA mode: every wave's last load into its first slot lies past its range (a
    # zero-size descriptor), and out-of-range lanes write zeros, so the sink reads 0.
    assert lib.maxsim_probe_read(buf.data_ptr(), nbytes, 0, blocks, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().max().item()) == 0
