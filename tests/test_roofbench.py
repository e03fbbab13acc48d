"""The roofline microbenchmark library: it loads and exports what include/mla_roofbench.h
declares, rejects bad arguments on the host (CPU), and on the GPU its kernels do the work they
claim: the stream read folds every 16-B word of its buffer (checked against the XOR of all
words computed on the host), and every MFMA of the loop lands in its accumulators."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from mla_latent_space_amd import roofbench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_roofbench.h")


def test_library_is_built_and_exports_every_declared_symbol():
    assert os.path.exists(roofbench.LIB_PATH), f"{roofbench.LIB_PATH} is missing: run __graft_entry__.build() first"
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mla_rb_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mla_rb_mfma_bf16_loop", "mla_rb_stream_read"]
    L = ctypes.CDLL(roofbench.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_host_rejects_bad_arguments():
    L = roofbench.lib()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    assert L.mla_rb_stream_read(None, 1024, p, 1, None) == 1
    assert L.mla_rb_stream_read(p, 1024, None, 1, None) == 1
    assert L.mla_rb_stream_read(p, 0, p, 1, None) == 1
    assert L.mla_rb_stream_read(p, 1000, p, 1, None) == 1        # not a multiple of 16
    assert L.mla_rb_stream_read(p + 4, 1024, p, 1, None) == 1    # misaligned
    assert L.mla_rb_stream_read(p, 1024, p, 0, None) == 1
    assert L.mla_rb_stream_read(p, 1024, p, 65537, None) == 1
    assert L.mla_rb_mfma_bf16_loop(1, 1, 1, None, p, None) == 1
    assert L.mla_rb_mfma_bf16_loop(1, 1, 1, p, None, None) == 1
    assert L.mla_rb_mfma_bf16_loop(0, 1, 1, p, p, None) == 1
    assert L.mla_rb_mfma_bf16_loop(1, 3, 1, p, p, None) == 1
    assert L.mla_rb_mfma_bf16_loop(1, 1, 0, p, p, None) == 1
    assert L.mla_rb_mfma_bf16_loop(1, 1, (1 << 20) + 1, p, p, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("nwords,blocks", [(1, 1), (4096 * 8 + 3, 1), (100_003, 7), (1 << 20, 64)])
def test_stream_read_folds_every_word(nwords, blocks):
    torch.cuda.set_device(0)
    g = torch.Generator().manual_seed(nwords)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nwords, 4), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    sink = torch.full((16 * roofbench.STREAM_THREADS * blocks,), 0x5A, dtype=torch.uint8, device="cuda")
    roofbench.stream_read(src, sink, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert (got == want).all(), (got, want)


@pytest.mark.gpu
@pytest.mark.parametrize("blocks,wps,iters", [(1, 1, 1), (3, 2, 7), (256, 1, 300), (256, 2, 1000)])
def test_mfma_loop_accumulates_every_mfma(blocks, wps, iters):
    torch.cuda.set_device(0)
    sink = torch.full((4 * 256 * wps * blocks,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    roofbench.mfma_loop(blocks, wps, iters, sink, clocks)
    torch.cuda.synchronize()
    assert bool((sink == 256.0 * iters).all())
    c = clocks.view(blocks, 4).cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] >= c[:, 2]).all()


@pytest.mark.gpu
def test_measure_reports_plausible_denominators():
    m = roofbench.measure(0, reps=3)
    assert 500 < m["stream_read_gbps"] < 8000 * 1.05
    for v in m["mfma_bf16_tflops"].values():
        assert 100 < v < 2517 * 1.02
    assert 0.5 < m["clock_ghz_under_mfma"] < 2.6
