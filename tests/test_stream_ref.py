"""The measurement reference that bench.py times beside every part
(hadamard_rotation_preprocessing_amd/csrc/stream_ref.hip, built as
lib/libhrstream.so; not part of the rotate + quantize path).

CPU: the library exists and exports its two entry points, and invalid
arguments are refused before any HIP call.  GPU: a launch reads and writes
exactly the byte counts it is given, each written 16-byte piece being the
documented XOR of the pieces its thread loaded, so the floor bench.py reports
is a kernel that really moves those bytes."""
import ctypes
import os

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "hadamard_rotation_preprocessing_amd", "lib", "libhrstream.so")


def lib():
    if not os.path.exists(PATH):
        pytest.fail("libhrstream.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.hr_stream_ref.argtypes = [vp, i64, vp, i64, vp]
    L.hr_stream_ref.restype = ci
    L.hr_clock_ref.argtypes = [vp, ci, ci, vp]
    L.hr_clock_ref.restype = ci
    return L


def test_exports_and_rejects_invalid_arguments():
    L = lib()
    fake = ctypes.c_void_p(0x7F0000000000)
    assert L.hr_stream_ref(fake, 17, fake, 16, None) == -1          # not a multiple of 16
    assert L.hr_stream_ref(fake, 16, fake, -16, None) == -1         # negative
    assert L.hr_stream_ref(None, 16, fake, 16, None) == -1          # NULL source with bytes to read
    assert L.hr_stream_ref(ctypes.c_void_p(0x7F0000000008), 16, fake, 16, None) == -1   # misaligned
    assert L.hr_stream_ref(None, 0, None, 0, None) == 0             # nothing to do: no launch
    assert L.hr_clock_ref(None, 4, 10, None) == -1
    assert L.hr_clock_ref(fake, 0, 10, None) == -1


def expected(src_words, nr, nw):
    """dst pieces of the kernel: thread t of block b handles pieces
    p = 1024 b + t + 256 k (k < 4), loads those below nr (zero otherwise) and
    stores acc ^ v_k for those below nw, acc being the XOR of its four."""
    n = max(nr, nw)
    blocks = -(-n // 1024)
    pieces = np.zeros((blocks * 1024, 4), dtype=np.uint32)
    pieces[:nr] = src_words[:nr]
    v = pieces.reshape(blocks, 4, 256, 4)           # [block, k, thread, word]
    acc = np.bitwise_xor.reduce(v, axis=1)          # [block, thread, word]
    out = (v ^ acc[:, None, :, :]).reshape(blocks * 1024, 4)
    return out[:nw]


@pytest.mark.gpu
@pytest.mark.parametrize("nr,nw", [(3000, 1000), (1000, 3000), (4096, 4096), (1, 0), (0, 5)])
def test_stream_ref_moves_the_given_bytes(nr, nw):
    print("stream_ref case", nr, nw, flush=True)
    L = lib()
    g = torch.Generator().manual_seed(nr * 7 + nw)
    src = torch.randint(0, 2 ** 31 - 1, (max(nr, 1) * 4,), dtype=torch.int64, generator=g).to(torch.int32)
    srcg = src.to("cuda:0")
    guard = 64                                         # pieces past the end that must stay untouched
    dst = torch.full(((nw + guard) * 4,), -1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert L.hr_stream_ref(srcg.data_ptr(), 16 * nr, dst.data_ptr(), 16 * nw, st) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)
    want = expected(src.numpy().view(np.uint32).reshape(-1, 4), nr, nw)
    assert np.array_equal(got[:nw], want)
    assert np.all(got[nw:] == 0xFFFFFFFF)


@pytest.mark.gpu
def test_clock_ref_runs():
    L = lib()
    out = torch.zeros(1024, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert L.hr_clock_ref(out.data_ptr(), 1024, 100, st) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0      # the chains' sum is never the sentinel
