"""The access-pattern reference kernels (libep_ceiling.so) that the
benchmark times beside the path: exports and argument checks on the CPU, the
bytes each kernel moves on the GPU (a reference that moved fewer bytes would
overstate the memory system's rate for the pattern)."""
import ctypes

import numpy as np
import pytest

from combine_ep_layout_10_amd import ceiling


def test_exports_and_argument_checks():
    lib = ceiling.lib()
    for name in ceiling.SIGNATURES:
        assert hasattr(lib, name)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below is rejected first
    with pytest.raises(RuntimeError):
        ceiling.write_rows(fake, 4, 24)                   # not a multiple of 16 bytes
    with pytest.raises(RuntimeError):
        ceiling.write_rows(None, 4, 32)
    with pytest.raises(RuntimeError):
        ceiling.copy(fake, fake, 100)
    with pytest.raises(RuntimeError):
        ceiling.broadcast(fake, 4, 96, fake, 32, fake, 2)  # a source row neither 1 nor 2 receive rows
    with pytest.raises(RuntimeError):
        ceiling.broadcast(fake, 4, 64, fake, 32, fake, 65)
    with pytest.raises(RuntimeError):
        ceiling.gather(fake, 32 * 1024, fake, 2, 4, fake)  # rows wider than one block
    with pytest.raises(RuntimeError):
        ceiling.read_rows(fake, 4, 32, None)
    # empty work launches nothing
    ceiling.write_rows(fake, 0, 32)
    ceiling.copy(fake, fake, 0)


@pytest.mark.gpu
def test_reference_kernels_move_the_stated_bytes():
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(61)
    T, k, R, row = 37, 5, 300, 7168 * 2
    src = torch.from_numpy(rng.integers(0, 256, size=(T, row), dtype=np.uint8)).to(dev)
    rows = rng.permutation(R)[:T * k].reshape(T, k).astype(np.int32)
    rows[3, 1] = -1
    rows_d = torch.from_numpy(rows).to(dev)
    # broadcast, a row to k rows
    dst = torch.zeros((R, row), dtype=torch.uint8, device=dev)
    ceiling.broadcast(src.data_ptr(), T, row, dst.data_ptr(), row, rows_d.data_ptr(), k)
    d, s = dst.cpu().numpy(), src.cpu().numpy()
    for t in range(T):
        for j in range(k):
            if rows[t, j] >= 0:
                assert np.array_equal(d[rows[t, j]], s[t])
    assert not d[[r for r in range(R) if r not in set(rows.ravel())]].any()
    # broadcast, a bf16-sized row to k half-size rows: the two 16-byte halves of each 32 combined
    dst2 = torch.zeros((R, row // 2), dtype=torch.uint8, device=dev)
    ceiling.broadcast(src.data_ptr(), T, row, dst2.data_ptr(), row // 2, rows_d.data_ptr(), k)
    d2 = dst2.cpu().numpy()
    v = s.reshape(T, -1, 2, 16)
    want = (v[:, :, 0] ^ v[:, :, 1]).reshape(T, row // 2)
    for t in range(T):
        for j in range(k):
            if rows[t, j] >= 0:
                assert np.array_equal(d2[rows[t, j]], want[t])
    # gather: k rows in, their xor out
    g = torch.empty((T, row), dtype=torch.uint8, device=dev)
    ceiling.gather(dst.data_ptr(), row, rows_d.data_ptr(), k, T, g.data_ptr())
    assert np.array_equal(g.cpu().numpy(), np.where((rows >= 0).sum(1)[:, None] % 2 == 1, s, 0))
    # copy and row writes
    a = torch.from_numpy(rng.integers(0, 256, size=(1 << 20) + 4096, dtype=np.uint8)).to(dev)
    b = torch.zeros_like(a)
    ceiling.copy(a.data_ptr(), b.data_ptr(), a.numel())
    assert torch.equal(a, b)
    w = torch.zeros((R, row), dtype=torch.uint8, device=dev)
    ceiling.write_rows(w.data_ptr(), R, row)
    wv = w.view(torch.int32).view(R, row // 16, 4).cpu().numpy()
    assert (wv[:, :, 0] == np.arange(R)[:, None]).all() and (wv[:, :, 2:] == [1, 2]).all()
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    ceiling.read_rows(src.data_ptr(), T, row, sink.data_ptr())
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
