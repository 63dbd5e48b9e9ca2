"""The streaming copy the kernels are measured against: every byte lands,
for aligned and unaligned pointers, sizes below, at and above the 16-byte
vectors and the 4096-byte groups of one workgroup, and more groups than the
fixed grid (so that workgroups loop)."""
import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 15, 16, 17, 4095, 4096, 4097, 65536 * 16 + 5, (8192 * 4096) * 3 + 4096 + 48]


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("src_off,dst_off", [(0, 0), (1, 0), (0, 3), (8, 8)])
def test_copy(gpu_lib, nbytes, src_off, dst_off):
    print(f"\n[copy] bytes={nbytes} src+{src_off} dst+{dst_off}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(nbytes + 7 * src_off + dst_off)
    host = torch.randint(0, 256, (nbytes + src_off,), dtype=torch.uint8, generator=g)
    src_buf = host.to(DEV)
    dst_buf = torch.full((nbytes + dst_off + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    src = src_buf[src_off:src_off + nbytes]
    dst = dst_buf[dst_off:dst_off + nbytes]
    gpu_lib.vjp_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((dst_buf[:dst_off] == 0xA5).all()) and bool((dst_buf[dst_off + nbytes:] == 0xA5).all())


@pytest.mark.parametrize("vpl", [1, 2, 4, 8])
@pytest.mark.parametrize("max_wg", [1, 3, 32768])
@pytest.mark.parametrize("nbytes", [4097, 65536 * 16 + 5, 5 * 1024 * 1024 + 24])
def test_copy_shaped(gpu_lib, vpl, max_wg, nbytes):
    """Every launch shape of the copy reference: few workgroups loop over the
    data many times; the last partial group and the byte tail land too."""
    print(f"\n[copy shaped] bytes={nbytes} vpl={vpl} max_wg={max_wg}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(nbytes + vpl + max_wg)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(DEV)
    dst_buf = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    gpu_lib.vjp_copy_shaped(src, dst_buf[:nbytes], vpl, max_wg)
    torch.cuda.synchronize()
    assert torch.equal(dst_buf[:nbytes], src) and bool((dst_buf[nbytes:] == 0xA5).all())
