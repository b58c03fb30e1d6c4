"""The library's device copy (the bandwidth probe of bench.py): exact copies
at sizes that leave partial chunks, a byte tail and fewer threads than one
chunk; misaligned and overlapping pointers refused on the host."""

import ctypes

import pytest
import torch


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 7, 3 * (1 << 20) + 4096 * 16 + 5,
                                    64 << 20])
def test_device_copy_is_exact(nbytes):
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = torch.Generator().manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to("cuda:0")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda:0")
    ca.device_copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].abs().sum()) == 0, "wrote past the end"


def test_device_copy_refuses_bad_pointers():
    import gathered_local_attention_amd as ca

    lib = ca._lib.load()
    vp = ctypes.c_void_p
    assert lib.cluster_attn_device_copy(vp(4096 + 8), vp(1 << 20), 1024, vp(0)) != 0   # misaligned
    assert lib.cluster_attn_device_copy(vp(4096), vp(4096 + 512), 1024, vp(0)) != 0    # overlap
    assert lib.cluster_attn_device_copy(vp(0), vp(4096), 16, vp(0)) != 0               # NULL
    assert lib.cluster_attn_device_copy(vp(4096), vp(1 << 20), 0, vp(0)) == 0          # nothing to do
