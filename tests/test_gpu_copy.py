"""GPU check of sc_reference_copy, the streaming copy kernel that serves as
the bandwidth reference of the roofline figures: byte-exact copies of sizes
that end inside a 512 KiB chunk, on one, and across many, and bytes beyond
the copied range untouched."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


@pytest.mark.parametrize("nbytes", [16, 4096, 512 << 10, (512 << 10) + 16, (3 << 20) - 48,
                                    (64 << 20) + 1024])
def test_reference_copy_is_byte_exact(nbytes):
    print(f"[case] reference copy {nbytes} bytes", flush=True)
    g = torch.Generator(device=DEV).manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.full((nbytes + 4096,), 7, dtype=torch.uint8, device=DEV)
    sc.reference_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 7).all())
