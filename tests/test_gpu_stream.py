"""The streaming probe (a measurement hook) writes what glu_mx.h defines, for every source
and destination count and every destination width, so the ceilings it measures move the
bytes they claim."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_src", [1, 2, 3])
@pytest.mark.parametrize("n_dst", [1, 2, 4])
@pytest.mark.parametrize("width", [4, 8, 16])
def test_probe_output(gpu, n_src, n_dst, width):
    n = 16 * 5000 + 16 * 37              # vectors past a whole number of workgroups
    g = torch.Generator(device="cuda").manual_seed(n_src * 10 + n_dst)
    srcs = [torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8, device="cuda") for _ in range(n_src)]
    dsts = [torch.empty(n * width // 16, dtype=torch.uint8, device="cuda") for _ in range(n_dst)]
    gpu.glu_stream_probe(srcs, dsts)
    x = srcs[0].view(torch.int32).view(-1, 4).clone()
    for t in srcs[1:]:
        x ^= t.view(torch.int32).view(-1, 4)
    for k, d in enumerate(dsts):
        if width == 16:
            want = x.clone()
            want[:, 0] += k
        elif width == 8:
            want = torch.stack([(x[:, 0] ^ x[:, 2]) + k, x[:, 1] ^ x[:, 3]], 1)
        else:
            want = (x[:, 0] ^ x[:, 1] ^ x[:, 2] ^ x[:, 3]) + k
        assert torch.equal(d.view(torch.int32).view(want.shape), want), k
