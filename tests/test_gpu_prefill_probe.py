"""The prefill inner-loop probe (moe_prefill_inner_probe): every variant runs
to completion and writes one finite sum per thread (the bf16 variant's 256
workgroups the first half of out, each int8 variant's 512 all of it), the
same sums on a second launch, and bad arguments are refused before any
launch."""
import pytest
import torch

import quantized_routed_expert_moe_amd as Q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant,threads", [(0, 65536), (1, 131072), (2, 131072)])
def test_prefill_probe_writes_its_sums(variant, threads):
    out = torch.full((Q.PREFILL_PROBE_OUT_FLOATS + 64,), float("nan"), dtype=torch.float32, device="cuda")
    flops = Q.moe_prefill_inner_probe(variant, 64, out)
    torch.cuda.synchronize()
    assert flops == 1024 * 64 * 2 * 256 * 64 * 32
    first = out.clone()
    assert torch.isfinite(first[:threads]).all()
    assert torch.isnan(first[threads:]).all()  # nothing past the variant's threads
    Q.moe_prefill_inner_probe(variant, 64, out)
    torch.cuda.synchronize()
    assert torch.equal(out[:threads], first[:threads])


def test_prefill_probe_refusals():
    out = torch.zeros(Q.PREFILL_PROBE_OUT_FLOATS, dtype=torch.float32, device="cuda")
    with pytest.raises(Q.QmoeError, match="variant"):
        Q.moe_prefill_inner_probe(3, 8, out)
    with pytest.raises(Q.QmoeError, match="variant"):
        Q.moe_prefill_inner_probe(-1, 8, out)
    with pytest.raises(Q.QmoeError, match="sub_blocks"):
        Q.moe_prefill_inner_probe(0, 0, out)
    with pytest.raises(Q.QmoeError, match="fewer than"):
        Q.moe_prefill_inner_probe(0, 8, out[:1000])
    with pytest.raises(TypeError, match="dtype"):
        Q.moe_prefill_inner_probe(0, 8, out.view(torch.int32))
