"""The matrix-core rate probe (measurement support, not part of the emulation) runs
through the C ABI, reports its operation count, and is deterministic."""
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
from gpu_common import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,per_inst", [(0, 65536), (1, 131072)])
def test_probe_mfma_runs(kind, per_inst):
    announce(f"probe kind={kind}")
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    operands = torch.randint(-128, 128, (4096,), dtype=torch.int8, device="cuda", generator=g)
    sink1 = torch.full((8 * 512,), 7, dtype=torch.int32, device="cuda")
    sink2 = torch.full((8 * 512,), 9, dtype=torch.int32, device="cuda")
    ops = ozk.ozk_probe_mfma(kind, operands, 3, 8, sink=sink1)
    ozk.ozk_probe_mfma(kind, operands, 3, 8, sink=sink2)
    torch.cuda.synchronize()
    assert ops == 8 * 8 * 32 * per_inst * 3
    assert torch.equal(sink1, sink2)
