"""The prefill prepare's gates against torch's eager expressions on the same
device (core.ssm.ops.gdp.prepare, module description: the gates are to match
the eager path bit for bit).  The library evaluates beta = 1 / (1 + exp(-b))
and g = -exp(A_log) * softplus(a + dt_bias) in float32 with the device's exp
and log1p, in the eager expressions' order, so the results must be equal bit
for bit, over inputs that span the gates' ranges (saturated sigmoids both
ways, both softplus branches and the switch at 20), for float32 and bfloat16
inputs."""
import pytest
import torch
import torch.nn.functional as F

from gated_delta_product_amd import binding as G

pytestmark = pytest.mark.gpu


def _ulps(a, b):
    """Distance in float32 ulps (ordered integer representation)."""
    ia = a.contiguous().view(torch.int32).to(torch.int64)
    ib = b.contiguous().view(torch.int32).to(torch.int64)
    ia = torch.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = torch.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return (ia - ib).abs()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prepare_gates_against_torch_eager(dtype):
    dev = "cuda:0"
    n, T, M, H, Gq, P, N = 1, 4096, 2, 8, 2, 16, 16
    gen = torch.Generator(device="cpu").manual_seed(16)
    x = torch.randn(n, T, M * H * P + M * Gq * N + Gq * N, generator=gen).to(dtype)
    # b over [-40, 40] (saturating sigmoid both ways); a + dt_bias over
    # [-30, 30] (both softplus branches, including around 20)
    b = (torch.rand(n, T, M * H, generator=gen) * 80 - 40)
    a = (torch.rand(n, T, H, generator=gen) * 60 - 30)
    ba = torch.cat([b, a], dim=-1).to(dtype)
    A_log = (torch.rand(H, generator=gen) * 4 - 2).float()
    dt_bias = (torch.rand(H, generator=gen) * 2 - 1).float()
    x, ba, A_log, dt_bias = x.to(dev), ba.to(dev), A_log.to(dev), dt_bias.to(dev)
    _, _, _, beta, g = G.prefill_prepare(x, ba, A_log, dt_bias, M, H, Gq, P, N)
    torch.cuda.synchronize()

    bf = ba[:, :, : M * H].float().reshape(n, T * M, H)
    af = ba[:, :, M * H:].float()
    beta_eager = torch.sigmoid(bf)
    g_eager = -torch.exp(A_log) * F.softplus(af + dt_bias)
    ub = _ulps(beta, beta_eager)
    ug = _ulps(g, g_eager)
    rep = {"beta": (int(ub.max()), int((ub > 0).sum()), ub.numel()),
           "g": (int(ug.max()), int((ug > 0).sum()), ug.numel())}
    print("\n%s eager gates: beta max %d ulp, %d of %d differ; g max %d ulp, %d of %d differ"
          % (str(dtype).replace("torch.", ""), *rep["beta"], *rep["g"]))
    assert rep["beta"][0] == 0 and rep["g"][0] == 0, rep
