"""GPU mean-pool parity: libgqa's gqa_mean_pool_kv against the fp64 oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
import oracle as O
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import assert_parity, say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("N,H,G,D,dtype", [
    (1000, 64, 8, 128, torch.bfloat16),
    (333, 64, 1, 128, torch.bfloat16),
    (257, 32, 8, 64, torch.bfloat16),
    (100, 12, 3, 64, torch.float32),
    (8192, 64, 8, 128, torch.float32),   # a Llama-2-70B W_K viewed as [d, H, d_h]
])
def test_mean_pool_parity(N, H, G, D, dtype):
    say(f"mean-pool N={N} H={H} G={G} D={D} {dtype}")
    x = I.mean_pool_inputs(N, H, D, dtype=dtype, seed=N + G, device=DEV)
    out = gq.mean_pool_kv(x, G)
    torch.cuda.synchronize()
    ref = O.mean_pool(to_host(x), G)
    if dtype == torch.float32:
        assert_parity(out, ref, dtype, "mean-pool fp32")
    else:
        # one bf16 rounding of the fp32 mean: at most half an ulp
        got = out.float().cpu().double().numpy()
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


def test_mean_pool_identity_and_empty():
    say("mean-pool identity")
    x = I.mean_pool_inputs(77, 16, 128, dtype=torch.bfloat16, seed=1, device=DEV)
    assert torch.equal(gq.mean_pool_kv(x, 16), x)
    e = torch.empty(0, 16, 128, dtype=torch.bfloat16, device=DEV)
    assert gq.mean_pool_kv(e, 4).shape == (0, 4, 128)
    with pytest.raises(gq.GqaError):
        gq.mean_pool_kv(x, 5)
