"""The binding's argument checks: a tensor on another device than the metadata, a wrong
dtype or shape, a workspace too small (the library's synchronous MOE_ENOSPC) or on
another device are refused before anything is enqueued, and a correct call afterwards
gives the same result as before them."""
import pytest

import synth
from _util import Gpu, np64

pytestmark = pytest.mark.gpu


def test_binding_refuses_bad_arguments():
    import numpy as np
    import torch

    import token_routing_grouped_amd as moe

    d = synth.case(N=64, H=128, I=128, E=4, K=2, seed=41)
    g = Gpu(d)
    g.build()
    ref = np64(g.forward(save_h=False)).copy()
    out = torch.empty(g.N, g.H, dtype=torch.bfloat16, device=g.x.device)
    fwd = lambda **kw: moe.moe_expert_forward(
        g.meta, kw.get("x", g.x), kw.get("w_up", g.w_up), g.w_down, kw.get("out", out),
        workspace=kw.get("workspace"))
    with pytest.raises(ValueError, match="is on cpu"):
        fwd(x=g.x.cpu())
    with pytest.raises(TypeError):
        fwd(w_up=g.w_up.float())
    with pytest.raises(ValueError, match="shape"):
        fwd(out=out[:-1])
    with pytest.raises(moe.MoeError):
        fwd(workspace=torch.empty(16, dtype=torch.uint8, device=g.x.device))
    with pytest.raises(ValueError, match="workspace is on"):
        fwd(workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="is on cpu"):
        moe.moe_build_metadata(g.topk_idx.cpu(), g.topk_weights, g.meta)
    fwd()
    torch.cuda.synchronize()
    assert np.array_equal(np64(out), ref)
