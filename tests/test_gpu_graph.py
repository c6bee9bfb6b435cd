"""Both entry points under HIP graph capture: the library allocates nothing
and records no memory fills, so a captured launch sequence replays. Each of
three replays runs after the outputs were cleared by eager work, and every
replay must equal the eager result bit for bit."""
import numpy as np
import pytest

from parity import gpu_available
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("split", [1, 3], ids=["single_pass", "splitkv3"])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_graph_replays_equal_eager(split, causal):
    import torch

    import exact_attention_forward_05_amd as attn

    print(f"[gpu-graph] split={split} causal={causal}", flush=True)
    B, H, S, D = 1, 4, 700, 64
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in make_qkv(B, H, S, D, 6100 + split))
    scale = 0.125
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, attn.splitkv_workspace_size(B, H, S, D, split)), dtype=torch.uint8,
                     device=dev)
    st = torch.cuda.Stream(device=dev)

    def call():
        if split == 1:
            attn.fwd(q, k, v, scale=scale, causal=causal, out=o, lse=lse,
                     stream=torch.cuda.current_stream(dev))
        else:
            attn.fwd_splitkv(q, k, v, n_splits=split, scale=scale, causal=causal, out=o,
                             lse=lse, workspace=ws, stream=torch.cuda.current_stream(dev))

    with torch.cuda.stream(st):
        call()
    st.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        call()
    for rep in range(3):
        o.zero_()
        lse.fill_(-1.0)
        torch.cuda.synchronize(dev)
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager result"
        assert torch.equal(lse, l_ref), f"replay {rep}: LSE differs from the eager result"
    assert np.isfinite(o_ref.float().cpu().numpy()).all()
