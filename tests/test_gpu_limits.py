"""GPU parity at the size limits of the boundary: one very long head (32-bit
byte offsets within a head, up to S*D*2 = 256 MB here), and a tensor of more
than 2^31 elements (64-bit head offsets). Both are checked on sampled rows
against the fp64 oracle; the large tensor is built on the device from one
seeded head plus a distinct per-head offset, and the sampled heads are copied
back so the oracle sees exactly the operands the kernel read.
"""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, sample_rows
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _announce(what):
    print(f"[gpu-limits] {what}", flush=True)


@pytest.mark.parametrize("S,D,causal", [(1 << 20, 64, False), (1 << 20, 128, True)])
def test_one_long_head(S, D, causal):
    import torch

    import exact_attention_forward_05_amd as attn

    _announce(f"S={S} D={D} causal={causal}")
    q, k, v = make_qkv(1, 1, S, D, 9701 + D)
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o, lse = attn.fwd(qt, kt, vt, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(S, np.random.default_rng(S + D), n_random=8)
    O, L = oracle.sdpa_rows(q, k, v, scale, causal, 0, 0, rows)
    _announce(str(compare(o[0, 0, rows], lse[0, 0, rows], O, L, f"long head S={S} D={D}")))


def test_more_than_2_31_elements():
    import torch

    import exact_attention_forward_05_amd as attn

    B, H, S, D = 4100, 4, 1024, 128      # 2^31 + 2^23 elements per tensor
    n_heads = B * H
    assert n_heads * S * D > (1 << 31)
    free, _ = torch.cuda.mem_get_info()
    need = 4 * n_heads * S * D * 2 + n_heads * S * 4
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 2**30:.1f} GiB of free device memory")
    _announce(f"B={B} H={H} S={S} D={D} causal")
    dev = torch.device("cuda:0")
    q0, k0, v0 = make_qkv(1, 1, S, D, 9801)
    idx = torch.arange(n_heads, device=dev)

    def build(base, mult):
        # head h = base + ((h * mult) % 61 - 30) / 32, rounded to fp16 once
        off = (((idx * mult) % 61) - 30).to(torch.float32) / 32.0
        t = torch.from_numpy(base[0, 0]).to(dev).to(torch.float32)
        return (t[None] + off[:, None, None]).to(torch.float16).reshape(B, H, S, D)

    qt, kt, vt = build(q0, 7), build(k0, 13), build(v0, 29)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o, lse = attn.fwd(qt, kt, vt, scale=scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9801)
    for b, h in [(0, 0), (B // 2, 1), (B - 1, H - 1)]:
        qh, kh, vh = (t[b:b + 1, h:h + 1].cpu().numpy() for t in (qt, kt, vt))
        rows = sample_rows(S, rng, n_random=8)
        O, L = oracle.sdpa_rows(qh, kh, vh, scale, True, 0, 0, rows)
        og = o[b, h].cpu().numpy()[rows]
        lg = lse[b, h].cpu().numpy()[rows]
        _announce(f"head ({b},{h}) {compare(og, lg, O, L, f'head ({b},{h})')}")
