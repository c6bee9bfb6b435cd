"""The allocation-free split-KV entry point (attn_fwd_splitkv_noalloc), called
through the C ABI on the GPU: its outputs equal attn_fwd_splitkv's with a
caller workspace and the same split count, bit for bit, and match the fp64
oracle, on two calls in a row (the second on a smaller input, so the static
scratch still holds the first call's partial results)."""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # B, H, S, D, causal, scale, n_splits, seed -- the second is smaller
    (2, 3, 700, 64, True, 0.125, 3, 9901),
    (1, 2, 300, 128, False, 0.08838834764831845, 2, 9902),
]


def _run(entry, q, k, v, B, H, S, D, causal, scale, n_splits):
    import torch

    from exact_attention_forward_05_amd import _lib

    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.full_like(qt, float("nan"))
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if entry == "noalloc":
        rc = _lib.attn_fwd_splitkv_noalloc(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                           o.data_ptr(), lse.data_ptr(), B, H, S, D, scale,
                                           int(causal), n_splits, stream)
    else:
        need = _lib.splitkv_workspace_size(B, H, S, D, n_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        rc = _lib.attn_fwd_splitkv(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, S, D, scale, int(causal), n_splits,
                                   ws.data_ptr(), ws.numel(), stream)
    _lib.check(rc)
    torch.cuda.synchronize(dev)
    return o.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    for (B, H, S, D, causal, scale, ns, seed) in CASES:
        print(f"[no-alloc] B{B} H{H} S{S} D{D} causal={causal} n_splits={ns}", flush=True)
        q, k, v = make_qkv(B, H, S, D, seed)
        o1, l1 = _run("noalloc", q, k, v, B, H, S, D, causal, scale, ns)
        o2, l2 = _run("workspace", q, k, v, B, H, S, D, causal, scale, ns)
        assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
        O, L = oracle.sdpa_forward(q, k, v, scale, causal)
        print(f"[no-alloc] {compare(o1, l1, O, L, 'noalloc')}", flush=True)


def test_noalloc_single_pass_and_oversized_request():
    from exact_attention_forward_05_amd import _lib

    B, H, S, D = 1, 2, 200, 64
    q, k, v = make_qkv(B, H, S, D, 9903)
    o, l = _run("noalloc", q, k, v, B, H, S, D, True, 0.125, 1)
    O, L = oracle.sdpa_forward(q, k, v, 0.125, True)
    compare(o, l, O, L, "noalloc n_splits=1")
    # more partial results than the static buffer holds: rejected on the host
    Sbig = 1 << 16
    assert _lib.splitkv_workspace_size(1, 8, Sbig, 64, 8) > _lib.NOALLOC_SCRATCH_BYTES
    import torch

    dev = torch.device("cuda:0")
    t = torch.zeros((1, 8, 128, 64), dtype=torch.float16, device=dev)
    rc = _lib.attn_fwd_splitkv_noalloc(t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                       t.data_ptr(), 1, 8, Sbig, 64, 0.125, 0, 8, 0)
    assert _lib.STATUS_NAMES[rc] == "ATTN_ERR_ARG"
    assert "static scratch" in _lib.load().attn_last_error().decode()
