"""GPU parity of the split-KV entry point (attn_fwd_splitkv) through the C ABI.

Each query tile's key pairs are cut into n_splits runs (some empty when a tile
has fewer pairs than runs) and merged by the combine kernel; the result is
compared with the fp64 oracle like the single-pass path, and with the
single-pass path itself.
"""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, run_gpu, sample_rows
from testkit import WORKLOADS, make_qkv, workload_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _announce(what):
    print(f"[gpu-splitkv] {what}", flush=True)


def run_split(q, k, v, scale, causal, n_splits, ws_fill=None):
    import torch

    import exact_attention_forward_05_amd as attn

    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    B, H, S, D = q.shape
    ws = None
    need = attn.splitkv_workspace_size(B, H, S, D, n_splits)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        if ws_fill is not None:
            ws.fill_(ws_fill)
    o, lse = attn.fwd_splitkv(qt, kt, vt, n_splits=n_splits, scale=scale, causal=causal,
                              workspace=ws)
    torch.cuda.synchronize(dev)
    return o.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # B, H, S, D, causal, scale, n_splits, seed
    (1, 2, 17, 64, False, 0.125, 2, 1),        # one pair: the second run is empty
    (1, 2, 300, 64, True, 0.125, 2, 2),
    (2, 3, 300, 64, False, 0.125, 3, 3),
    (1, 2, 640, 64, True, -0.2, 4, 4),         # negative scale
    (1, 1, 1000, 64, True, 0.125, 7, 5),       # more runs than most tiles have pairs
    (1, 2, 129, 128, False, 0.08838834764831845, 2, 6),
    (2, 2, 257, 128, True, 0.08838834764831845, 3, 7),
    (1, 1, 1000, 128, True, 0.08838834764831845, 5, 8),
    (1, 2, 333, 128, False, 0.5, 16, 9),       # peaked rows, many empty runs
    # enough rows that the combine takes a thread per row and 4 columns
    # (the cases above take a wave per row)
    (1, 4, 1100, 64, True, 0.125, 3, 10),
    (1, 2, 1100, 128, False, 0.08838834764831845, 2, 11),
    # from 2048 keys the non-causal D = 64 runs take three waves per SIMD
    # (192-key intervals): ragged tails, uneven runs, peaked and negative scales
    (1, 2, 2500, 64, False, 0.125, 2, 12),
    (1, 1, 3001, 64, False, 0.125, 3, 13),
    (1, 2, 2048, 64, False, 1.0, 4, 14),     # peaked rows: frequent max redos per run
    (1, 1, 2113, 64, False, -0.5, 5, 15),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}S{}D{}{}s{}x{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "n", c[5], c[6]))
def test_splitkv_small_full_compare(case):
    B, H, S, D, causal, scale, n_splits, seed = case
    _announce(f"small {case}")
    q, k, v = make_qkv(B, H, S, D, 9500 + seed)
    o, l = run_split(q, k, v, scale, causal, n_splits, ws_fill=0xFF)  # NaN-filled workspace
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    compare(o, l, O, L, f"splitkv {case}")
    # Against the single-pass path. Each path rounds every probability to fp16
    # (relative error at most 2^-11) against its own running maximum, which
    # the lazy rescale lets lag the true one, so the dominant terms of a
    # peaked row need not be exactly 1: either denominator may sit up to
    # 2^-11 relative from the exact sum, the two in opposite directions, and
    # LSE (the log of the denominator) differs by up to 2^-10 = 9.8e-4. O
    # divides by the same rounded sum it weights with, so its error stays
    # at the fp16 output rounding.
    o1, l1 = run_gpu(q, k, v, scale, causal)
    assert np.abs(o.astype(np.float64) - o1).max() <= 2e-3
    assert np.abs(l.astype(np.float64) - l1).max() <= 1e-3


def test_one_split_is_the_single_pass_path_bitwise():
    q, k, v = make_qkv(1, 2, 700, 64, 9601)
    o, l = run_split(q, k, v, 0.125, True, 1)
    o1, l1 = run_gpu(q, k, v, 0.125, True)
    assert np.array_equal(o.view(np.uint16), o1.view(np.uint16))
    assert np.array_equal(l.view(np.uint32), l1.view(np.uint32))


@pytest.mark.parametrize("name,n_splits", [("sweep_causal_b1h8s4096d64", "auto"),
                                           ("single_head_b1h1s16384d64", "auto"),
                                           ("sdpa_b1h8s4096d64", 2),
                                           ("causal_b2h16s8192d128", 3)])
def test_splitkv_workload_sampled_rows(name, n_splits):
    import exact_attention_forward_05_amd as attn

    w = WORKLOADS[name]
    ns = attn.choose_splits(w.B, w.H, w.S, w.D, w.causal) if n_splits == "auto" else n_splits
    _announce(f"{name} n_splits={ns}")
    q, k, v = workload_inputs(w)
    o, l = run_split(q, k, v, w.scale, w.causal, ns)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    rng = np.random.default_rng(w.seed + 17)
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        rows = sample_rows(w.S, rng)
        O, L = oracle.sdpa_rows(q, k, v, w.scale, w.causal, b, h, rows)
        compare(o[b, h, rows], l[b, h, rows], O, L, f"{name} b{b} h{h}")


@pytest.mark.parametrize("S,D,causal", [(500, 128, True), (2300, 64, False)],
                         ids=["two_waves_d128_causal", "three_waves_d64"])
def test_workspace_and_outputs_stay_in_bounds(S, D, causal):
    """Workspace and outputs inside larger canary-filled buffers, raw C entry
    point on a non-default stream."""
    import torch

    from exact_attention_forward_05_amd import _lib

    B, H, ns = 1, 2, 3
    scale = float(1.0 / np.sqrt(D))
    _announce(f"canary S={S} D={D} causal={causal}")
    q, k, v = make_qkv(B, H, S, D, 9602)
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    need = _lib.splitkv_workspace_size(B, H, S, D, ns)
    assert need == ns * B * H * S * (D + 1) * 4
    guard = 4096
    wbuf = torch.full((need + 2 * guard,), 0xA5, dtype=torch.uint8, device=dev)
    n = B * H * S * D
    obuf = torch.full((n + 2 * guard,), -7.0, dtype=torch.float16, device=dev)
    lbuf = torch.full((B * H * S + 2 * guard,), -7.0, dtype=torch.float32, device=dev)
    st = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(st):
        rc = _lib.attn_fwd_splitkv(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                   obuf.data_ptr() + 2 * guard, lbuf.data_ptr() + 4 * guard,
                                   B, H, S, D, scale, int(causal), ns,
                                   wbuf.data_ptr() + guard, need, st.cuda_stream)
    _lib.check(rc)
    st.synchronize()
    wb = wbuf.cpu().numpy()
    assert (wb[:guard] == 0xA5).all() and (wb[guard + need:] == 0xA5).all()
    ob, lb = obuf.cpu().numpy(), lbuf.cpu().numpy()
    assert (ob[:guard] == -7.0).all() and (ob[guard + n:] == -7.0).all()
    assert (lb[:guard] == -7.0).all() and (lb[guard + B * H * S:] == -7.0).all()
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    compare(ob[guard:guard + n].reshape(B, H, S, D), lb[guard:guard + B * H * S].reshape(B, H, S),
            O, L, "splitkv canary")
