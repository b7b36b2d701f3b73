"""Checked mode (SFFN_DEBUG_CHECKS): calls that take device index lists read
them on the host first and refuse a list that breaks the preconditions --
an index out of range, a repeated index, a negative count -- with
SFFN_EINVAL, launching nothing (the output keeps its sentinel); valid lists
run and give the same bits as without the check.  The invalid lists are
only ever passed with the check on, so no kernel sees them."""
import numpy as np
import pytest
import torch

from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from gpu_common import banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("SFFN_DEBUG_CHECKS", "1")


def refused(call, needle):
    with pytest.raises(B.SffnError) as e:
        call()
    assert e.value.status == B.SFFN_EINVAL and needle in str(e.value), str(e.value)


def test_gemv_and_fused_lists(checked):
    banner("debug checks: gemv, fused")
    N, d = 512, 256
    W = dev(synth.weight_bf16(1, synth.W_C0, 0, 0, synth.T_DOWN, N, d))
    Wg = dev(synth.weight_bf16(1, synth.W_C0, 0, 0, synth.T_GATE, N, d))
    a = torch.randn(N, device="cuda")
    x = torch.randn(d, device="cuda")
    ws = B.new_workspace(1, N, d)
    y = torch.full((d,), 9.0, device="cuda")
    cnt = lambda c: torch.tensor([c], dtype=torch.int32, device="cuda")  # noqa: E731
    good = torch.arange(0, N, 3, dtype=torch.int32, device="cuda")
    bad_range = good.clone(); bad_range[7] = N
    bad_neg = good.clone(); bad_neg[3] = -2
    bad_dup = good.clone(); bad_dup[10] = bad_dup[2]
    for idx, needle in ((bad_range, "idx[7]"), (bad_neg, "idx[3]"), (bad_dup, "repeats")):
        refused(lambda: B.sparse_ffn_gemv(B.OP_AXPY, W, None, a, y, idx=idx, count=cnt(idx.numel()),
                                          k_max=idx.numel(), workspace=ws), needle)
        refused(lambda: B.sparse_ffn_fused_swiglu(Wg, Wg, W, x, y, idx=idx, count=cnt(idx.numel()),
                                                  k_max=idx.numel(), workspace=ws), needle)
    refused(lambda: B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wg, x, torch.zeros(N, device="cuda"),
                                      idx=good, count=cnt(-1), k_max=good.numel()), "count -1")
    torch.cuda.synchronize()
    assert torch.all(y == 9.0), "a refused call wrote its output"
    # entries past the count are not checked (nor read by the kernels)
    B.sparse_ffn_gemv(B.OP_AXPY, W, None, a, y, idx=bad_range, count=cnt(7), k_max=bad_range.numel(),
                      workspace=ws)
    y_checked = host(y).copy()
    y2 = torch.full((d,), 9.0, device="cuda")
    import os
    os.environ.pop("SFFN_DEBUG_CHECKS")
    B.sparse_ffn_gemv(B.OP_AXPY, W, None, a, y2, idx=bad_range, count=cnt(7), k_max=bad_range.numel(),
                      workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(y_checked.view(np.uint32), host(y2).view(np.uint32))


def test_lists_tiered_and_compact(checked):
    banner("debug checks: lists, tiered, compact")
    N, d = 448, 256
    W = dev(synth.weight_bf16(2, synth.W_C3, 0, 0, synth.T_DOWN, N, d))
    a = torch.randn(N, device="cuda")
    ws = B.new_workspace(1, N, d)
    y = torch.zeros(d, device="cuda")
    cnt = lambda c: torch.tensor([c], dtype=torch.int32, device="cuda")  # noqa: E731
    good = torch.arange(0, 14, dtype=torch.int32, device="cuda")
    bad = good.clone(); bad[5] = 14                       # 14 clusters of 32 rows: 0..13
    refused(lambda: B.sparse_ffn_gemv_lists([W, W], [a, a], [good, bad], [cnt(14), cnt(14)],
                                            [14, 14], y, group=32, workspace=ws), "list 1")
    refused(lambda: B.sparse_ffn_rowop_lists(B.OP_DOT, [W, W], None, torch.randn(d, device="cuda"),
                                             [torch.zeros(N, device="cuda")] * 2, idxs=[bad, good],
                                             counts=[cnt(14), cnt(14)], k_maxs=[14, 14], group=32),
            "list 0")
    # compaction (count from the host)
    out = torch.zeros(8, d, dtype=torch.int16, device="cuda")
    refused(lambda: B.sparse_ffn_compact(W, torch.tensor([0, 3, N, 5], dtype=torch.int32,
                                                         device="cuda"), 4, False, out), "idx[2]")
    # tiered: a middle-tier index beyond the input columns
    n_in, d_out = 512, 256
    Wt = dev(synth.weight_bf16(3, synth.W_C2, 0, 0, synth.T_DOWN, n_in, d_out))
    rec_b = B.tier_record_bytes(d_out, 1)
    rec = torch.zeros(n_in, rec_b, dtype=torch.uint8, device="cuda")
    B.sparse_ffn_encode_tiers(Wt, [0, d_out], rec)
    top = torch.arange(0, 40, dtype=torch.int32, device="cuda")
    mid = torch.arange(40, 100, dtype=torch.int32, device="cuda"); mid[9] = n_in + 3
    yt = torch.zeros(d_out, device="cuda")
    refused(lambda: B.sparse_ffn_tiered_gemv(Wt, rec, [0, d_out], torch.randn(n_in, device="cuda"),
                                             top, cnt(40), 40, mid, cnt(60), 60, yt,
                                             workspace=B.new_workspace(1, 100, d_out)), "(mid)")
