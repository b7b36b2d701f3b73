"""The allocation-free gemv (static per-GPU scratch) against sparse_ffn_gemv
with its own workspace: bitwise the same outputs (same kernels, same
reduction order) and within tolerance of the oracle, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's partials,
which the second must not pick up)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]


def gathered_case(seed, N, d, k, batch):
    WdT = synth.weight_bf16(seed, synth.W_C4, 0, 0, synth.T_DOWN, N, d)
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((batch, N)).astype(np.float32)
    U = np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)
    M = np.zeros((batch, N), np.uint8)
    for b in range(batch):
        M[b, rng.choice(U, size=max(1, (3 * k) // 5), replace=False)] = 1
    return WdT, A, U, M


def run_both(WdT, A, U, M, batch, packed=False):
    N, d = WdT.shape
    W, Ad, Ud = dev(WdT), dev(A if batch > 1 else A[0]), dev(U)
    if packed:
        W = B.pack_weights(W, B.LAYOUT_COL_PANELS)
    cnt = torch.tensor([U.size], dtype=torch.int32, device="cuda")
    Md = dev(M) if batch > 1 else None
    shape = (batch, d) if batch > 1 else (d,)
    y_ws = torch.full(shape, 3.0, dtype=torch.float32, device="cuda")
    y_na = torch.full(shape, 3.0, dtype=torch.float32, device="cuda")
    ws = B.new_workspace(batch, N, d)
    B.sparse_ffn_gemv(B.OP_AXPY, W, None, Ad, y_ws, idx=Ud, count=cnt, k_max=N, row_mask=Md,
                      accumulate=True, workspace=ws)
    B.sparse_ffn_gemv_noalloc(B.OP_AXPY, W, None, Ad, y_na, idx=Ud, count=cnt, k_max=N,
                              row_mask=Md, accumulate=True)
    torch.cuda.synchronize()
    return host(y_ws), host(y_na)


def check(WdT, A, U, M, batch, what, packed=False):
    y_ws, y_na = run_both(WdT, A, U, M, batch, packed)
    assert np.array_equal(y_ws.view(np.uint32), y_na.view(np.uint32)), f"{what}: differs from gemv"
    y_na = y_na.reshape(batch, -1)
    for b in sorted({0, batch - 1}):
        s = np.flatnonzero(M[b]) if batch > 1 else U
        ref = 3.0 + oracle.down_gather(WdT, s.astype(np.int32), A[b, s])
        assert_close(y_na[b], ref, what=f"{what} token {b}")


def test_noalloc_batch1_two_calls():
    banner("noalloc batch 1: 8192x2048 k=4096, then 1000x512 k=300")
    check(*gathered_case(1, 8192, 2048, 4096, 1), 1, "batch 1 large")
    check(*gathered_case(2, 1000, 512, 300, 1), 1, "batch 1 small")


def test_noalloc_batched_two_calls():
    banner("noalloc batch 16: 17408x5120 k=16000, then batch 4 1000x256 k=300")
    check(*gathered_case(3, 17408, 5120, 16000, 16), 16, "batch 16 large")
    check(*gathered_case(4, 1000, 256, 300, 4), 4, "batch 4 small")


def test_noalloc_packed_batched_two_calls():
    """The same with packed column panels (the op flag reaches the static
    scratch path like a row-major AXPY)."""
    banner("noalloc packed: batch 16 17408x5120 k=16000, then batch 4 1000x256 k=300")
    check(*gathered_case(6, 17408, 5120, 16000, 16), 16, "packed batch 16 large", packed=True)
    check(*gathered_case(7, 1000, 256, 300, 4), 4, "packed batch 4 small", packed=True)


def masked_check(seed, N, d, batch, what):
    """The union formed in the product (SFFN_MASKED_ROWS, packed panels)
    through both entries: bitwise equal, and the oracle per token."""
    WdT, A, U, M = gathered_case(seed, N, d, max(1, N // 3), batch)
    ldm = (N + 15) // 16 * 16
    Md = torch.zeros(batch, ldm, dtype=torch.uint8, device="cuda")
    Md[:, :N] = dev(M)
    W = B.pack_weights(dev(WdT), B.LAYOUT_COL_PANELS)
    outs = []
    for noalloc in (False, True):
        y = torch.full((batch, d), 3.0, dtype=torch.float32, device="cuda")
        if noalloc:
            B.sparse_ffn_gemv_noalloc(B.OP_AXPY | B.MASKED_ROWS, W, None, dev(A), y,
                                      row_mask=Md[:, :N], accumulate=True)
        else:
            B.sparse_ffn_gemv(B.OP_AXPY | B.MASKED_ROWS, W, None, dev(A), y, row_mask=Md[:, :N],
                              accumulate=True, workspace=B.new_workspace(batch, N, d))
        torch.cuda.synchronize()
        outs.append(host(y))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), what
    for b in sorted({0, batch - 1}):
        s = np.flatnonzero(M[b])
        assert_close(outs[1][b], 3.0 + oracle.down_gather(WdT, s.astype(np.int32), A[b, s]),
                     what=f"{what} token {b}")


def test_noalloc_masked_rows_two_calls():
    banner("noalloc masked rows: batch 16 17408x5120, then batch 4 1000x256")
    masked_check(8, 17408, 5120, 16, "masked batch 16 large")
    masked_check(9, 1000, 256, 4, "masked batch 4 small")


def test_noalloc_row_op_and_limit():
    banner("noalloc row op and scratch limit")
    N, d = 2000, 1024
    Wg = synth.weight_bf16(5, synth.W_C0, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(5, synth.W_C0, 0, 0, synth.T_UP, N, d)
    x = synth.tokens(5, synth.W_C0, 0, 1, d)[0]
    a1 = torch.zeros(N, dtype=torch.float32, device="cuda")
    a2 = torch.zeros(N, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(x), a1)
    B.sparse_ffn_gemv_noalloc(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(x), a2)
    torch.cuda.synchronize()
    assert np.array_equal(host(a1).view(np.uint32), host(a2).view(np.uint32))
    assert_close(host(a2), oracle.swiglu_acts(Wg, Wu, x), what="GLU")
    # a product whose scratch exceeds the static array is refused before any launch
    W = torch.zeros((64, 1 << 16), dtype=torch.int16, device="cuda")
    a = torch.zeros(64, dtype=torch.float32, device="cuda")
    y = torch.full((1 << 16,), 5.0, dtype=torch.float32, device="cuda")
    with pytest.raises(B.SffnError) as e:
        B.sparse_ffn_gemv_noalloc(B.OP_AXPY, W, None, a, y)
    assert e.value.status == B.SFFN_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
