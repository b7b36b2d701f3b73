"""Python binding of libsparse_ffn.so (include/sparse_ffn.h).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, passes their device pointers, sizes and torch's current
HIP stream to the C entry point of the same name, and raises
:class:`SffnError` on a non-OK status.  Every step of the computation runs
in the library's HIP kernels; there is no fallback of any kind, and a
missing library is an error.
"""

from __future__ import annotations

import ctypes
import os

import torch  # imported first so the library binds to torch's HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_ffn.so")

SFFN_OK, SFFN_EINVAL, SFFN_EUNSUPPORTED, SFFN_EWORKSPACE, SFFN_EHIP = range(5)
KEY_ABS_F32, KEY_U32, KEY_F32 = 0, 1, 2
SCORE_SUM_ABS, SCORE_CLUSTER_MAX, SCORE_SOFTMAX_PICKED = 0, 1, 2
OP_GLU_SILU, OP_DOT_RELU, OP_GATED, OP_AXPY, OP_DOT, OP_GLU_RELU, OP_PREDICT = 0, 1, 2, 3, 4, 5, 6
OP_DOT_RELU_CLUSTER = 7
PACKED = 0x100                                  # op flag: W0 / W1 in a packed layout
MASKED_ROWS = 0x200                             # op flag: AXPY over the rows some token's mask selects
LAYOUT_ROW_TILES, LAYOUT_COL_PANELS = 1, 2

_STATUS = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "EWORKSPACE", 4: "EHIP"}


class SffnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libsparse_ffn.so (built in-tree by ``build.py``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m activation_sparse_decode_amd.build`"
                " (there is no fallback path)")
        L = ctypes.CDLL(_LIB_PATH)
        L.sffn_last_error.restype = ctypes.c_char_p
        L.sffn_abi_version.restype = _i
        L.sparse_ffn_workspace_size.restype = _sz
        L.sparse_ffn_workspace_size.argtypes = [_i, _i, _i]
        L.sparse_ffn_tier_record_bytes.restype = _sz
        L.sparse_ffn_tier_record_bytes.argtypes = [_i, _i]
        L.sparse_ffn_score.restype = _i
        L.sparse_ffn_score.argtypes = [_i, _vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp]
        L.sparse_ffn_select.restype = _i
        L.sparse_ffn_select.argtypes = [_vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                                        _i, _vp, _i, _vp, _vp, _i, _vp, _vp, _i, _vp]
        L.sparse_ffn_row_norms.restype = _i
        L.sparse_ffn_row_norms.argtypes = [_vp, _i, _i, _i, _vp, _vp]
        L.sparse_ffn_gemv.restype = _i
        L.sparse_ffn_gemv.argtypes = [_i, _vp, _vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _i, _i,
                                      _vp, _i, _f, _f, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _sz, _vp]
        L.sparse_ffn_gemv_noalloc.restype = _i
        L.sparse_ffn_gemv_noalloc.argtypes = [_i, _vp, _vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _i,
                                              _i, _vp, _i, _f, _f, _vp, _i, _vp, _vp, _vp, _i, _i,
                                              _vp]
        L.sparse_ffn_gemv_lists.restype = _i
        L.sparse_ffn_gemv_lists.argtypes = [_i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _i, _vp,
                                            _vp, _i, _vp, _sz, _vp]
        L.sparse_ffn_rowop_lists.restype = _i
        L.sparse_ffn_rowop_lists.argtypes = [_i, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp,
                                             _i, _f, _f, _vp, _vp, _vp, _i, _vp]
        L.sparse_ffn_compact.restype = _i
        L.sparse_ffn_compact.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _vp, _i, _vp]
        L.sparse_ffn_gather.restype = _i
        L.sparse_ffn_gather.argtypes = [_vp, _i, _vp, _vp, _i, _vp, _vp]
        L.sparse_ffn_encode_tiers.restype = _i
        L.sparse_ffn_encode_tiers.argtypes = [_vp, _i, _i, _i, _vp, _i, _vp, _i, _vp]
        L.sparse_ffn_tiered_gemv.restype = _i
        L.sparse_ffn_tiered_gemv.argtypes = [_vp, _i, _vp, _i, _vp, _i, _i, _i, _vp, _vp, _vp, _i,
                                             _vp, _vp, _i, _vp, _i, _vp, _sz, _vp]
        L.sparse_ffn_fused_swiglu.restype = _i
        L.sparse_ffn_fused_swiglu.argtypes = [_vp, _vp, _vp, _i, _i, _i, _vp, _f, _vp, _vp, _i,
                                              _vp, _vp, _i, _vp, _sz, _vp]
        L.sparse_ffn_packed_elems.restype = _sz
        L.sparse_ffn_packed_elems.argtypes = [_i, _i, _i]
        L.sparse_ffn_pack_weights.restype = _i
        L.sparse_ffn_pack_weights.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp]
        L.sparse_ffn_select_threshold.restype = _i
        L.sparse_ffn_select_threshold.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]
        L.sparse_ffn_gemv_keyed.restype = _i
        L.sparse_ffn_gemv_keyed.argtypes = [_vp, _i, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _vp, _i,
                                            _vp, _sz, _vp]
        L.sparse_ffn_tiered_gemv_keyed.restype = _i
        L.sparse_ffn_tiered_gemv_keyed.argtypes = [_vp, _i, _vp, _i, _vp, _i, _i, _i, _vp, _vp, _i,
                                                   _vp, _vp, _i, _i, _vp, _i, _vp, _sz, _vp]
        if L.sffn_abi_version() != 17:
            raise RuntimeError("libsparse_ffn.so ABI version mismatch; rebuild it")
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != SFFN_OK:
        raise SffnError(status, lib().sffn_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ld(t, default: int) -> int:
    return t.stride(0) if (t is not None and t.dim() == 2) else default


class PackedWeights:
    """A weight matrix in a packed layout of the batched kernels: the flat
    packed data and the logical [n_rows][d] shape (built by pack_weights)."""

    def __init__(self, data: torch.Tensor, n_rows: int, d: int, layout: int):
        self.data, self.n_rows, self.d, self.layout = data, n_rows, d, layout

    @property
    def shape(self):
        return (self.n_rows, self.d)


def _weights(op: int, W0, W1):
    """Pointers, op and shape for row-major tensors or PackedWeights."""
    W = W0 if W0 is not None else W1
    if isinstance(W, PackedWeights):
        ptr = lambda w: None if w is None else ctypes.c_void_p(w.data.data_ptr())  # noqa: E731
        return op | PACKED, ptr(W0), ptr(W1), W.n_rows, W.d, W.d
    return op, _p(W0), _p(W1), W.shape[0], W.shape[1], W.stride(0)


# ------------------------------------------------------------------ sizes

def workspace_size(batch: int, n_rows: int, d_out: int) -> int:
    return int(lib().sparse_ffn_workspace_size(batch, n_rows, d_out))


def tier_record_bytes(d_out: int, n_seg: int) -> int:
    return int(lib().sparse_ffn_tier_record_bytes(d_out, n_seg))


def new_workspace(batch: int, n_rows: int, d_out: int, device="cuda") -> torch.Tensor:
    """A workspace of the size the gathered products need."""
    return torch.zeros(workspace_size(batch, n_rows, d_out), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def sparse_ffn_score(mode: int, inp: torch.Tensor, out: torch.Tensor, *, cluster: int = 1,
                     accumulate: bool = False, picked: torch.Tensor | None = None,
                     stream=None) -> None:
    T, n = (inp.shape[0], inp.shape[1]) if inp.dim() == 2 else (1, inp.shape[0])
    k = picked.shape[-1] if picked is not None else 0
    _check(lib().sparse_ffn_score(mode, _p(inp), T, n, _ld(inp, n), cluster, int(accumulate),
                                  _p(picked), k, _p(out), _stream(stream)))


def sparse_ffn_select(keys: torch.Tensor, key_type: int, r_lo: int, r_hi: int, *,
                      cluster: int = 1, nonzero_only: bool = False,
                      include_mask: torch.Tensor | None = None,
                      exclude_mask: torch.Tensor | None = None,
                      mask_out: torch.Tensor | None = None, idx_out: torch.Tensor | None = None,
                      count_out: torch.Tensor | None = None,
                      idx_top_out: torch.Tensor | None = None,
                      count_top_out: torch.Tensor | None = None,
                      freq: torch.Tensor | None = None, key_scale: torch.Tensor | None = None,
                      clear_keys: bool = False, stream=None) -> None:
    rows, width = (keys.shape[0], keys.shape[1]) if keys.dim() == 2 else (1, keys.shape[0])
    n = width // cluster
    _check(lib().sparse_ffn_select(
        _p(keys), key_type, _p(key_scale), rows, n, _ld(keys, width), cluster, r_lo, r_hi,
        int(nonzero_only),
        _p(include_mask), _p(exclude_mask), _p(mask_out), _ld(mask_out, n), _p(idx_out),
        _ld(idx_out, idx_out.shape[-1] if idx_out is not None else 0), _p(count_out),
        _p(idx_top_out), _ld(idx_top_out, idx_top_out.shape[-1] if idx_top_out is not None else 0),
        _p(count_top_out), _p(freq), int(clear_keys), _stream(stream)))


def sparse_ffn_select_threshold(keys: torch.Tensor, key_type: int, k: int, thr_out: torch.Tensor,
                                stream=None, *, k_top: int = 0,
                                thr_top_out: torch.Tensor | None = None) -> None:
    """Per row of keys ([n] or [rows][n]): the top-k range [0, k) as a
    threshold pair (T, I) in thr_out (int32/uint32 [rows][2] or [2]), and
    with thr_top_out the pair of [0, k_top) there."""
    rows, n = (keys.shape[0], keys.shape[1]) if keys.dim() == 2 else (1, keys.shape[0])
    _check(lib().sparse_ffn_select_threshold(_p(keys), key_type, rows, n, _ld(keys, n), k_top, k,
                                             _p(thr_top_out), _p(thr_out), _stream(stream)))


def sparse_ffn_gemv_keyed(W: torch.Tensor, inp: torch.Tensor, keys: torch.Tensor, key_type: int,
                          thr: torch.Tensor, k_max: int, out: torch.Tensor, *,
                          alpha: torch.Tensor | None = None, accumulate: bool = False,
                          workspace: torch.Tensor | None = None, stream=None) -> None:
    """out (+)= alpha * sum of inp[n] * W[n] over the rows the threshold thr
    selects among keys (batch 1)."""
    n_rows, d = W.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sparse_ffn_gemv_keyed(_p(W), n_rows, d, _ld(W, d), _p(inp), _p(keys), key_type,
                                       _p(thr), k_max, _p(alpha), _p(out), int(accumulate),
                                       _p(workspace), ws_bytes, _stream(stream)))


def sparse_ffn_gemv(op: int, W0: torch.Tensor | None, W1: torch.Tensor | None,
                    inp: torch.Tensor, out: torch.Tensor, *, idx: torch.Tensor | None = None,
                    count: torch.Tensor | None = None, k_max: int = 0, group: int = 1,
                    row_mask: torch.Tensor | None = None, tau_scale: float = 0.0,
                    rms_eps: float = 0.0,
                    aux: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                    key_out: torch.Tensor | None = None, accumulate: bool = False,
                    workspace: torch.Tensor | None = None, stream=None) -> None:
    op, p0, p1, n_rows, d, ld_w = _weights(op, W0, W1)
    batch = inp.shape[0] if inp.dim() == 2 else 1
    ld_in = _ld(inp, inp.shape[-1])
    ld_out = _ld(out, out.shape[-1])
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_ffn_gemv(
        op, p0, p1, n_rows, d, ld_w, _p(inp), batch, ld_in, _p(idx), _p(count),
        k_max, group, _p(row_mask), _ld(row_mask, n_rows), float(tau_scale), float(rms_eps), _p(aux),
        _ld(aux, n_rows), _p(alpha), _p(out), _p(key_out), ld_out, int(accumulate),
        _p(workspace), ws_bytes, _stream(stream)))


def sparse_ffn_gemv_noalloc(op: int, W0: torch.Tensor | None, W1: torch.Tensor | None,
                            inp: torch.Tensor, out: torch.Tensor, *,
                            idx: torch.Tensor | None = None, count: torch.Tensor | None = None,
                            k_max: int = 0, group: int = 1,
                            row_mask: torch.Tensor | None = None, tau_scale: float = 0.0,
                            rms_eps: float = 0.0, aux: torch.Tensor | None = None,
                            alpha: torch.Tensor | None = None,
                            key_out: torch.Tensor | None = None, accumulate: bool = False,
                            stream=None) -> None:
    """sparse_ffn_gemv without a workspace: AXPY's scratch is the library's
    static per-GPU array (shared by every call on that GPU)."""
    op, p0, p1, n_rows, d, ld_w = _weights(op, W0, W1)
    batch = inp.shape[0] if inp.dim() == 2 else 1
    _check(lib().sparse_ffn_gemv_noalloc(
        op, p0, p1, n_rows, d, ld_w, _p(inp), batch, _ld(inp, inp.shape[-1]),
        _p(idx), _p(count), k_max, group, _p(row_mask), _ld(row_mask, n_rows), float(tau_scale),
        float(rms_eps), _p(aux), _ld(aux, n_rows), _p(alpha), _p(out), _p(key_out),
        _ld(out, out.shape[-1]), int(accumulate), _stream(stream)))


def sparse_ffn_fused_swiglu(Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor,
                            x: torch.Tensor, y: torch.Tensor, *, idx: torch.Tensor | None = None,
                            count: torch.Tensor | None = None, k_max: int = 0,
                            rms_eps: float = 0.0, a_out: torch.Tensor | None = None,
                            accumulate: bool = False, workspace: torch.Tensor | None = None,
                            stream=None) -> None:
    """One sparse SwiGLU FFN at batch 1, a pass per neuron (gate, up, silu *
    mul, down row).  Wg / Wu / Wd are [n_rows][d] views with one row stride
    (e.g. the three column blocks of a [n][3d] per-neuron record buffer)."""
    n_rows, d = Wg.shape[0], Wg.shape[1]
    ld_w = Wg.stride(0)
    if Wu.stride(0) != ld_w or Wd.stride(0) != ld_w:
        raise ValueError("Wg, Wu and Wd must share one row stride")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_ffn_fused_swiglu(
        _p(Wg), _p(Wu), _p(Wd), n_rows, d, ld_w, _p(x), float(rms_eps), _p(idx), _p(count),
        k_max, _p(a_out), _p(y), int(accumulate), _p(workspace), ws_bytes, _stream(stream)))


def packed_elems(n_rows: int, d: int, layout: int) -> int:
    return int(lib().sparse_ffn_packed_elems(n_rows, d, layout))


def pack_weights(W: torch.Tensor, layout: int, out: torch.Tensor | None = None,
                 stream=None) -> PackedWeights:
    """W [n_rows][d] (row-major bf16 bits) re-laid in a packed layout of the
    batched kernels (LAYOUT_ROW_TILES for row ops, LAYOUT_COL_PANELS for AXPY)."""
    n_rows, d = W.shape[0], W.shape[1]
    n_out = packed_elems(n_rows, d, layout)
    if out is None:
        out = torch.empty(max(n_out, 8), dtype=torch.int16, device=W.device)
    _check(lib().sparse_ffn_pack_weights(_p(W), n_rows, d, W.stride(0), layout, _p(out),
                                         _stream(stream)))
    return PackedWeights(out, n_rows, d, layout)


def sparse_ffn_row_norms(W: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _check(lib().sparse_ffn_row_norms(_p(W), W.shape[0], W.shape[1], W.stride(0), _p(out),
                                      _stream(stream)))


def sparse_ffn_gemv_lists(Ws, ins, idxs, counts, k_maxs, out: torch.Tensor, *, group: int = 1,
                          alphas=None, accumulate: bool = False,
                          workspace: torch.Tensor | None = None, stream=None) -> None:
    """One gathered product over several row lists into ``out`` (batch 1):
    list l reads rows of ``Ws[l]`` picked by ``idxs[l]`` / ``counts[l]``,
    weighted by ``ins[l]`` and the device scalar ``alphas[l]`` (or 1)."""
    n = len(Ws)
    ptrs = lambda ts: (_vp * n)(*[None if t is None else t.data_ptr() for t in ts])  # noqa: E731
    ints = lambda vs: (_i * n)(*[int(v) for v in vs])  # noqa: E731
    d, ld_w = Ws[0].shape[1], Ws[0].stride(0)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_ffn_gemv_lists(
        n, ptrs(Ws), ints([w.shape[0] for w in Ws]), d, ld_w, ptrs(ins), ptrs(idxs), ptrs(counts),
        ints(k_maxs), group, None if alphas is None else ptrs(alphas), _p(out), int(accumulate),
        _p(workspace), ws_bytes, _stream(stream)))


def sparse_ffn_gather(src: torch.Tensor, idx: torch.Tensor, dst: torch.Tensor, *,
                      count: torch.Tensor | None = None, k_max: int | None = None,
                      stream=None) -> None:
    """dst[i] = src[idx[i]] (4-byte elements) for i < min(*count, k_max)."""
    k = idx.shape[0] if k_max is None else k_max
    _check(lib().sparse_ffn_gather(_p(src), src.numel(), _p(idx), _p(count), k, _p(dst),
                                   _stream(stream)))


def sparse_ffn_rowop_lists(op: int, W0s, W1s, x: torch.Tensor, outs, *, idxs=None, counts=None,
                           k_maxs=None, group: int = 1, tau_scale: float = 0.0,
                           rms_eps: float = 0.0, auxs=None, key_outs=None,
                           accumulate: bool = False, stream=None) -> None:
    """One row op over several row lists (batch 1): list l reads W0s[l] /
    W1s[l] and writes outs[l] (and key_outs[l]) as sparse_ffn_gemv would."""
    n = len(outs)
    ptrs = lambda ts: None if ts is None else (_vp * n)(  # noqa: E731
        *[None if t is None else t.data_ptr() for t in ts])
    ints = lambda vs: None if vs is None else (_i * n)(*[int(v) for v in vs])  # noqa: E731
    W = next(w for w in (list(W0s or []) + list(W1s or [])) if w is not None)
    _check(lib().sparse_ffn_rowop_lists(
        op, n, ptrs(W0s), ptrs(W1s), W.shape[0], W.shape[1], W.stride(0), _p(x), ptrs(idxs),
        ptrs(counts), ints(k_maxs), group, float(tau_scale), float(rms_eps), ptrs(auxs),
        ptrs(outs), ptrs(key_outs), int(accumulate), _stream(stream)))


def sparse_ffn_compact(W: torch.Tensor, idx: torch.Tensor | None, k: int, transpose: bool,
                       out: torch.Tensor, stream=None) -> None:
    _check(lib().sparse_ffn_compact(_p(W), W.shape[0], W.shape[1], W.stride(0), _p(idx), k,
                                    int(transpose), _p(out), out.stride(0), _stream(stream)))


def _seg_array(seg_rows):
    arr = (ctypes.c_int32 * len(seg_rows))(*[int(v) for v in seg_rows])
    return arr, len(seg_rows) - 1


def sparse_ffn_encode_tiers(Wt: torch.Tensor, seg_rows, mid_rec: torch.Tensor,
                            stream=None) -> None:
    arr, n_seg = _seg_array(seg_rows)
    _check(lib().sparse_ffn_encode_tiers(
        _p(Wt), Wt.stride(0), Wt.shape[0], Wt.shape[1], arr, n_seg, _p(mid_rec),
        mid_rec.stride(0), _stream(stream)))


def sparse_ffn_tiered_gemv(Wt: torch.Tensor, mid_rec: torch.Tensor, seg_rows, x: torch.Tensor,
                           idx_top, cnt_top, k_top_max: int, idx_mid, cnt_mid, k_mid_max: int,
                           y: torch.Tensor, *, accumulate: bool = False,
                           workspace: torch.Tensor | None = None, stream=None) -> None:
    arr, n_seg = _seg_array(seg_rows)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_ffn_tiered_gemv(
        _p(Wt), Wt.stride(0), _p(mid_rec), mid_rec.stride(0), arr, n_seg, Wt.shape[0],
        Wt.shape[1], _p(x), _p(idx_top), _p(cnt_top), k_top_max, _p(idx_mid), _p(cnt_mid),
        k_mid_max, _p(y), int(accumulate), _p(workspace), ws_bytes, _stream(stream)))


def sparse_ffn_tiered_gemv_keyed(Wt: torch.Tensor, mid_rec: torch.Tensor, seg_rows,
                                 x: torch.Tensor, keys: torch.Tensor, key_type: int,
                                 thr_top: torch.Tensor, thr: torch.Tensor, k_top_max: int,
                                 k_mid_max: int, y: torch.Tensor, *, accumulate: bool = False,
                                 workspace: torch.Tensor | None = None, stream=None) -> None:
    """The three-tier read with the tiers given as threshold pairs over keys."""
    arr, n_seg = _seg_array(seg_rows)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_ffn_tiered_gemv_keyed(
        _p(Wt), Wt.stride(0), _p(mid_rec), mid_rec.stride(0), arr, n_seg, Wt.shape[0],
        Wt.shape[1], _p(x), _p(keys), key_type, _p(thr_top), _p(thr), k_top_max, k_mid_max,
        _p(y), int(accumulate), _p(workspace), ws_bytes, _stream(stream)))
