"""Python binding of libtopk_transform.so (the gfx950 fused top-k + page-table transform).

Argument marshalling only: every step of the operation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is not built, or the call fails, this raises.

The C entry points have the same names; see include/topk_transform.h and
include/indexer_topk.h for the argument meaning, layouts, ownership and error
behaviour.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

from .build import LIB_PATH

TOPK_MAX_K = 2048
STREAM_SHAPES = 3   # compiled streaming-kernel shapes: topk_set_stream_shape accepts -1 and 0..STREAM_SHAPES-1
SPLIT_STREAM_SHAPES = 2   # compiled split streaming shapes: topk_set_split_stream accepts -1 and 0..1
STATUS = {0: "TOPK_SUCCESS", 1: "TOPK_ERROR_INVALID_VALUE", 2: "TOPK_ERROR_UNSUPPORTED",
          3: "TOPK_ERROR_OUT_OF_MEMORY", 4: "TOPK_ERROR_LAUNCH", 5: "TOPK_ERROR_DEVICE_FAULT"}
TOPK_ERROR_DEVICE_FAULT = 5

EXPORTED = ("topk_transform", "topk_transform_sorted", "topk_transform_noalloc", "topk_init", "topk_status_string", "topk_last_error", "topk_last_launch",
            "topk_release_workspaces", "topk_set_dispatch_override", "topk_set_stream_shape", "topk_set_split_stream",
            "topk_set_sorted_finish",
            "topk_check_faults", "topk_set_wait_limit", "topk_set_scratch_limit", "topk_abi_version",
            "indexer_logits", "indexer_topk",
            "indexer_set_window_override", "indexer_set_select_mode")
INDEXER_HEADS = 32
INDEXER_HEAD_DIM = 128

_lib: Optional[ctypes.CDLL] = None


class TopkError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    try:  # make torch's HIP runtime the one the library binds to, when torch is present
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    c_i32, c_i64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    for fn in (lib.topk_transform, lib.topk_transform_sorted, lib.topk_transform_noalloc):
        fn.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64]
        fn.restype = ctypes.c_int
    lib.topk_init.argtypes = []
    lib.topk_init.restype = ctypes.c_int
    lib.topk_status_string.argtypes = [ctypes.c_int]
    lib.topk_status_string.restype = ctypes.c_char_p
    lib.topk_last_error.argtypes = []
    lib.topk_last_error.restype = ctypes.c_char_p
    lib.topk_last_launch.argtypes = []
    lib.topk_last_launch.restype = ctypes.c_char_p
    lib.topk_release_workspaces.argtypes = []
    lib.topk_release_workspaces.restype = ctypes.c_int
    lib.topk_set_dispatch_override.argtypes = [c_i32, c_i32]
    lib.topk_set_dispatch_override.restype = ctypes.c_int
    lib.topk_set_stream_shape.argtypes = [c_i32]
    lib.topk_set_stream_shape.restype = ctypes.c_int
    lib.topk_set_sorted_finish.argtypes = [c_i32]
    lib.topk_set_sorted_finish.restype = ctypes.c_int
    lib.topk_set_split_stream.argtypes = [c_i32, c_i32]
    lib.topk_set_split_stream.restype = ctypes.c_int
    lib.topk_check_faults.argtypes = [c_vp]
    lib.topk_check_faults.restype = ctypes.c_int
    lib.topk_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.topk_set_wait_limit.restype = ctypes.c_int
    lib.topk_set_scratch_limit.argtypes = [ctypes.c_uint64]
    lib.topk_set_scratch_limit.restype = ctypes.c_int
    lib.topk_abi_version.argtypes = []
    lib.topk_abi_version.restype = c_i32
    lib.indexer_logits.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64]
    lib.indexer_logits.restype = ctypes.c_int
    lib.indexer_topk.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i64]
    lib.indexer_topk.restype = ctypes.c_int
    lib.indexer_set_window_override.argtypes = [c_i64]
    lib.indexer_set_window_override.restype = ctypes.c_int
    lib.indexer_set_select_mode.argtypes = [c_i32]
    lib.indexer_set_select_mode.restype = ctypes.c_int
    _lib = lib
    return lib


_raw_stream = None   # torch's accessor of the current stream's raw handle, when it has one


def _stream_handle(stream, dev) -> int:
    """The HIP stream handle for a call: `stream`'s, or the current stream of
    device `dev`.  The current stream is read through torch's raw accessor
    (the one torch._dynamo uses), which builds no Stream object: about 0.2 us
    per call instead of 2 us."""
    global _raw_stream
    if stream is not None:
        return stream.cuda_stream
    import torch
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream and dev.index is not None:
        return _raw_stream(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int) -> None:
    if status != 0:
        text = load().topk_last_error().decode(errors="replace")
        if status == 1:
            raise ValueError(f"{STATUS[1]}: {text}")
        raise TopkError(status, text)


def topk_transform(scores, seq_lens, page_table, k: int, page_size: int, out=None, out_raw=None,
                   want_raw: bool = False, stream=None) -> Tuple[object, Optional[object]]:
    """Exact per-row top-k of `scores` fused with the page-table transform.

    scores (B, W) float32, seq_lens (B,) int32, page_table (B, P) int32, all
    contiguous on one GPU.  Returns (out (B, k) int32, out_raw (B, k) int32 or
    None).  `out` / `out_raw` may be passed preallocated; `want_raw` allocates
    out_raw when it is not passed.  The call is asynchronous on `stream`
    (default: torch's current stream of the tensors' device).  The selected
    positions of a row come in no particular order.
    """
    return _call(load().topk_transform, scores, seq_lens, page_table, k, page_size, out, out_raw, want_raw, stream)


def topk_transform_sorted(scores, seq_lens, page_table, k: int, page_size: int, out=None, out_raw=None,
                          want_raw: bool = False, stream=None) -> Tuple[object, Optional[object]]:
    """As topk_transform, deterministic: each row's selected positions by score
    descending, equal scores by position ascending, the lowest tied positions
    taken at the threshold (the plain definition's order)."""
    return _call(load().topk_transform_sorted, scores, seq_lens, page_table, k, page_size, out, out_raw, want_raw,
                 stream)


def topk_transform_noalloc(scores, seq_lens, page_table, k: int, page_size: int, out, out_raw=None,
                           stream=None) -> Tuple[object, Optional[object]]:
    """As topk_transform, through the entry point that allocates nothing: its
    workspace is the library's static device scratch, and `out` (and
    `out_raw`, if wanted) must be passed preallocated.  Calls that overlap on
    one device race on the scratch."""
    if out is None:
        raise ValueError("topk_transform_noalloc needs a preallocated out")
    return _call(load().topk_transform_noalloc, scores, seq_lens, page_table, k, page_size, out, out_raw, False,
                 stream)


def topk_init() -> None:
    """Sets up the current device (also the pinned page of fault words)."""
    _check(load().topk_init())


def _call(fn, scores, seq_lens, page_table, k, page_size, out, out_raw, want_raw, stream):
    import torch
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous 2-D float32 tensor")
    B, W = scores.shape
    dev = scores.device
    if seq_lens.shape != (B,) or seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape (B,)")
    if (page_table.dim() != 2 or page_table.shape[0] != B or page_table.dtype != torch.int32
            or not page_table.is_contiguous()):
        raise ValueError("page_table must be a contiguous int32 tensor of shape (B, P)")
    if dev.type != "cuda" or seq_lens.device != dev or page_table.device != dev:
        raise ValueError("scores, seq_lens and page_table must be on one GPU")
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=dev)
    elif (out.shape != (B, k) or out.dtype != torch.int32 or not out.is_contiguous() or out.device != dev):
        raise ValueError("out must be a contiguous int32 tensor of shape (B, k)")
    if out_raw is None and want_raw:
        out_raw = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out_raw is not None and (out_raw.shape != (B, k) or out_raw.dtype != torch.int32
                                or not out_raw.is_contiguous() or out_raw.device != dev):
        raise ValueError("out_raw must be a contiguous int32 tensor of shape (B, k)")
    args = (scores.data_ptr(), seq_lens.data_ptr(), page_table.data_ptr(), int(k), int(page_size), out.data_ptr(),
            out_raw.data_ptr() if out_raw is not None else None, _stream_handle(stream, dev), int(B), int(W),
            int(page_table.shape[1]))
    # The library works on the current device: switch only when the tensors
    # live on another one (the switch costs a device get/set round trip).
    if dev.index is None or dev.index == torch.cuda.current_device():
        st = fn(*args)
    else:
        with torch.cuda.device(dev):
            st = fn(*args)
    _check(st)
    return out, out_raw


def topk_status_string(status: int) -> str:
    return load().topk_status_string(int(status)).decode()


def topk_last_error() -> str:
    return load().topk_last_error().decode(errors="replace")


def topk_last_launch() -> str:
    return load().topk_last_launch().decode(errors="replace")


def topk_release_workspaces() -> None:
    _check(load().topk_release_workspaces())


def topk_set_dispatch_override(elems_per_thread: int = 0, wgs_per_row: int = 0) -> None:
    _check(load().topk_set_dispatch_override(int(elems_per_thread), int(wgs_per_row)))


def topk_set_split_stream(shape: int = -1, wgs_per_row: int = 0) -> None:
    """Testing/tuning override: force the split streaming kernel's shape with
    `wgs_per_row` workgroups per row (shape -1 restores automatic dispatch)."""
    _check(load().topk_set_split_stream(int(shape), int(wgs_per_row)))


def topk_set_stream_shape(shape: int = -1) -> None:
    _check(load().topk_set_stream_shape(int(shape)))


def topk_set_sorted_finish(mode: int = -1) -> None:
    """Testing/tuning override of the sorted finish: -1 automatic, 0 one
    workgroup per row (LDS bitonic sort), 1 rank finish (G workgroups per row)."""
    _check(load().topk_set_sorted_finish(int(mode)))


def topk_check_faults(stream=None) -> None:
    """Synchronises `stream` (default: torch's current stream) and raises
    TopkError(TOPK_ERROR_DEVICE_FAULT) once for each split-row launch on it
    whose bounded cross-workgroup wait gave up since the last report."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    _check(load().topk_check_faults(ctypes.c_void_p(stream.cuda_stream)))


def topk_set_wait_limit(polls: int = 0) -> None:
    """Testing override: polls of a split-row barrier wait before it gives up (0 = default)."""
    _check(load().topk_set_wait_limit(int(polls)))


def topk_set_scratch_limit(words: int = 0) -> None:
    """Testing override: 32-bit words of the static scratch topk_transform_noalloc may use (0 = all)."""
    _check(load().topk_set_scratch_limit(int(words)))


def topk_abi_version() -> int:
    return int(load().topk_abi_version())


def _indexer_inputs(q, weights, kv, kv_scale, ks, ke):
    import torch
    dev = q.device
    H, D = INDEXER_HEADS, INDEXER_HEAD_DIM
    if q.dim() != 3 or tuple(q.shape[1:]) != (H, D) or q.dtype != torch.uint8 or not q.is_contiguous():
        raise ValueError("q must be a contiguous uint8 (fp8 E4M3 codes) tensor of shape (num_q, 32, 128)")
    nq = q.shape[0]
    if weights.shape != (nq, H) or weights.dtype != torch.float32 or not weights.is_contiguous() \
            or weights.device != dev:
        raise ValueError("weights must be a contiguous float32 tensor of shape (num_q, 32) on q's device")
    if kv.dim() != 2 or kv.shape[1] != D or kv.dtype != torch.uint8 or not kv.is_contiguous() or kv.device != dev:
        raise ValueError("kv must be a contiguous uint8 (fp8 E4M3 codes) tensor of shape (num_kv, 128) on q's device")
    nkv = kv.shape[0]
    if (kv_scale.shape != (nkv,) or kv_scale.dtype != torch.float32 or not kv_scale.is_contiguous()
            or kv_scale.device != dev):
        raise ValueError("kv_scale must be a contiguous float32 tensor of shape (num_kv,) on q's device")
    for name, t in (("ks", ks), ("ke", ke)):
        if t.shape != (nq,) or t.dtype != torch.int32 or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor of shape (num_q,) on q's device")
    if dev.type != "cuda":
        raise ValueError("the indexer inputs must be on a GPU")
    return dev, nq, nkv


def indexer_logits(q, weights, kv, kv_scale, ks, ke, width: int, out=None, stream=None):
    """Dense indexer scores: out[r, c] = score of position ks[r] + c (c < ke[r] - ks[r]
    and c < width); other entries are left as they are.  Returns out (num_q, width) float32."""
    import torch
    dev, nq, nkv = _indexer_inputs(q, weights, kv, kv_scale, ks, ke)
    if out is None:
        out = torch.empty((nq, int(width)), dtype=torch.float32, device=dev)
    elif out.shape != (nq, int(width)) or out.dtype != torch.float32 or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous float32 tensor of shape (num_q, width)")
    handle = _stream_handle(stream, dev)
    with torch.cuda.device(dev):
        st = load().indexer_logits(q.data_ptr(), weights.data_ptr(), kv.data_ptr(), kv_scale.data_ptr(),
                                   ks.data_ptr(), ke.data_ptr(), out.data_ptr(), handle, int(nq), int(nkv), int(width))
    _check(st)
    return out


def indexer_topk(q, weights, kv, kv_scale, ks, ke, k: int, out=None, stream=None):
    """Fused indexer scoring + exact top-k: out (num_q, k) int32 absolute key positions,
    -1 padded, order within a row unspecified."""
    import torch
    dev, nq, nkv = _indexer_inputs(q, weights, kv, kv_scale, ks, ke)
    if out is None:
        out = torch.empty((nq, int(k)), dtype=torch.int32, device=dev)
    elif out.shape != (nq, int(k)) or out.dtype != torch.int32 or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous int32 tensor of shape (num_q, k)")
    handle = _stream_handle(stream, dev)
    with torch.cuda.device(dev):
        st = load().indexer_topk(q.data_ptr(), weights.data_ptr(), kv.data_ptr(), kv_scale.data_ptr(),
                                 ks.data_ptr(), ke.data_ptr(), int(k), out.data_ptr(), handle, int(nq), int(nkv))
    _check(st)
    return out


def indexer_set_window_override(window: int = 0) -> None:
    """Key positions per workgroup window (0 = automatic; else a multiple of 64)."""
    _check(load().indexer_set_window_override(int(window)))


def indexer_set_select_mode(mode: int = -1) -> None:
    """Testing/tuning override of indexer_topk's internal form: -1 automatic,
    0 the fused scan, 1 dense scores into a buffer + select."""
    _check(load().indexer_set_select_mode(int(mode)))
