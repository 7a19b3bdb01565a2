"""Block-hybrid attention on MI355X (gfx950): Python binding of libbha.so.

This module only marshals arguments: it takes PyTorch tensors that live on a
ROCm device, passes their device pointers, element strides and the current
HIP stream to the C ABI declared in ``include/bha.h``, and turns a non-zero
status into an exception. Every step of the computation runs in the library's
HIP kernels; there is no other implementation behind these functions, and they
raise if ``libbha.so`` has not been built.

Tensor conventions (element strides are taken from the tensors themselves):

* tokens ``q, k, v, out, x``: [R][B][H][d], last dimension contiguous,
  bfloat16 or float32 (all of one call share the dtype).
* ``w``: [H][FW][d] (row j of head h is column j of that head's d x FW map)
  or [FW][d] to share one map across heads; same dtype as the tokens.
* ``gamma``: float32 [H].
* ``state``: float32, ``num_slots * H * (d + 1) * 2FW`` elements, any shape
  (``new_state`` makes a zeroed [num_slots][H][record] tensor).
* ``slot_ids``: int32 [R].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BhaError", "library_path", "load_library", "version", "status_string",
    "state_record_floats", "new_state", "feature_map", "block_forward", "state_commit",
    "prepare_forward", "prepare_commit", "state_prefill",
    "BHA_F32", "BHA_BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbha.so")
_BUILT_LIB_PATH = _LIB_PATH
_lib = None

BHA_F32 = 0
BHA_BF16 = 1

# Every symbol include/bha.h declares.
EXPORTED_SYMBOLS = (
    "bha_feature_map", "bha_block_forward", "bha_block_forward_gqa", "bha_block_forward_commit", "bha_state_commit", "bha_state_prefill",
    "bha_prefix_attention", "bha_prefix_attention_workspace", "bha_prefix_attention_noalloc",
    "bha_prefix_attention_noalloc_scratch_bytes",
    "bha_state_record_floats", "bha_status_string", "bha_version", "bha_source_hash",
)


class BhaError(RuntimeError):
    """A bha_* entry point returned a non-zero bha_status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


class bha_dims(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("feat_half", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class bha_strides(ctypes.Structure):
    _fields_ = [("req", ctypes.c_int64), ("tok", ctypes.c_int64), ("head", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libbha.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m linear_attention_block_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    PD, PS = ctypes.POINTER(bha_dims), ctypes.POINTER(bha_strides)
    lib.bha_feature_map.argtypes = [PD, P, PS, P, I64, P, P]
    lib.bha_block_forward.argtypes = [PD, P, P, P, PS, P, I64, P, P, I32, P, P, PS, P]
    lib.bha_state_commit.argtypes = [PD, P, P, PS, P, I64, P, I32, P, P]
    lib.bha_block_forward_commit.argtypes = [PD, P, P, P, PS, P, I64, P, P, I32, P, P, P, PS, P]
    lib.bha_block_forward_gqa.argtypes = [PD, I32, P, PS, P, P, PS, P, I64, P, P, I32, P, P, PS, P]
    lib.bha_block_forward_gqa.restype = ctypes.c_int
    lib.bha_block_forward_commit.restype = ctypes.c_int
    lib.bha_state_prefill.argtypes = [PD, P, P, PS, P, I64, P, I64, P, I32, P, P]
    lib.bha_state_prefill.restype = ctypes.c_int
    lib.bha_prefix_attention.argtypes = [PD, P, P, P, PS, P, P, PS, P, I64, P, I64, P, PS, P]
    lib.bha_prefix_attention.restype = ctypes.c_int
    lib.bha_prefix_attention_workspace.argtypes = [PD, I64]
    lib.bha_prefix_attention_workspace.restype = ctypes.c_int64
    lib.bha_prefix_attention_noalloc.argtypes = [PD, P, P, P, PS, P, P, PS, P, I64, P, PS, P]
    lib.bha_prefix_attention_noalloc.restype = ctypes.c_int
    lib.bha_prefix_attention_noalloc_scratch_bytes.argtypes = []
    lib.bha_prefix_attention_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.bha_state_record_floats.argtypes = [I32, I32]
    lib.bha_state_record_floats.restype = I64
    lib.bha_status_string.argtypes = [ctypes.c_int]
    lib.bha_status_string.restype = ctypes.c_char_p
    lib.bha_version.argtypes = []
    for f in (lib.bha_feature_map, lib.bha_block_forward, lib.bha_state_commit, lib.bha_version):
        f.restype = ctypes.c_int
    lib.bha_source_hash.argtypes = []
    lib.bha_source_hash.restype = ctypes.c_char_p
    if _LIB_PATH == _BUILT_LIB_PATH:
        # the in-tree library must have been built from the sources beside it
        from .build import source_hash
        built, here = lib.bha_source_hash().decode(), source_hash()
        if built != here:
            raise RuntimeError(
                f"{_LIB_PATH} was built from other sources (library {built}, sources on disk {here}): "
                "rebuild it with `python -m linear_attention_block_amd.build`")
    _lib = lib
    return lib


def version() -> int:
    return int(load_library().bha_version())


def source_hash() -> str:
    """The hash of the sources the loaded library was built from."""
    return load_library().bha_source_hash().decode()


def status_string(status: int) -> str:
    return load_library().bha_status_string(int(status)).decode()


def state_record_floats(head_dim: int, feat_half: int) -> int:
    return int(load_library().bha_state_record_floats(int(head_dim), int(feat_half)))


def new_state(num_slots: int, num_heads: int, head_dim: int, feat_half: int, device) -> torch.Tensor:
    """A zeroed state pool: [num_slots][H][(d + 1) * 2FW] float32 (nothing committed)."""
    rec = (head_dim + 1) * 2 * feat_half
    return torch.zeros((num_slots, num_heads, rec), dtype=torch.float32, device=device)


# ------------------------------------------------------------------ marshalling
def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BHA_BF16
    if t.dtype == torch.float32:
        return BHA_F32
    raise TypeError(f"token tensors must be bfloat16 or float32, got {t.dtype}")


def _tok_strides(t: torch.Tensor, name: str) -> bha_strides:
    if t.dim() != 4:
        raise ValueError(f"{name} must be [R][B][H][d], got shape {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return bha_strides(t.stride(0), t.stride(1), t.stride(2))


def _w_stride(w: torch.Tensor, H: int, d: int):
    if w.dim() == 2:
        fw, dd = w.shape
        if not w.is_contiguous() or dd != d:
            raise ValueError("w [FW][d] must be contiguous with d columns")
        return fw, 0
    if w.dim() == 3:
        hh, fw, dd = w.shape
        if hh != H or dd != d or w.stride(2) != 1 or w.stride(1) != d:
            raise ValueError("w must be [H][FW][d] with contiguous [FW][d] rows per head")
        return fw, w.stride(0)
    raise ValueError("w must be [H][FW][d] or [FW][d]")


def _stream(dev: torch.device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _check_device(dev, *ts):
    if dev.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    for t in ts:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")


def _feature_map_args(x, w, out, stream):
    xs = _tok_strides(x, "x")
    R, B, H, d = x.shape
    fw, wh = _w_stride(w, H, d)
    if w.dtype != x.dtype:
        raise TypeError("w must have the dtype of x")
    _check_device(x.device, w)
    if out is None:
        out = torch.empty((R, B, H, 2 * fw), dtype=torch.float32, device=x.device)
    elif out.shape != (R, B, H, 2 * fw) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [R][B][H][2FW] tensor")
    _check_device(x.device, out)
    dims = bha_dims(R, H, d, fw, B, _io_dtype(x), 0.0)
    args = (ctypes.byref(dims), _ptr(x), ctypes.byref(xs), _ptr(w), wh, _ptr(out), _stream(x.device, stream))
    return args, (dims, xs), out


def feature_map(x: torch.Tensor, w: torch.Tensor, *, out=None, stream=None) -> torch.Tensor:
    """phi(x) = [softmax(x W), softmax(-x W)] -> float32 [R][B][H][2FW]."""
    lib = load_library()
    args, _keep, out = _feature_map_args(x, w, out, stream)
    st = lib.bha_feature_map(*args)
    if st != 0:
        raise BhaError("bha_feature_map", st)
    return out


def _forward_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream):
    qs = _tok_strides(q, "q")
    R, B, H, d = q.shape
    for t, n in ((k, "k"), (v, "v")):
        if t.shape != q.shape:
            raise ValueError(f"{n} must match q in shape")
        if (t.stride(0), t.stride(1), t.stride(2)) != (qs.req, qs.tok, qs.head) or t.stride(3) != 1:
            raise ValueError(f"{n} must have the strides of q")
        if t.dtype != q.dtype:
            raise TypeError(f"{n} must have the dtype of q")
    fw, wh = _w_stride(w, H, d)
    if w.dtype != q.dtype:
        raise TypeError("w must have the dtype of q")
    if gamma.dtype != torch.float32 or gamma.numel() != H or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 [H] tensor")
    num_slots = _num_slots(state, H, d, fw)
    if slot_ids.dtype != torch.int32 or slot_ids.numel() != R or not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be a contiguous int32 [R] tensor")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    os_ = _tok_strides(out, "out")
    _check_device(q.device, k, v, w, gamma, state, slot_ids, out)
    dims = bha_dims(R, H, d, fw, B, _io_dtype(q), float(scale))
    return (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(qs), _ptr(w), wh,
            _ptr(gamma), _ptr(state), num_slots, _ptr(slot_ids), _ptr(out), ctypes.byref(os_),
            _stream(q.device, stream)), (dims, qs, os_)


def _forward_commit_args(q, k, v, w, gamma, state, slot_ids, commit_mask, out, scale, stream):
    args, keep = _forward_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream)
    if commit_mask is None:
        mask_ptr = ctypes.c_void_p(0)
    else:
        if commit_mask.dtype not in (torch.uint8, torch.bool) or commit_mask.numel() != q.shape[0] or \
                not commit_mask.is_contiguous():
            raise ValueError("commit_mask must be a contiguous uint8 (or bool) [R] tensor")
        _check_device(q.device, commit_mask)
        mask_ptr = _ptr(commit_mask)
    # forward arguments with the commit mask inserted after slot_ids
    return args[:11] + (mask_ptr,) + args[11:], keep


def _commit_args(k, v, w, state, slot_ids, stream):
    ks = _tok_strides(k, "k")
    R, B, H, d = k.shape
    if v.shape != k.shape or (v.stride(0), v.stride(1), v.stride(2)) != (ks.req, ks.tok, ks.head):
        raise ValueError("v must match k in shape and strides")
    if v.dtype != k.dtype or w.dtype != k.dtype:
        raise TypeError("k, v and w must share one dtype")
    fw, wh = _w_stride(w, H, d)
    num_slots = _num_slots(state, H, d, fw)
    if slot_ids.dtype != torch.int32 or slot_ids.numel() != R or not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be a contiguous int32 [R] tensor")
    _check_device(k.device, v, w, state, slot_ids)
    dims = bha_dims(R, H, d, fw, B, _io_dtype(k), 0.0)
    return (ctypes.byref(dims), _ptr(k), _ptr(v), ctypes.byref(ks), _ptr(w), wh, _ptr(state),
            num_slots, _ptr(slot_ids), _stream(k.device, stream)), (dims, ks)


def _num_slots(state, H, d, fw):
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous float32 tensor")
    rec = (d + 1) * 2 * fw
    if state.numel() % (H * rec) != 0 or state.numel() == 0:
        raise ValueError("state size is not a whole number of [H][record] slots")
    return state.numel() // (H * rec)


def block_forward(q, k, v, w, gamma, state, slot_ids, *, out=None, scale: float = 0.0,
                  stream=None) -> torch.Tensor:
    """One block-hybrid attention step for every (request, head); returns ``out``."""
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, _keep = _forward_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream)
    st = lib.bha_block_forward(*args)
    if st != 0:
        raise BhaError("bha_block_forward", st)
    return out


def _forward_gqa_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream):
    qs = _tok_strides(q, "q")
    R, B, H, d = q.shape
    ks = _tok_strides(k, "k")
    Rk, Bk, HK, dk = k.shape
    if (Rk, Bk, dk) != (R, B, d) or HK < 1 or H % HK != 0:
        raise ValueError("k must be [R][B][Hkv][d] with Hkv dividing the query heads of q")
    if v.shape != k.shape or (v.stride(0), v.stride(1), v.stride(2)) != (ks.req, ks.tok, ks.head) or \
            v.stride(3) != 1:
        raise ValueError("v must match k in shape and strides")
    if k.dtype != q.dtype or v.dtype != q.dtype or w.dtype != q.dtype:
        raise TypeError("q, k, v and w must share one dtype")
    fw, wh = _w_stride(w, HK, d)
    if gamma.dtype != torch.float32 or gamma.numel() != H or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 [H] tensor (one gate per query head)")
    num_slots = _num_slots(state, HK, d, fw)
    if slot_ids.dtype != torch.int32 or slot_ids.numel() != R or not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be a contiguous int32 [R] tensor")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    os_ = _tok_strides(out, "out")
    _check_device(q.device, k, v, w, gamma, state, slot_ids, out)
    dims = bha_dims(R, H, d, fw, B, _io_dtype(q), float(scale))
    return (ctypes.byref(dims), HK, _ptr(q), ctypes.byref(qs), _ptr(k), _ptr(v), ctypes.byref(ks), _ptr(w), wh,
            _ptr(gamma), _ptr(state), num_slots, _ptr(slot_ids), _ptr(out), ctypes.byref(os_),
            _stream(q.device, stream)), (dims, qs, ks, os_)


def block_forward_gqa(q, k, v, w, gamma, state, slot_ids, *, out=None, scale: float = 0.0,
                      stream=None) -> torch.Tensor:
    """block_forward with grouped K/V heads: q [R][B][H][d], k, v
    [R][B][Hkv][d] (Hkv dividing H), w and the state per K/V head, gamma per
    query head; query head h uses K/V head h // (H // Hkv). Returns ``out``."""
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, _keep = _forward_gqa_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream)
    st = lib.bha_block_forward_gqa(*args)
    if st != 0:
        raise BhaError("bha_block_forward_gqa", st)
    return out


def block_forward_commit(q, k, v, w, gamma, state, slot_ids, *, commit_mask=None, out=None,
                         scale: float = 0.0, stream=None) -> torch.Tensor:
    """The last denoising step of a block: the forward from the state as it
    stands, then the commit of (k, v) for the requests whose ``commit_mask``
    entry is non-zero (every request when it is None); returns ``out``."""
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, _keep = _forward_commit_args(q, k, v, w, gamma, state, slot_ids, commit_mask, out, scale, stream)
    st = lib.bha_block_forward_commit(*args)
    if st != 0:
        raise BhaError("bha_block_forward_commit", st)
    return out


def state_commit(k, v, w, state, slot_ids, *, stream=None) -> None:
    """Fold the block (k, v) into the state records of ``slot_ids`` (in place)."""
    lib = load_library()
    args, _keep = _commit_args(k, v, w, state, slot_ids, stream)
    st = lib.bha_state_commit(*args)
    if st != 0:
        raise BhaError("bha_state_commit", st)


def state_prefill(k, v, seq_offsets, w, state, slot_ids, *, stream=None) -> None:
    """Fold each request's packed token range into its state records (in place).

    k, v: [T][H][d] packed tokens (last dimension contiguous); seq_offsets:
    int32 [R + 1] on the device, request r owning rows seq_offsets[r] ..
    seq_offsets[r+1]-1; slot_ids: int32 [R], distinct."""
    lib = load_library()
    if k.dim() != 3 or v.shape != k.shape or k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("k and v must be [T][H][d] with a contiguous last dimension")
    if (v.stride(0), v.stride(1)) != (k.stride(0), k.stride(1)):
        raise ValueError("v must have the strides of k")
    if v.dtype != k.dtype or w.dtype != k.dtype:
        raise TypeError("k, v and w must share one dtype")
    T, H, d = k.shape
    fw, wh = _w_stride(w, H, d)
    num_slots = _num_slots(state, H, d, fw)
    R = slot_ids.numel()
    if slot_ids.dtype != torch.int32 or not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be a contiguous int32 tensor")
    if seq_offsets.dtype != torch.int32 or seq_offsets.numel() != R + 1 or not seq_offsets.is_contiguous():
        raise ValueError("seq_offsets must be a contiguous int32 [R + 1] tensor")
    _check_device(k.device, v, w, state, slot_ids, seq_offsets)
    dims = bha_dims(R, H, d, fw, 1, _io_dtype(k), 0.0)
    ks = bha_strides(0, k.stride(0), k.stride(1))
    st = lib.bha_state_prefill(ctypes.byref(dims), _ptr(k), _ptr(v), ctypes.byref(ks), _ptr(seq_offsets), T,
                               _ptr(w), wh, _ptr(state), num_slots, _ptr(slot_ids), _stream(k.device, stream))
    if st != 0:
        raise BhaError("bha_state_prefill", st)


_NO_WORKSPACE = object()  # marshal a prefix-attention call without a workspace argument


def _prefix_args(q, k, v, kp, vp, seq_offsets, out, scale, stream, workspace):
    qs = _tok_strides(q, "q")
    R, B, H, d = q.shape
    for t, n in ((k, "k"), (v, "v")):
        if t.shape != q.shape or (t.stride(0), t.stride(1), t.stride(2)) != (qs.req, qs.tok, qs.head) or \
                t.stride(3) != 1:
            raise ValueError(f"{n} must match q in shape and strides")
        if t.dtype != q.dtype:
            raise TypeError(f"{n} must have the dtype of q")
    if kp.dim() != 3 or vp.shape != kp.shape or kp.shape[1:] != (H, d) or kp.stride(2) != 1 or vp.stride(2) != 1:
        raise ValueError("kp and vp must be [T][H][d] with a contiguous last dimension")
    if (vp.stride(0), vp.stride(1)) != (kp.stride(0), kp.stride(1)):
        raise ValueError("vp must have the strides of kp")
    if kp.dtype != q.dtype or vp.dtype != q.dtype:
        raise TypeError("kp and vp must have the dtype of q")
    if seq_offsets.dtype != torch.int32 or seq_offsets.numel() != R + 1 or not seq_offsets.is_contiguous():
        raise ValueError("seq_offsets must be a contiguous int32 [R + 1] tensor")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    os_ = _tok_strides(out, "out")
    _check_device(q.device, k, v, kp, vp, seq_offsets, out)
    # feat_half is not used by this call; any supported value passes
    dims = bha_dims(R, H, d, 64, B, _io_dtype(q), float(scale))
    ps = bha_strides(0, kp.stride(0), kp.stride(1))
    T = kp.shape[0]
    if workspace is _NO_WORKSPACE:
        workspace = None
        wptr, wbytes = None, 0
    elif workspace is None:
        need = load_library().bha_prefix_attention_workspace(ctypes.byref(dims), T)
        if need < 0:
            raise BhaError("bha_prefix_attention_workspace", int(need))
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if workspace is not None:
        _check_device(q.device, workspace)
        wptr, wbytes = _ptr(workspace), workspace.numel()
    return (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(qs), _ptr(kp), _ptr(vp), ctypes.byref(ps),
            _ptr(seq_offsets), T, wptr, wbytes, _ptr(out), ctypes.byref(os_),
            _stream(q.device, stream)), (dims, qs, ps, os_, workspace)


def prefix_attention_workspace(R, H, d, B, total_tokens, dtype=torch.bfloat16) -> int:
    """Workspace bytes prefix_attention uses for these sizes (0: none)."""
    dims = bha_dims(R, H, d, 64, B, BHA_BF16 if dtype == torch.bfloat16 else BHA_F32, 0.0)
    n = load_library().bha_prefix_attention_workspace(ctypes.byref(dims), int(total_tokens))
    if n < 0:
        raise BhaError("bha_prefix_attention_workspace", int(n))
    return int(n)


def prefix_attention(q, k, v, kp, vp, seq_offsets, *, out=None, scale: float = 0.0, workspace=None,
                     stream=None) -> torch.Tensor:
    """Exact softmax attention of each block's queries over its request's
    packed prefix (rows seq_offsets[r] .. seq_offsets[r+1]-1 of kp, vp,
    [T][H][d]) and the block's own keys; returns ``out`` [R][B][H][d].
    ``workspace`` (uint8 device tensor) holds split partial results; when None
    one of the size bha_prefix_attention_workspace gives is allocated."""
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, _keep = _prefix_args(q, k, v, kp, vp, seq_offsets, out, scale, stream, workspace)
    st = lib.bha_prefix_attention(*args)
    if st != 0:
        raise BhaError("bha_prefix_attention", st)
    return out


def prefix_attention_noalloc(q, k, v, kp, vp, seq_offsets, *, out, scale: float = 0.0,
                             stream=None) -> torch.Tensor:
    """bha_prefix_attention_noalloc: the same attention as ``prefix_attention``
    with a full workspace, its split partials kept in the library's static
    device buffer; ``out`` must be given (nothing is allocated)."""
    lib = load_library()
    args, _keep = _prefix_args(q, k, v, kp, vp, seq_offsets, out, scale, stream, _NO_WORKSPACE)
    # the same arguments without the workspace pointer and size
    st = lib.bha_prefix_attention_noalloc(*args[:10], *args[12:])
    if st != 0:
        raise BhaError("bha_prefix_attention_noalloc", st)
    return out


def prefix_attention_noalloc_scratch_bytes() -> int:
    return int(load_library().bha_prefix_attention_noalloc_scratch_bytes())


class _Prepared:
    """A C-ABI call whose arguments were checked and marshalled once; calling it
    enqueues the same call again (on the stream captured at preparation). The
    tensors must stay alive and keep their storage while it is used."""

    def __init__(self, fn, name, args, keep):
        self._fn, self._name, self._args, self._keep = fn, name, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            raise BhaError(self._name, st)


def prepare_forward(q, k, v, w, gamma, state, slot_ids, out, *, scale: float = 0.0, stream=None):
    """Marshal a bha_block_forward call once, for launch-rate-bound loops."""
    args, keep = _forward_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream)
    keep = keep + (q, k, v, w, gamma, state, slot_ids, out)
    return _Prepared(load_library().bha_block_forward, "bha_block_forward", args, keep)


def prepare_forward_gqa(q, k, v, w, gamma, state, slot_ids, out, *, scale: float = 0.0, stream=None):
    """Marshal a bha_block_forward_gqa call once, for launch-rate-bound loops."""
    args, keep = _forward_gqa_args(q, k, v, w, gamma, state, slot_ids, out, scale, stream)
    keep = keep + (q, k, v, w, gamma, state, slot_ids, out)
    return _Prepared(load_library().bha_block_forward_gqa, "bha_block_forward_gqa", args, keep)


def prepare_forward_commit(q, k, v, w, gamma, state, slot_ids, out, *, commit_mask=None, scale: float = 0.0,
                           stream=None):
    """Marshal a bha_block_forward_commit call once, for launch-rate-bound loops."""
    args, keep = _forward_commit_args(q, k, v, w, gamma, state, slot_ids, commit_mask, out, scale, stream)
    keep = keep + (q, k, v, w, gamma, state, slot_ids, out, commit_mask)
    return _Prepared(load_library().bha_block_forward_commit, "bha_block_forward_commit", args, keep)


def prepare_prefix_attention(q, k, v, kp, vp, seq_offsets, out, *, scale: float = 0.0, workspace=None,
                             stream=None):
    """Marshal a bha_prefix_attention call once (its workspace included), for
    launch-rate-bound loops."""
    args, keep = _prefix_args(q, k, v, kp, vp, seq_offsets, out, scale, stream, workspace)
    keep = keep + (q, k, v, kp, vp, seq_offsets, out)
    return _Prepared(load_library().bha_prefix_attention, "bha_prefix_attention", args, keep)


def prepare_feature_map(x, w, out, *, stream=None):
    """Marshal a bha_feature_map call once, for launch-rate-bound loops."""
    args, keep, out = _feature_map_args(x, w, out, stream)
    return _Prepared(load_library().bha_feature_map, "bha_feature_map", args, keep + (x, w, out))


def prepare_commit(k, v, w, state, slot_ids, *, stream=None):
    """Marshal a bha_state_commit call once, for launch-rate-bound loops."""
    args, keep = _commit_args(k, v, w, state, slot_ids, stream)
    keep = keep + (k, v, w, state, slot_ids)
    return _Prepared(load_library().bha_state_commit, "bha_state_commit", args, keep)
