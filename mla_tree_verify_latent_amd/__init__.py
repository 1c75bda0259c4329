"""Python binding of the MI355X MLA tree-verify attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libverify_attn.so`` (built from ``csrc/verify_attn.hip`` by
``build.py``). PyTorch provides device memory and the current stream. There is
no fallback: if the library is missing or the device is not gfx950 the calls
raise.

Entry points mirror the C ABI declared in ``include/verify_attn.h``:
``verify_attn``, ``verify_attn_noalloc``, ``verify_attn_partial``, ``verify_attn_combine``,
``verify_attn_append_kv``, ``verify_attn_compact_kv``, ``verify_attn_f32``,
``verify_attn_f32_workspace_size``, ``verify_attn_debug_validate``, ``verify_attn_workspace_size``, ``verify_attn_plan``,
``verify_attn_plan_for``, ``verify_attn_strerror``, ``verify_attn_version``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libverify_attn.so")

KV_DIM = 576
V_DIM = 512
MAX_TREE = 64

EXPORTS = (
    "verify_attn", "verify_attn_noalloc", "verify_attn_partial", "verify_attn_combine", "verify_attn_append_kv",
    "verify_attn_compact_kv", "verify_attn_f32", "verify_attn_f32_workspace_size",
    "verify_attn_debug_validate",
    "verify_attn_workspace_size",
    "verify_attn_plan", "verify_attn_plan_for", "verify_attn_strerror", "verify_attn_version",
)


class Params(ctypes.Structure):
    """Mirror of ``verify_attn_params``."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("tree_size", ctypes.c_int32), ("kv_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("nsplit", ctypes.c_int32), ("total_kv", ctypes.c_int64), ("pool_slots", ctypes.c_int64),
        ("sm_scale", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``verify_attn_plan_info``."""
    _fields_ = [
        ("rows_per_tile", ctypes.c_int32), ("row_tiles", ctypes.c_int32),
        ("keys_per_split", ctypes.c_int32), ("max_splits", ctypes.c_int32),
        ("partial_blocks", ctypes.c_int32), ("combine_blocks", ctypes.c_int32),
        ("threads_per_block", ctypes.c_int32), ("keys_per_tile", ctypes.c_int32),
    ]


class VerifyAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"verify_attn status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of libverify_attn.so."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m mla_tree_verify_latent_amd.build` (hipcc, gfx950)")
    # torch first: its bundled HIP runtime has the system runtime's soname, so the
    # library then binds to the runtime that owns torch's tensors and streams (loaded
    # the other way round, torch would bring a second runtime into the process).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, vp, i32p = ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p
    lib.verify_attn_workspace_size.argtypes = [P]
    lib.verify_attn_workspace_size.restype = ctypes.c_size_t
    lib.verify_attn.argtypes = [P, vp, vp, i32p, i32p, i32p, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn.restype = ctypes.c_int
    lib.verify_attn_noalloc.argtypes = [P, vp, vp, i32p, i32p, i32p, vp, vp]
    lib.verify_attn_noalloc.restype = ctypes.c_int
    lib.verify_attn_f32.argtypes = [P, vp, vp, i32p, i32p, i32p, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_f32.restype = ctypes.c_int
    lib.verify_attn_debug_validate.argtypes = [P, i32p, i32p, i32p, vp, vp]
    lib.verify_attn_debug_validate.restype = ctypes.c_int
    lib.verify_attn_f32_workspace_size.argtypes = [P]
    lib.verify_attn_f32_workspace_size.restype = ctypes.c_size_t
    lib.verify_attn_partial.argtypes = [P, vp, vp, i32p, i32p, i32p, vp, ctypes.c_size_t, vp]
    lib.verify_attn_partial.restype = ctypes.c_int
    lib.verify_attn_combine.argtypes = [P, i32p, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_combine.restype = ctypes.c_int
    lib.verify_attn_append_kv.argtypes = [P, vp, i32p, i32p, vp, vp]
    lib.verify_attn_append_kv.restype = ctypes.c_int
    lib.verify_attn_compact_kv.argtypes = [P, vp, i32p, vp, vp]
    lib.verify_attn_compact_kv.restype = ctypes.c_int
    lib.verify_attn_plan.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.verify_attn_plan.restype = ctypes.c_int
    lib.verify_attn_plan_for.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(PlanInfo)]
    lib.verify_attn_plan_for.restype = ctypes.c_int
    lib.verify_attn_strerror.argtypes = [ctypes.c_int]
    lib.verify_attn_strerror.restype = ctypes.c_char_p
    lib.verify_attn_version.argtypes = []
    lib.verify_attn_version.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def make_params(*, num_seqs: int, num_heads: int, tree_size: int, max_seq_len: int,
                total_kv: int, pool_slots: int, sm_scale: float, nsplit: int = 0,
                page_size: int = 1, kv_dim: int = KV_DIM, v_dim: int = V_DIM) -> Params:
    return Params(num_seqs, num_heads, tree_size, kv_dim, v_dim, page_size, max_seq_len, nsplit,
                  total_kv, pool_slots, sm_scale, 0)


def verify_attn_strerror(status: int) -> str:
    return load_library().verify_attn_strerror(int(status)).decode()


def verify_attn_version() -> int:
    return int(load_library().verify_attn_version())


def verify_attn_workspace_size(params: Params) -> int:
    return int(load_library().verify_attn_workspace_size(ctypes.byref(params)))


def verify_attn_plan(params: Params) -> dict:
    """The launch decomposition for the current device (see verify_attn_plan_info)."""
    info = PlanInfo()
    _check(load_library().verify_attn_plan(ctypes.byref(params), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def verify_attn_plan_for(params: Params, fp32_inputs: bool = False, num_cus: int = 0,
                         num_xcds: int = 0) -> dict:
    """The decomposition for either input type and an explicit device shape
    (num_cus compute units in num_xcds XCDs; both 0 = the current device)."""
    info = PlanInfo()
    _check(load_library().verify_attn_plan_for(ctypes.byref(params), int(bool(fp32_inputs)), int(num_cus),
                                               int(num_xcds), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def _check(status: int):
    if status != 0:
        raise VerifyAttnError(status, verify_attn_strerror(status))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_tensors(q, kv_pool, slot_idx, seq_lens, tree_parent, out=None, dtype=None):
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    named = dict(q=q, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens,
                 tree_parent=tree_parent)
    if out is not None:
        named["out"] = out
    for name, t in named.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name in ("q", "kv_pool") + (("out",) if out is not None else ()):
        if named[name].dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
    for name in ("slot_idx", "seq_lens", "tree_parent"):
        if named[name].dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if q.dim() != 4 or q.shape[-1] != KV_DIM:
        raise ValueError("q must be [B, T, H, 576]")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != KV_DIM:
        raise ValueError("kv_pool must be [slots, 576]")
    B, T, H, _ = q.shape
    if tuple(seq_lens.shape) != (B,) or tuple(tree_parent.shape) != (B, T):
        raise ValueError("seq_lens must be [B] and tree_parent [B, T]")
    if out is not None and tuple(out.shape) != (B, T, H, V_DIM):
        raise ValueError("out must be [B, T, H, 512]")


def _check_sizes(params: Params, *, q=None, kv_pool=None, slot_idx=None, seq_lens=None,
                 tree_parent=None, out=None):
    """The tensors must hold what `params` says they hold: the kernels index them by
    these sizes, so a tensor smaller than its params would be read or written past
    its end."""
    B, T, H = int(params.num_seqs), int(params.tree_size), int(params.num_heads)
    if q is not None and tuple(q.shape) != (B, T, H, KV_DIM):
        raise ValueError(f"q is {tuple(q.shape)}, params say [{B}, {T}, {H}, {KV_DIM}]")
    if out is not None and tuple(out.shape) != (B, T, H, V_DIM):
        raise ValueError(f"out is {tuple(out.shape)}, params say [{B}, {T}, {H}, {V_DIM}]")
    if kv_pool is not None and int(kv_pool.shape[0]) < int(params.pool_slots):
        raise ValueError(f"kv_pool has {kv_pool.shape[0]} rows, params say pool_slots={params.pool_slots}")
    if slot_idx is not None and slot_idx.numel() != int(params.total_kv):
        raise ValueError(f"slot_idx has {slot_idx.numel()} entries, params say total_kv={params.total_kv}")
    if seq_lens is not None and tuple(seq_lens.shape) != (B,):
        raise ValueError(f"seq_lens is {tuple(seq_lens.shape)}, params say [{B}]")
    if tree_parent is not None and tuple(tree_parent.shape) != (B, T):
        raise ValueError(f"tree_parent is {tuple(tree_parent.shape)}, params say [{B}, {T}]")


def _check_workspace(workspace):
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")


def _check_device(stream, *tensors):
    """All tensors on one device, the one the kernels are launched on (that of
    `stream`, else the current device): a pointer into another GPU's memory would
    be dereferenced as if it were local."""
    import torch
    devs = {t.device for t in tensors}
    if len(devs) != 1:
        raise ValueError(f"the tensors are on {sorted(str(d) for d in devs)}: they must share one device")
    dev = devs.pop()
    run = stream.device if stream is not None else torch.device("cuda", torch.cuda.current_device())
    if dev != run:
        raise ValueError(f"the tensors are on {dev} but the kernels would run on {run}")


def params_for(q, kv_pool, slot_idx, *, max_seq_len: int, sm_scale: float, nsplit: int = 0,
               page_size: int = 1) -> Params:
    """Params of a call on these tensors. max_seq_len is host-known by the caller."""
    B, T, H, _ = q.shape
    return make_params(num_seqs=B, num_heads=H, tree_size=T, max_seq_len=int(max_seq_len),
                       total_kv=int(slot_idx.numel()), pool_slots=int(kv_pool.shape[0]),
                       sm_scale=float(sm_scale), nsplit=int(nsplit), page_size=int(page_size))


def verify_attn(q, kv_pool, slot_idx, seq_lens, tree_parent, out, workspace, params: Params,
                stream=None) -> None:
    """Enqueue the verify attention on `stream` (default: torch's current stream)."""
    _check_tensors(q, kv_pool, slot_idx, seq_lens, tree_parent, out)
    _check_sizes(params, q=q, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens,
                 tree_parent=tree_parent, out=out)
    _check_workspace(workspace)
    _check_device(stream, q, kv_pool, slot_idx, seq_lens, tree_parent, out, workspace)
    _check(load_library().verify_attn(
        ctypes.byref(params), _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens),
        _ptr(tree_parent), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


NOALLOC_SCRATCH_BYTES = 80 << 20  # VERIFY_ATTN_NOALLOC_SCRATCH_BYTES


def verify_attn_noalloc(q, kv_pool, slot_idx, seq_lens, tree_parent, out, params: Params,
                        stream=None) -> None:
    """verify_attn without a workspace: the split-K partials go to the library's
    per-GPU scratch array (NOALLOC_SCRATCH_BYTES; calls needing more raise with
    VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL). Calls that overlap on one GPU race on it."""
    _check_tensors(q, kv_pool, slot_idx, seq_lens, tree_parent, out)
    _check_sizes(params, q=q, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens,
                 tree_parent=tree_parent, out=out)
    _check_device(stream, q, kv_pool, slot_idx, seq_lens, tree_parent, out)
    _check(load_library().verify_attn_noalloc(
        ctypes.byref(params), _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens),
        _ptr(tree_parent), _ptr(out), _stream(stream)))


def verify_attn_f32_workspace_size(params: Params) -> int:
    return int(load_library().verify_attn_f32_workspace_size(ctypes.byref(params)))


def verify_attn_f32(q, kv_pool, slot_idx, seq_lens, tree_parent, out, workspace, params: Params,
                    stream=None) -> None:
    """Enqueue the fp32-input verify attention (float32 q, kv_pool and out)."""
    import torch
    _check_tensors(q, kv_pool, slot_idx, seq_lens, tree_parent, out, dtype=torch.float32)
    _check_sizes(params, q=q, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens,
                 tree_parent=tree_parent, out=out)
    _check_workspace(workspace)
    _check_device(stream, q, kv_pool, slot_idx, seq_lens, tree_parent, out, workspace)
    _check(load_library().verify_attn_f32(
        ctypes.byref(params), _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens),
        _ptr(tree_parent), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


# Bits of verify_attn_debug_validate's result
BAD_LENGTH, BAD_TOTAL, BAD_PARENT, BAD_SLOT = 1, 2, 4, 8


def verify_attn_debug_validate(slot_idx, seq_lens, tree_parent, params: Params, flags=None,
                               stream=None) -> int:
    """Check the device-resident inputs; returns the BAD_* bits (0 = valid).
    Debug only: reads the result back (synchronises the stream)."""
    import torch
    for name, t in dict(slot_idx=slot_idx, seq_lens=seq_lens, tree_parent=tree_parent).items():
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    _check_sizes(params, slot_idx=slot_idx, seq_lens=seq_lens, tree_parent=tree_parent)
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=slot_idx.device)
    elif not flags.is_cuda or flags.dtype != torch.int32 or flags.numel() < 1:
        raise ValueError("flags must be an int32 device tensor of at least one element")
    _check_device(stream, slot_idx, seq_lens, tree_parent, flags)
    _check(load_library().verify_attn_debug_validate(
        ctypes.byref(params), _ptr(slot_idx), _ptr(seq_lens), _ptr(tree_parent), _ptr(flags),
        _stream(stream)))
    return int(flags.item())


def verify_attn_partial(q, kv_pool, slot_idx, seq_lens, tree_parent, workspace, params: Params,
                        stream=None) -> None:
    _check_tensors(q, kv_pool, slot_idx, seq_lens, tree_parent)
    _check_sizes(params, q=q, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens,
                 tree_parent=tree_parent)
    _check_workspace(workspace)
    _check_device(stream, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace)
    _check(load_library().verify_attn_partial(
        ctypes.byref(params), _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens),
        _ptr(tree_parent), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def verify_attn_combine(seq_lens, out, workspace, params: Params, stream=None) -> None:
    import torch
    for name, t in dict(seq_lens=seq_lens, out=out).items():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if seq_lens.dtype != torch.int32 or out.dtype != torch.bfloat16:
        raise ValueError("seq_lens must be int32 and out bfloat16")
    _check_sizes(params, seq_lens=seq_lens, out=out)
    _check_workspace(workspace)
    _check_device(stream, seq_lens, out, workspace)
    _check(load_library().verify_attn_combine(
        ctypes.byref(params), _ptr(seq_lens), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def verify_attn_append_kv(kv_new, slot_idx, seq_lens, kv_pool, params: Params, stream=None) -> None:
    """Enqueue the draft-row KV append: kv_new [B, T, 576] -> kv_pool at the
    tree nodes' slots (the last T entries of each sequence's slot_idx segment)."""
    import torch
    for name, t in dict(kv_new=kv_new, slot_idx=slot_idx, seq_lens=seq_lens, kv_pool=kv_pool).items():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if kv_new.dtype != torch.bfloat16 or kv_pool.dtype != torch.bfloat16:
        raise ValueError("kv_new and kv_pool must be bfloat16")
    if slot_idx.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("slot_idx and seq_lens must be int32")
    if tuple(kv_new.shape) != (params.num_seqs, params.tree_size, KV_DIM):
        raise ValueError("kv_new must be [B, T, 576]")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != KV_DIM:
        raise ValueError("kv_pool must be [slots, 576]")
    _check_sizes(params, kv_pool=kv_pool, slot_idx=slot_idx, seq_lens=seq_lens)
    _check_device(stream, kv_new, slot_idx, seq_lens, kv_pool)
    _check(load_library().verify_attn_append_kv(
        ctypes.byref(params), _ptr(kv_new), _ptr(slot_idx), _ptr(seq_lens), _ptr(kv_pool),
        _stream(stream)))


def verify_attn_compact_kv(kv_pool, slot_idx, kv_dst, params: Params, stream=None) -> None:
    """Enqueue the KV defragmentation: kv_dst[i] = kv_pool[slot_idx[i]]."""
    import torch
    for name, t in dict(kv_pool=kv_pool, slot_idx=slot_idx, kv_dst=kv_dst).items():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if kv_pool.dtype != torch.bfloat16 or kv_dst.dtype != torch.bfloat16 or slot_idx.dtype != torch.int32:
        raise ValueError("kv_pool / kv_dst must be bfloat16, slot_idx int32")
    if tuple(kv_dst.shape) != (int(params.total_kv), KV_DIM) or kv_pool.dim() != 2 or kv_pool.shape[1] != KV_DIM:
        raise ValueError("kv_dst must be [total_kv, 576] and kv_pool [slots, 576]")
    _check_sizes(params, kv_pool=kv_pool, slot_idx=slot_idx)
    _check_device(stream, kv_pool, slot_idx, kv_dst)
    _check(load_library().verify_attn_compact_kv(
        ctypes.byref(params), _ptr(kv_pool), _ptr(slot_idx), _ptr(kv_dst), _stream(stream)))


class VerifyAttention:
    """A call shape with its workspace allocated once (torch, on the device).

    ``__call__`` makes no allocation other than ``out`` when it is not given,
    so with ``out`` passed in it can be captured in a HIP graph.
    """

    def __init__(self, params: Params, device="cuda"):
        import torch
        self.params = params
        nbytes = verify_attn_workspace_size(params)
        if nbytes == 0:
            raise ValueError("invalid verify_attn params")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def __call__(self, q, kv_pool, slot_idx, seq_lens, tree_parent, out=None, stream=None):
        import torch
        if out is None:
            B, T, H, _ = q.shape
            out = torch.empty((B, T, H, V_DIM), dtype=torch.bfloat16, device=q.device)
        verify_attn(q, kv_pool, slot_idx, seq_lens, tree_parent, out, self.workspace, self.params,
                    stream)
        return out
