"""ctypes binding of libpsa.so (shared-prefix block-sparse attention, gfx950).

Argument marshalling only: tensors are passed as device pointers plus the current
HIP stream, and every step of the computation runs in the library's HIP kernels.
If libpsa.so is missing the first call raises; there is no fallback path.

    m = psa.build_tile_map_tokens(group, suffix, is_prefix)          # device int32/uint8
    o, lse = psa.fwd(m, q, k, v)                                      # [T,hq,d], [hq,T]
    dq, dk, dv = psa.bwd(m, q, k, v, o, lse, do)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import numpy as np
import torch  # loaded first so that its HIP runtime is the one libpsa.so binds to

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpsa.so")
_lib = None
_lock = threading.Lock()

PSA_FP32, PSA_BF16, PSA_FP8_E4M3 = 0, 1, 2
PASS_FWD, PASS_BWD = 0, 1
STATUS = {0: "PSA_OK", 1: "PSA_ERR_NULL", 2: "PSA_ERR_SHAPE", 3: "PSA_ERR_LAYOUT",
          4: "PSA_ERR_DTYPE", 5: "PSA_ERR_UNSUPPORTED", 6: "PSA_ERR_MAP_MISMATCH",
          7: "PSA_ERR_WORKSPACE", 8: "PSA_ERR_HIP", 9: "PSA_ERR_ALLOC", 10: "PSA_ERR_VALUE"}

EXPORTS = ["psa_abi_version", "psa_status_string", "psa_last_error", "psa_tile_shape",
           "psa_build_tile_map_tokens", "psa_build_tile_map_tree", "psa_tile_map_info_get",
           "psa_tile_map_export", "psa_tile_map_destroy", "psa_fwd", "psa_bwd_workspace_size",
           "psa_bwd", "psa_bwd_stages", "psa_fold_workspace_size", "psa_fold_rollouts",
           "psa_unfold_rows", "psa_build_tile_map_tokens_ex", "psa_build_tile_map_tree_ex",
           "psa_tile_map_export_nodes", "psa_build_tile_map_draft", "psa_bwd_noalloc"]
FORM_INTERVAL, FORM_NODES = 0, 1  # mask encodings of a map (info["form"])
MAP_NODE_FORM = 1  # build flag: the node form even where the interval form exists
DRAFT_CAUSAL = 1  # flag of psa_build_tile_map_draft: causal attention inside a block
STAGE_PREPARE, STAGE_DKDV, STAGE_DQ, STAGE_ALL = 1, 2, 4, 7
BWD_SPLIT_PDS = 16  # option bit of psa_bwd_stages: P and dS as hi + lo bf16 pairs


class PsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class TileMapInfo(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("n_qtiles", ctypes.c_int64), ("n_ktiles", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("n_full", ctypes.c_int64),
                ("n_partial", ctypes.c_int64), ("form", ctypes.c_int32),
                ("causal", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Open libpsa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python -m shared_prefix_block_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t)
        PP = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "psa_abi_version": (I32, []),
            "psa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "psa_last_error": (ctypes.c_char_p, []),
            "psa_tile_shape": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, I32,
                                              ctypes.POINTER(I32), ctypes.POINTER(I32)]),
            "psa_build_tile_map_tokens": (ctypes.c_int, [I64, P, P, P, I32, I32, P, PP]),
            "psa_build_tile_map_tree": (ctypes.c_int, [I64, P, I64, P, P, I64, I32, I32, P, PP]),
            "psa_build_tile_map_tokens_ex": (ctypes.c_int, [I64, P, P, P, I32, I32, I32, P, PP]),
            "psa_build_tile_map_tree_ex": (ctypes.c_int, [I64, P, I64, P, P, I64, I32, I32, I32,
                                                          P, PP]),
            "psa_tile_map_export_nodes": (ctypes.c_int, [P, P, P, P]),
            "psa_build_tile_map_draft": (ctypes.c_int, [I64, I32, I64, P, P, P, P, I32, I64, I32,
                                                        I32, P, PP]),
            "psa_tile_map_info_get": (ctypes.c_int, [P, ctypes.POINTER(TileMapInfo)]),
            "psa_tile_map_export": (ctypes.c_int, [P, P, P, P, P, P, P, P, P]),
            "psa_tile_map_destroy": (None, [P]),
            "psa_fwd": (ctypes.c_int, [P, ctypes.c_int, I64, I32, I32, I32, F, P, P, P, P, P, P]),
            "psa_bwd_workspace_size": (ctypes.c_int, [P, ctypes.c_int, I64, I32, I32, I32,
                                                      ctypes.POINTER(SZ)]),
            "psa_bwd": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, I64, I32, I32, I32, F, P, P,
                                       P, P, P, P, P, P, P, P, SZ, P]),
            "psa_bwd_stages": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, I64, I32, I32, I32, F,
                                              P, P, P, P, P, P, P, P, P, P, SZ, I32, P]),
            "psa_bwd_noalloc": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, I64, I32, I32, I32,
                                               F, P, P, P, P, P, P, P, P, P, P]),
            "psa_fold_workspace_size": (ctypes.c_int, [I64, I64, ctypes.POINTER(SZ)]),
            "psa_fold_rollouts": (ctypes.c_int, [I64, P, P, P, P, P, I64, I32, I32, P, P, P, P,
                                                 P, P, P, SZ, P]),
            "psa_unfold_rows": (ctypes.c_int, [I64, P, P, P, I64, I64, P, P, SZ, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != 0:
        detail = _lib.psa_last_error().decode(errors="replace")
        raise PsaError(status, detail)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return PSA_FP32
    if dt == torch.bfloat16:
        return PSA_BF16
    if dt == torch.float8_e4m3fn:
        return PSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {dt} (float32, bfloat16 or float8_e4m3fn)")


def tile_shape(pass_: int, dtype: torch.dtype, d: int):
    lib = load()
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.psa_tile_shape(pass_, _dtype_code(dtype), d, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


class TileMap:
    """Owning handle of a psa_tile_map (destroyed when collected or on close())."""

    def __init__(self, handle: int, device: torch.device, keepalive=None):
        self._h = ctypes.c_void_p(handle)
        self.device = device
        self._keep = keepalive
        info = TileMapInfo()
        _check(load().psa_tile_map_info_get(self._h, ctypes.byref(info)))
        self.info = {f: getattr(info, f) for f, _ in TileMapInfo._fields_}
        self.T = info.T

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise RuntimeError("tile map already destroyed")
        return self._h

    def close(self) -> None:
        if self._h:
            torch.cuda.synchronize(self.device)
            load().psa_tile_map_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            if self._h and _lib is not None:
                torch.cuda.synchronize(self.device)
                _lib.psa_tile_map_destroy(self._h)
                self._h = ctypes.c_void_p(0)
        except Exception:
            pass

    def export(self) -> dict:
        """kinds [nq, nk], CSR and CSC as numpy arrays, and the mask encoding: end (an
        interval-form map) and key, lo, w (either form; see export_nodes)."""
        i = self.info
        T, nq, nk, nnz = i["T"], i["n_qtiles"], i["n_ktiles"], i["nnz"]
        interval = i["form"] == FORM_INTERVAL
        out = {"end": np.zeros(T if interval else 0, np.int32),
               "kinds": np.zeros(nq * nk, np.uint8),
               "row_ptr": np.zeros(nq + 1, np.int32), "col": np.zeros(nnz, np.int32),
               "kind": np.zeros(nnz, np.uint8), "col_ptr": np.zeros(nk + 1, np.int32),
               "row": np.zeros(nnz, np.int32), "kind_csc": np.zeros(nnz, np.uint8)}
        args = [ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)
                for a in out.values()]
        _check(load().psa_tile_map_export(self.handle, *args))
        out["kinds"] = out["kinds"].reshape(nq, nk)
        if not interval:
            del out["end"]
        out.update(self.export_nodes())
        return out

    def export_nodes(self) -> dict:
        """key, lo, w [T] int32: kv visible to q iff kv <= q and lo[kv] <= key[q] <
        lo[kv] + w[kv] (an interval-form map as key = lo = t, w = end - t)."""
        T = self.info["T"]
        out = {n: np.zeros(T, np.int32) for n in ("key", "lo", "w")}
        args = [ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)
                for a in out.values()]
        _check(load().psa_tile_map_export_nodes(self.handle, *args))
        return out


def build_tile_map_tokens(group: torch.Tensor, suffix: torch.Tensor, is_prefix: torch.Tensor,
                          block_m: Optional[int] = None, block_n: Optional[int] = None,
                          dtype: torch.dtype = torch.bfloat16, d: int = 128,
                          form: str = "auto") -> TileMap:
    """Tile map from per-token labels (device tensors: int32, int32, uint8).  form
    "auto": the interval form for packed layouts, else the node form; "nodes": always
    the node form."""
    lib = load()
    if block_m is None or block_n is None:
        block_m, block_n = tile_shape(PASS_FWD, dtype, d)
    for t, dt in ((group, torch.int32), (suffix, torch.int32), (is_prefix, torch.uint8)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise TypeError("labels must be contiguous device tensors (int32, int32, uint8)")
    T = group.numel()
    if suffix.numel() != T or is_prefix.numel() != T:
        raise ValueError("label tensors differ in length")
    dev = group.device
    out = ctypes.c_void_p()
    with torch.cuda.device(dev):
        _check(lib.psa_build_tile_map_tokens_ex(T, _ptr(group), _ptr(suffix), _ptr(is_prefix),
                                                block_m, block_n, _form_flags(form),
                                                _stream(dev), ctypes.byref(out)))
    return TileMap(out.value, dev)


def _form_flags(form: str) -> int:
    if form not in ("auto", "nodes"):
        raise ValueError('form must be "auto" or "nodes"')
    return MAP_NODE_FORM if form == "nodes" else 0


def build_tile_map_tree(node_lengths: Sequence[int], sample_paths: Sequence[Sequence[int]],
                        T: Optional[int] = None, device=None, block_m: Optional[int] = None,
                        block_n: Optional[int] = None, dtype: torch.dtype = torch.bfloat16,
                        d: int = 128, form: str = "auto") -> TileMap:
    """Tile map from a prefix tree given on the host (form as build_tile_map_tokens:
    "auto" takes the interval form for depth-first node orders)."""
    lib = load()
    if block_m is None or block_n is None:
        block_m, block_n = tile_shape(PASS_FWD, dtype, d)
    dev = torch.device(device) if device is not None else torch.device("cuda",
                                                                       torch.cuda.current_device())
    nl = np.ascontiguousarray(np.asarray(node_lengths, dtype=np.int32))
    ptr = np.zeros(len(sample_paths) + 1, np.int32)
    for s, p in enumerate(sample_paths):
        ptr[s + 1] = ptr[s] + len(p)
    nodes = np.ascontiguousarray(np.asarray([n for p in sample_paths for n in p], dtype=np.int32))
    if T is None:
        T = int(nl.sum())
    out = ctypes.c_void_p()

    def addr(a):
        return ctypes.c_void_p(a.ctypes.data if a.size else 0)

    with torch.cuda.device(dev):
        _check(lib.psa_build_tile_map_tree_ex(len(nl), addr(nl), len(sample_paths), addr(ptr),
                                              addr(nodes), int(T), block_m, block_n,
                                              _form_flags(form), _stream(dev),
                                              ctypes.byref(out)))
    return TileMap(out.value, dev)


def build_tile_map_draft(ctx_len: int, block_size: int, anchors: torch.Tensor,
                         keep: Optional[torch.Tensor] = None,
                         ctx_doc: Optional[torch.Tensor] = None,
                         anchor_doc: Optional[torch.Tensor] = None, causal: bool = False,
                         T: Optional[int] = None, block_m: Optional[int] = None,
                         block_n: Optional[int] = None, dtype: torch.dtype = torch.bfloat16,
                         d: int = 128) -> TileMap:
    """Tile map of the packed-document draft mask (device tensors: anchors int32 [N],
    keep uint8 [N] or None, ctx_doc int32 [ctx_len] and anchor_doc int32 [N], or both
    None).  Positions: the context, then N blocks of block_size draft tokens, then pads
    up to T."""
    lib = load()
    if block_m is None or block_n is None:
        block_m, block_n = tile_shape(PASS_FWD, dtype, d)
    n = anchors.numel()
    arrays = [(t, dt, size, name) for t, dt, size, name in (
        (anchors, torch.int32, n, "anchors"), (keep, torch.uint8, n, "keep"),
        (ctx_doc, torch.int32, ctx_len, "ctx_doc"), (anchor_doc, torch.int32, n, "anchor_doc"))
        if t is not None]
    for t, _, size, name in arrays:
        if t.numel() != size:
            raise ValueError(f"{name} must hold {size} values, not {t.numel()}")
    if (ctx_doc is None) != (anchor_doc is None):
        raise ValueError("ctx_doc and anchor_doc go together (both or neither)")
    for t, dt, _, name in arrays:
        if t.device != anchors.device:
            raise ValueError(f"{name} is on {t.device}, anchors on {anchors.device}")
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise TypeError("draft arrays must be contiguous device tensors (int32 / uint8)")
    if T is None:
        T = ctx_len + n * block_size
    dev = anchors.device
    out = ctypes.c_void_p()
    with torch.cuda.device(dev):
        _check(lib.psa_build_tile_map_draft(int(ctx_len), int(block_size), n, _ptr(anchors),
                                            _ptr(keep), _ptr(ctx_doc), _ptr(anchor_doc),
                                            DRAFT_CAUSAL if causal else 0, int(T), block_m,
                                            block_n, _stream(dev), ctypes.byref(out)))
    return TileMap(out.value, dev)


def _check_qkv(q, k, v):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, heads, d]")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v must share a dtype")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("shape mismatch between q and k/v")


def _check_buf(t: torch.Tensor, shape, dtype: torch.dtype, device, name: str) -> None:
    """A caller-supplied buffer the kernels read or write whole: its shape, dtype,
    layout and device must be the ones they assume."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {device}")


def fwd(m: TileMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, with_lse: bool = True):
    """O [T, hq, d] (q's dtype; bfloat16 for float8_e4m3fn inputs) and LSE [hq, T]
    float32.  with_lse=False: a forward without gradient; no LSE is written and None is
    returned in its place."""
    lib = load()
    _check_qkv(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    o_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if out is None:
        o = torch.empty(q.shape, device=q.device, dtype=o_dtype)
    else:
        _check_buf(out, q.shape, o_dtype, q.device, "out")
        o = out
    if not with_lse:
        lse_t = None
    elif lse is None:
        lse_t = torch.empty(hq, T, device=q.device, dtype=torch.float32)
    else:
        _check_buf(lse, (hq, T), torch.float32, q.device, "lse")
        lse_t = lse
    with torch.cuda.device(q.device):
        _check(lib.psa_fwd(m.handle, _dtype_code(q.dtype), T, hq, hkv, d,
                           0.0 if scale is None else float(scale), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(o), _ptr(lse_t), _stream(q.device)))
    return o, lse_t


def bwd_workspace_size(m: TileMap, q: torch.Tensor, k: torch.Tensor) -> int:
    lib = load()
    T, hq, d = q.shape
    n = ctypes.c_size_t()
    _check(lib.psa_bwd_workspace_size(m.handle, _dtype_code(q.dtype), T, hq, k.shape[1], d,
                                      ctypes.byref(n)))
    return n.value


def bwd(m: TileMap, q, k, v, o, lse, do, scale: Optional[float] = None,
        workspace: Optional[torch.Tensor] = None, grad_dtype: torch.dtype = torch.float32,
        stages: int = STAGE_ALL, out=None, split: bool = False):
    """dQ, dK, dV in ``grad_dtype`` (float32, the default, or q's dtype).

    ``stages`` selects backward stages (psa_bwd_stages); ``split`` carries P and dS as
    hi + lo bf16 pairs (PSA_BWD_SPLIT_PDS); ``out`` = (dq, dk, dv) reuses output
    buffers."""
    lib = load()
    _check_qkv(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    _check_buf(o, q.shape, q.dtype, q.device, "o")
    _check_buf(do, q.shape, q.dtype, q.device, "do")
    _check_buf(lse, (hq, T), torch.float32, q.device, "lse")
    need = bwd_workspace_size(m, q, k)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif not ws.is_contiguous() or ws.device != q.device:
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    if out is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    else:
        dq, dk, dv = out
        _check_buf(dq, q.shape, grad_dtype, q.device, "dq")
        _check_buf(dk, k.shape, grad_dtype, q.device, "dk")
        _check_buf(dv, v.shape, grad_dtype, q.device, "dv")
    with torch.cuda.device(q.device):
        _check(lib.psa_bwd_stages(m.handle, _dtype_code(q.dtype), _dtype_code(grad_dtype), T, hq,
                                  hkv, d, 0.0 if scale is None else float(scale), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(),
                                  stages | (BWD_SPLIT_PDS if split else 0), _stream(q.device)))
    return dq, dk, dv


class PrefixAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libpsa's kernels."""

    @staticmethod
    def forward(ctx, q, k, v, tile_map, scale=None):
        o, lse = fwd(tile_map, q.contiguous(), k.contiguous(), v.contiguous(), scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.tile_map = tile_map
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(ctx.tile_map, q, k, v, o, lse, do.to(q.dtype).contiguous(), ctx.scale)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None


def layout_tile_map(layout, device, dtype: torch.dtype = torch.bfloat16, d: int = 128,
                    block_m: Optional[int] = None, block_n: Optional[int] = None,
                    form: str = "auto") -> TileMap:
    """Tile map of a workloads.Layout (token labels are copied to the device)."""
    if layout.kind == "draft":
        x = layout.extra
        dv = lambda a, dt: torch.as_tensor(a, dtype=dt).to(device)  # noqa: E731
        docs = x["ctx_len"] > 0  # an empty context has no documents to compare
        return build_tile_map_draft(x["ctx_len"], x["block_size"], dv(x["anchors"], torch.int32),
                                    dv(x["keep"], torch.uint8),
                                    dv(x["ctx_doc"], torch.int32) if docs else None,
                                    dv(x["anchor_doc"], torch.int32) if docs else None,
                                    x["causal"], layout.T, block_m, block_n, dtype, d)
    if layout.kind == "tokens":
        g = torch.as_tensor(layout.group, dtype=torch.int32).to(device)
        s = torch.as_tensor(layout.suffix, dtype=torch.int32).to(device)
        p = torch.as_tensor(layout.is_prefix, dtype=torch.uint8).to(device)
        return build_tile_map_tokens(g, s, p, block_m, block_n, dtype, d, form)
    return build_tile_map_tree(layout.node_lengths, layout.sample_paths, layout.T, device,
                               block_m, block_n, dtype, d, form)


# ----------------------------------------------------------------------------
# fold / unfold of rollout groups
# ----------------------------------------------------------------------------
class Rollouts:
    """Host length tables of rollout groups: prompt_len[g], and per group the lengths
    of its completions.  ``fold_len`` is the folded length (sum of all lengths)."""

    def __init__(self, prompt_lens: Sequence[int], comp_lens: Sequence[Sequence[int]]):
        if len(prompt_lens) != len(comp_lens):
            raise ValueError("one completion list per prompt")
        self.prompt_len = np.ascontiguousarray(prompt_lens, dtype=np.int32)
        self.comp_ptr = np.zeros(len(comp_lens) + 1, dtype=np.int32)
        self.comp_ptr[1:] = np.cumsum([len(c) for c in comp_lens])
        flat = [r for c in comp_lens for r in c]
        self.comp_len = np.ascontiguousarray(flat if flat else [0], dtype=np.int32)
        self.n_groups = len(prompt_lens)
        self.n_comp = int(self.comp_ptr[-1])
        self.fold_len = int(self.prompt_len.sum()) + int(sum(flat))
        self.unfold_len = int(sum(self.prompt_len[g] * (self.comp_ptr[g + 1] - self.comp_ptr[g])
                                  for g in range(self.n_groups))) + int(sum(flat))

    def _tables(self):
        np_ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        return (self.n_groups, np_ptr(self.prompt_len), np_ptr(self.comp_ptr),
                np_ptr(self.comp_len))


def _fold_ws_bytes(r: Rollouts) -> int:
    b = ctypes.c_size_t(0)
    _check(load().psa_fold_workspace_size(r.n_groups, r.n_comp, ctypes.byref(b)))
    return b.value


def fold_workspace(r: Rollouts, device) -> torch.Tensor:
    return torch.empty(_fold_ws_bytes(r), dtype=torch.uint8, device=device)


def _check_ws(ws: torch.Tensor, r: Rollouts, device) -> None:
    if not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < _fold_ws_bytes(r):
        raise ValueError("workspace smaller than psa_fold_workspace_size")


def fold_rollouts(r: Rollouts, prompt_tok: torch.Tensor, comp_tok: torch.Tensor, T: int,
                  pad_id: int = 0, ignore_index: int = -100,
                  workspace: Optional[torch.Tensor] = None) -> dict:
    """input_ids, labels, position_ids, group, suffix (int32 [T]) and is_prefix (uint8
    [T]) of the folded layout; prompt_tok / comp_tok: int32 device tokens."""
    lib = load()
    dev = prompt_tok.device
    n_prompt = int(r.prompt_len.sum())
    toks = ((prompt_tok, n_prompt, "prompt_tok"), (comp_tok, r.fold_len - n_prompt, "comp_tok"))
    for t, size, name in toks:
        if t.numel() != size:
            raise ValueError(f"{name} must hold {size} tokens, not {t.numel()}")
    if comp_tok.device != dev:
        raise ValueError("prompt_tok and comp_tok must be on one device")
    for t, _, name in toks:
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    out = {k: torch.empty(T, dtype=torch.int32, device=dev)
           for k in ("input_ids", "labels", "position_ids", "group", "suffix")}
    out["is_prefix"] = torch.empty(T, dtype=torch.uint8, device=dev)
    ws = fold_workspace(r, dev) if workspace is None else workspace
    _check_ws(ws, r, dev)
    with torch.cuda.device(dev):
        _check(lib.psa_fold_rollouts(*r._tables(), _ptr(prompt_tok), _ptr(comp_tok), T, pad_id,
                                     ignore_index, _ptr(out["input_ids"]), _ptr(out["labels"]),
                                     _ptr(out["position_ids"]), _ptr(out["group"]),
                                     _ptr(out["suffix"]), _ptr(out["is_prefix"]), _ptr(ws),
                                     ws.numel(), _stream(dev)))
    return out


def unfold_rows(r: Rollouts, src: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of a folded [T, ...] device tensor gathered per sample ([prompt_g | c_gi])."""
    lib = load()
    if src.dim() < 1 or src.shape[0] < r.fold_len:
        raise ValueError(f"src must have at least the folded layout's {r.fold_len} rows")
    if not src.is_contiguous() or not src.is_cuda:
        raise ValueError("src must be a contiguous device tensor [T, ...]")
    T = src.shape[0]
    row_bytes = (src.numel() // T) * src.element_size() if T else 0
    shape = (r.unfold_len,) + tuple(src.shape[1:])
    if out is None:
        dst = torch.empty(shape, dtype=src.dtype, device=src.device)
    else:
        _check_buf(out, shape, src.dtype, src.device, "out")
        dst = out
    ws = fold_workspace(r, src.device) if workspace is None else workspace
    _check_ws(ws, r, src.device)
    with torch.cuda.device(src.device):
        _check(lib.psa_unfold_rows(*r._tables(), T, row_bytes, _ptr(src), _ptr(dst),
                                   dst.numel() * dst.element_size(), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(src.device)))
    return dst
