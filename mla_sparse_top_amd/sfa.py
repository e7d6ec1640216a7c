"""Thin ctypes binding over libsfa.so (include/sfa.h). Argument marshalling only: every step of
the attention runs in the library's HIP kernels. PyTorch supplies device memory and streams.

Importing this module loads the native library and raises ImportError if it has not been built
(``python -m mla_sparse_top_amd.build``). There is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsfa.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m mla_sparse_top_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

KV_LORA_RANK = 512
ROPE_DIM = 64
BLOCK_SIZE = 128
KV_BF16 = 0
KV_INT8 = 1

STATUS = {
    0: "SFA_OK", -1: "SFA_ERR_NULL", -2: "SFA_ERR_DIMS", -3: "SFA_ERR_ALIGN", -4: "SFA_ERR_WORKSPACE",
    -5: "SFA_ERR_SCALES", -6: "SFA_ERR_ALIAS", -7: "SFA_ERR_SCALE_VALUE", -8: "SFA_ERR_HIP",
    -9: "SFA_ERR_SCRATCH_LIMIT",
}


class SfaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s1", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("n_kv", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("max_blocks_per_batch", ctypes.c_int32),
        ("num_cache_rows", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_ATTN_ARGS = [ctypes.POINTER(SfaDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
              ctypes.c_size_t, _vp]
for _name in ("sfa_decode", "sfa_prefill"):
    getattr(_lib, _name).argtypes = _ATTN_ARGS
    getattr(_lib, _name).restype = ctypes.c_int
_lib.sfa_decode_noalloc.argtypes = _ATTN_ARGS[:11] + [_vp]
_lib.sfa_decode_noalloc.restype = ctypes.c_int
# fixed scratch of sfa_decode_noalloc per GPU (SFA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 72 << 20
_lib.sfa_workspace_size.argtypes = [ctypes.POINTER(SfaDims), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
_lib.sfa_workspace_size.restype = ctypes.c_int
_lib.sfa_num_splits.argtypes = [ctypes.POINTER(SfaDims), ctypes.c_int]
_lib.sfa_num_splits.restype = ctypes.c_int
_lib.sfa_resolve_rows.argtypes = [ctypes.POINTER(SfaDims), _vp, _vp, _vp, _vp, _vp]
_lib.sfa_resolve_rows.restype = ctypes.c_int
_lib.sfa_status_string.argtypes = [ctypes.c_int]
_lib.sfa_status_string.restype = ctypes.c_char_p

class SfaIndexerDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s1", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_batch", ctypes.c_int32),
        ("num_cache_rows", ctypes.c_int64),
        ("topk", ctypes.c_int32),
    ]


_lib.sfa_indexer_scores.argtypes = [ctypes.POINTER(SfaIndexerDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.sfa_indexer_scores.restype = ctypes.c_int
_lib.sfa_topk_select.argtypes = [ctypes.POINTER(SfaIndexerDims), _vp, _vp, _vp, _vp]
_lib.sfa_topk_select.restype = ctypes.c_int

_lib.sfa_cache_write.argtypes = [ctypes.POINTER(SfaDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.sfa_cache_write.restype = ctypes.c_int

class SfaWindowDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s1", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("n_kv", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("topk_cmp", ctypes.c_int32),
        ("max_blocks_ori", ctypes.c_int32),
        ("max_blocks_cmp", ctypes.c_int32),
        ("num_cache_rows", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


_lib.sfa_window_workspace_size.argtypes = [ctypes.POINTER(SfaWindowDims), ctypes.POINTER(ctypes.c_size_t)]
_lib.sfa_window_workspace_size.restype = ctypes.c_int
_lib.sfa_window_decode.argtypes = [ctypes.POINTER(SfaWindowDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]
_lib.sfa_window_decode.restype = ctypes.c_int



class SfaCompressDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s1", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("ratio", ctypes.c_int32),
        ("rope_positions", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("num_cache_rows", ctypes.c_int64),
    ]


_lib.sfa_compress.argtypes = [ctypes.POINTER(SfaCompressDims), _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp]
_lib.sfa_compress.restype = ctypes.c_int

class SfaPrologDims(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("qk_nope_dim", ctypes.c_int32),
        ("rope_positions", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


_lib.sfa_mla_prolog_workspace_size.argtypes = [ctypes.POINTER(SfaPrologDims), ctypes.POINTER(ctypes.c_size_t)]
_lib.sfa_mla_prolog_workspace_size.restype = ctypes.c_int
_lib.sfa_mla_prolog.argtypes = [ctypes.POINTER(SfaPrologDims)] + [_vp] * 16 + [ctypes.c_size_t, _vp]
_lib.sfa_mla_prolog.restype = ctypes.c_int


class SfaPrologV4Dims(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_positions", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


_lib.sfa_mla_prolog_v4_workspace_size.argtypes = [ctypes.POINTER(SfaPrologV4Dims), ctypes.POINTER(ctypes.c_size_t)]
_lib.sfa_mla_prolog_v4_workspace_size.restype = ctypes.c_int
_lib.sfa_mla_prolog_v4.argtypes = [ctypes.POINTER(SfaPrologV4Dims)] + [_vp] * 13 + [ctypes.c_size_t, _vp, _vp]
_lib.sfa_mla_prolog_v4.restype = ctypes.c_int


class SfaIndexerPrologDims(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_positions", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


_lib.sfa_indexer_prolog_workspace_size.argtypes = [ctypes.POINTER(SfaIndexerPrologDims),
                                                   ctypes.POINTER(ctypes.c_size_t)]
_lib.sfa_indexer_prolog_workspace_size.restype = ctypes.c_int
_lib.sfa_indexer_prolog.argtypes = [ctypes.POINTER(SfaIndexerPrologDims)] + [_vp] * 14 + [ctypes.c_size_t, _vp]
_lib.sfa_indexer_prolog.restype = ctypes.c_int



EXPORTED_SYMBOLS = ("sfa_workspace_size", "sfa_num_splits", "sfa_decode", "sfa_prefill", "sfa_resolve_rows",
                    "sfa_status_string", "sfa_indexer_scores", "sfa_topk_select", "sfa_cache_write",
                    "sfa_window_workspace_size", "sfa_window_decode", "sfa_compress", "sfa_decode_noalloc",
                    "sfa_mla_prolog_workspace_size", "sfa_mla_prolog", "sfa_mla_prolog_v4_workspace_size",
                    "sfa_mla_prolog_v4", "sfa_indexer_prolog_workspace_size", "sfa_indexer_prolog")


class SfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def status_string(status: int) -> str:
    return _lib.sfa_status_string(int(status)).decode()


def lib_path() -> str:
    return _LIB_PATH


def make_dims(*, batch: int, s1: int, n_q: int, topk: int, max_blocks_per_batch: int, num_cache_rows: int,
              kv_dtype: int = KV_BF16, num_splits: int = 0, n_kv: int = 1, kv_lora_rank: int = KV_LORA_RANK,
              rope_dim: int = ROPE_DIM, block_size: int = BLOCK_SIZE) -> SfaDims:
    return SfaDims(batch, s1, n_q, n_kv, kv_lora_rank, rope_dim, block_size, topk, max_blocks_per_batch,
                   num_cache_rows, kv_dtype, num_splits)


def workspace_size(dims: SfaDims, is_prefill: bool = False) -> int:
    out = ctypes.c_size_t(0)
    st = _lib.sfa_workspace_size(ctypes.byref(dims), int(bool(is_prefill)), ctypes.byref(out))
    if st != 0:
        raise SfaError(st, "sfa_workspace_size")
    return int(out.value)


def num_splits(dims: SfaDims, is_prefill: bool = False) -> int:
    st = _lib.sfa_num_splits(ctypes.byref(dims), int(bool(is_prefill)))
    if st < 0:
        raise SfaError(st, "sfa_num_splits")
    return st


# One workspace per (device, stream), grown on demand. Calls queued on one stream run one after
# the other and can share a buffer (each call tags its counters with a generation of its own, so
# no clearing is needed); calls on different streams may overlap, so they never share one.
_WORKSPACES: dict = {}


def get_workspace(device: torch.device, nbytes: int, stream=None) -> Optional[torch.Tensor]:
    """The cached workspace of (device, stream) with at least nbytes, or None for nbytes == 0.
    stream defaults to the device's current stream."""
    if nbytes == 0:
        return None
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        # The contents need no initialisation (the library's counters are generation-tagged).
        # The allocator ties a block to the stream current at allocation; record the stream the
        # kernels use so that the block is not handed out again while they may still run.
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if stream.cuda_stream != torch.cuda.current_stream(device).cuda_stream:
            ws.record_stream(stream)
        _WORKSPACES[key] = ws
    return ws


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


def _marshal_attention(fn_name: str, query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices,
                       block_table, kv_act_seqs, softmax_scale, *, batch, s1, out=None, workspace=None,
                       num_splits_override=0, stream=None):
    """Checks the tensors and builds the C argument tuple of sfa_decode / sfa_prefill, or of
    sfa_decode_noalloc (no workspace arguments). Returns (args, out, keepalive)."""
    dev = query_nope.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t_tokens = batch * s1
    n_q = query_nope.shape[0] // t_tokens if t_tokens else 0
    topk = topk_indices.shape[1] if topk_indices.dim() == 2 else 0
    rows = key_rope.shape[0]
    _check(query_nope, "query_nope", (torch.bfloat16,), (t_tokens * n_q, KV_LORA_RANK), dev)
    _check(query_rope, "query_rope", (torch.bfloat16,), (t_tokens * n_q, ROPE_DIM), dev)
    _check(key_nope, "key_nope", (torch.bfloat16, torch.int8), (rows, KV_LORA_RANK), dev)
    _check(key_rope, "key_rope", (torch.bfloat16,), (rows, ROPE_DIM), dev)
    int8 = key_nope.dtype == torch.int8
    if int8:
        if k_nope_scales is None:
            raise ValueError("an int8 key_nope needs k_nope_scales")
        _check(k_nope_scales, "k_nope_scales", (torch.float32,), (rows, 4), dev)
    _check(topk_indices, "topk_indices", (torch.int32,), (t_tokens, topk), dev)
    _check(block_table, "block_table", (torch.int32,), None, dev)
    _check(kv_act_seqs, "kv_act_seqs", (torch.int32,), (batch,), dev)
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be (batch, max_blocks_per_batch)")
    dims = make_dims(batch=batch, s1=s1, n_q=n_q, topk=topk, max_blocks_per_batch=block_table.shape[1],
                     num_cache_rows=rows, kv_dtype=KV_INT8 if int8 else KV_BF16, num_splits=num_splits_override)
    if out is None:
        out = torch.empty((batch, s1, n_q, KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    _check(out, "out", (torch.bfloat16,), (batch, s1, n_q, KV_LORA_RANK), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if fn_name == "sfa_decode_noalloc":
        args = (ctypes.byref(dims), _ptr(query_nope), _ptr(query_rope), _ptr(key_nope), _ptr(key_rope),
                _ptr(k_nope_scales if int8 else None), _ptr(topk_indices), _ptr(block_table), _ptr(kv_act_seqs),
                ctypes.c_float(softmax_scale), _ptr(out), ctypes.c_void_p(stream.cuda_stream))
        keep = (dims, query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table,
                kv_act_seqs, out, stream)
        return args, out, keep
    need = workspace_size(dims, fn_name == "sfa_prefill")
    if workspace is None:
        workspace = get_workspace(dev, need, stream)
    elif need:
        _check(workspace, "workspace", (torch.uint8,), None, dev)
    args = (ctypes.byref(dims), _ptr(query_nope), _ptr(query_rope), _ptr(key_nope), _ptr(key_rope),
            _ptr(k_nope_scales if int8 else None), _ptr(topk_indices), _ptr(block_table), _ptr(kv_act_seqs),
            ctypes.c_float(softmax_scale), _ptr(out), _ptr(workspace) if need else None,
            ctypes.c_size_t(workspace.numel() if (need and workspace is not None) else 0),
            ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table, kv_act_seqs,
            out, workspace, stream)
    return args, out, keep


def _attention(fn_name: str, *tensors, **kw):
    args, out, _keep = _marshal_attention(fn_name, *tensors, **kw)
    st = getattr(_lib, fn_name)(*args)
    if st != 0:
        raise SfaError(st, fn_name)
    return out


class PreparedCall:
    """One entry point bound to fixed tensors, for loops that repeat the same call (a serving
    step, a benchmark). The Python checks and the argument marshalling run once, here; each
    call only invokes the C function, which still validates its arguments on the host and
    queues the kernels on the bound stream. The tensors are kept alive by this object; their
    contents may change between calls, their storage must not."""

    def __init__(self, calls, out, keep):
        self._calls = calls  # [(c function, args, name)]
        self.out = out
        self._keep = keep

    def __call__(self):
        for fn, args, name in self._calls:
            st = fn(*args)
            if st != 0:
                raise SfaError(st, name)
        return self.out


def decode(query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table, kv_act_seqs,
           softmax_scale, *, batch, s1, out=None, workspace=None, num_splits=0, stream=None):
    """sfa_decode: returns out (batch, s1, n_q, 512) bf16."""
    return _attention("sfa_decode", query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices,
                      block_table, kv_act_seqs, softmax_scale, batch=batch, s1=s1, out=out, workspace=workspace,
                      num_splits_override=num_splits, stream=stream)


def prefill(query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table, kv_act_seqs,
            softmax_scale, *, batch, s1, out=None, workspace=None, num_splits=0, stream=None):
    """sfa_prefill: returns out (batch, s1, n_q, 512) bf16."""
    return _attention("sfa_prefill", query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices,
                      block_table, kv_act_seqs, softmax_scale, batch=batch, s1=s1, out=out, workspace=workspace,
                      num_splits_override=num_splits, stream=stream)


def decode_noalloc(query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table,
                   kv_act_seqs, softmax_scale, *, batch, s1, out=None, num_splits=0, stream=None):
    """sfa_decode_noalloc: sfa_decode with the library's fixed per-GPU scratch as its workspace
    (no device allocation by the library; out is allocated here only when not given). Calls
    that overlap on one GPU share that scratch and must not run at the same time."""
    return _attention("sfa_decode_noalloc", query_nope, query_rope, key_nope, key_rope, k_nope_scales,
                      topk_indices, block_table, kv_act_seqs, softmax_scale, batch=batch, s1=s1, out=out,
                      num_splits_override=num_splits, stream=stream)


def prepare_decode(query_nope, query_rope, key_nope, key_rope, k_nope_scales, topk_indices, block_table,
                   kv_act_seqs, softmax_scale, *, batch, s1, out=None, workspace=None, num_splits=0, stream=None,
                   prefill_mode=False) -> PreparedCall:
    """sfa_decode (or sfa_prefill) bound to these tensors: returns a PreparedCall whose call queues
    the attention and returns out."""
    name = "sfa_prefill" if prefill_mode else "sfa_decode"
    args, out, keep = _marshal_attention(name, query_nope, query_rope, key_nope, key_rope, k_nope_scales,
                                         topk_indices, block_table, kv_act_seqs, softmax_scale, batch=batch, s1=s1,
                                         out=out, workspace=workspace, num_splits_override=num_splits, stream=stream)
    return PreparedCall([(getattr(_lib, name), args, name)], out, keep)


def resolve_rows(topk_indices, block_table, kv_act_seqs, *, batch, s1, num_cache_rows, rows_out=None,
                 stream=None):
    """sfa_resolve_rows: returns rows_out (T, topk) int32, -1 for masked slots."""
    dev = topk_indices.device
    t_tokens = batch * s1
    topk = topk_indices.shape[1]
    _check(topk_indices, "topk_indices", (torch.int32,), (t_tokens, topk), dev)
    _check(block_table, "block_table", (torch.int32,), None, dev)
    _check(kv_act_seqs, "kv_act_seqs", (torch.int32,), (batch,), dev)
    dims = make_dims(batch=batch, s1=s1, n_q=128, topk=topk, max_blocks_per_batch=block_table.shape[1],
                     num_cache_rows=num_cache_rows)
    if rows_out is None:
        rows_out = torch.empty((t_tokens, topk), dtype=torch.int32, device=dev)
    _check(rows_out, "rows_out", (torch.int32,), (t_tokens, topk), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = _lib.sfa_resolve_rows(ctypes.byref(dims), _ptr(topk_indices), _ptr(block_table), _ptr(kv_act_seqs),
                               _ptr(rows_out), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise SfaError(st, "sfa_resolve_rows")
    return rows_out


def _marshal_cache_write(new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales, *, batch,
                        s1, stream=None):
    dev = new_nope.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t_tokens = batch * s1
    # new_rope and key_rope both None: 512-wide rows with the rotary channels inside (rope_dim 0)
    if (new_rope is None) != (key_rope is None):
        raise ValueError("new_rope and key_rope must both be given (512 + 64 channels) or both be None "
                         "(512-wide rows)")
    rope_dim = 0 if key_rope is None else ROPE_DIM
    rows = key_nope.shape[0]
    _check(new_nope, "new_nope", (torch.bfloat16,), (t_tokens, KV_LORA_RANK), dev)
    if rope_dim:
        _check(new_rope, "new_rope", (torch.bfloat16,), (t_tokens, ROPE_DIM), dev)
    _check(positions, "positions", (torch.int32,), (t_tokens,), dev)
    _check(block_table, "block_table", (torch.int32,), None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be (batch, max_blocks_per_batch)")
    _check(key_nope, "key_nope", (torch.bfloat16, torch.int8), (rows, KV_LORA_RANK), dev)
    if rope_dim:
        _check(key_rope, "key_rope", (torch.bfloat16,), (rows, ROPE_DIM), dev)
    int8 = key_nope.dtype == torch.int8
    if int8:
        if k_nope_scales is None:
            raise ValueError("an int8 key_nope needs k_nope_scales")
        _check(k_nope_scales, "k_nope_scales", (torch.float32,), (rows, 4), dev)
    dims = make_dims(batch=batch, s1=s1, n_q=128, topk=1, max_blocks_per_batch=block_table.shape[1],
                     num_cache_rows=rows, kv_dtype=KV_INT8 if int8 else KV_BF16, rope_dim=rope_dim)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (ctypes.byref(dims), _ptr(new_nope), _ptr(new_rope), _ptr(positions), _ptr(block_table), _ptr(key_nope),
            _ptr(key_rope), _ptr(k_nope_scales if int8 else None), ctypes.c_void_p(stream.cuda_stream))
    return args, (dims, new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales, stream)


def cache_write(new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales=None, *, batch, s1,
                stream=None):
    """sfa_cache_write: writes the new latent rows into the paged cache tensors in place (an int8
    key_nope is quantised per 128-element group into it and k_nope_scales). Returns key_nope."""
    args, _keep = _marshal_cache_write(new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales,
                                       batch=batch, s1=s1, stream=stream)
    st = _lib.sfa_cache_write(*args)
    if st != 0:
        raise SfaError(st, "sfa_cache_write")
    return key_nope


def window_workspace_size(dims: SfaWindowDims) -> int:
    out = ctypes.c_size_t(0)
    st = _lib.sfa_window_workspace_size(ctypes.byref(dims), ctypes.byref(out))
    if st != 0:
        raise SfaError(st, "sfa_window_workspace_size")
    return int(out.value)


def _marshal_window(query_nope, query_rope, key_nope, key_rope, k_nope_scales, cmp_indices, block_table_ori,
                    block_table_cmp, ori_len, cmp_len, softmax_scale, *, batch, s1, window, out=None, workspace=None,
                    num_splits=0, stream=None):
    dev = query_nope.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t_tokens = batch * s1
    n_q = query_nope.shape[0] // t_tokens if t_tokens else 0
    # query_rope and key_rope both None: 512-wide rows with the rotary channels inside (rope_dim 0)
    if (query_rope is None) != (key_rope is None):
        raise ValueError("query_rope and key_rope must both be given (512 + 64 channels) or both be None "
                         "(512-wide rows)")
    rope_dim = 0 if key_rope is None else ROPE_DIM
    rows = key_nope.shape[0]
    _check(query_nope, "query_nope", (torch.bfloat16,), (t_tokens * n_q, KV_LORA_RANK), dev)
    _check(key_nope, "key_nope", (torch.bfloat16, torch.int8), (rows, KV_LORA_RANK), dev)
    if rope_dim:
        _check(query_rope, "query_rope", (torch.bfloat16,), (t_tokens * n_q, ROPE_DIM), dev)
        _check(key_rope, "key_rope", (torch.bfloat16,), (rows, ROPE_DIM), dev)
    int8 = key_nope.dtype == torch.int8
    if int8:
        if k_nope_scales is None:
            raise ValueError("an int8 key_nope needs k_nope_scales")
        _check(k_nope_scales, "k_nope_scales", (torch.float32,), (rows, 4), dev)
    _check(block_table_ori, "block_table_ori", (torch.int32,), None, dev)
    _check(ori_len, "ori_len", (torch.int32,), (batch,), dev)
    topk_cmp = 0 if cmp_indices is None else int(cmp_indices.shape[1])
    if topk_cmp:
        _check(cmp_indices, "cmp_indices", (torch.int32,), (t_tokens, topk_cmp), dev)
        _check(block_table_cmp, "block_table_cmp", (torch.int32,), None, dev)
        _check(cmp_len, "cmp_len", (torch.int32,), (batch,), dev)
    dims = SfaWindowDims(batch, s1, n_q, 1, KV_LORA_RANK, rope_dim, BLOCK_SIZE, int(window), topk_cmp,
                         block_table_ori.shape[1], block_table_cmp.shape[1] if topk_cmp else 0, rows,
                         KV_INT8 if int8 else KV_BF16, num_splits)
    if out is None:
        out = torch.empty((batch, s1, n_q, KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    _check(out, "out", (torch.bfloat16,), (batch, s1, n_q, KV_LORA_RANK), dev)
    need = window_workspace_size(dims)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need:
        workspace = get_workspace(dev, need, stream)
    if workspace is not None:
        _check(workspace, "workspace", (torch.uint8,), None, dev)
    args = (ctypes.byref(dims), _ptr(query_nope), _ptr(query_rope), _ptr(key_nope), _ptr(key_rope),
            _ptr(k_nope_scales if int8 else None), _ptr(cmp_indices if topk_cmp else None), _ptr(block_table_ori),
            _ptr(block_table_cmp if topk_cmp else None), _ptr(ori_len), _ptr(cmp_len if topk_cmp else None),
            ctypes.c_float(softmax_scale), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() if workspace is not None else 0), ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, query_nope, query_rope, key_nope, key_rope, k_nope_scales, cmp_indices, block_table_ori,
            block_table_cmp, ori_len, cmp_len, out, workspace, stream)
    return args, out, keep


def window_decode(*tensors, **kw):
    """sfa_window_decode (SWA / CFA / SCFA): returns out (batch, s1, n_q, 512) bf16. With
    query_rope and key_rope None the rows are 512 wide with the rotary channels inside them."""
    args, out, _keep = _marshal_window(*tensors, **kw)
    st = _lib.sfa_window_decode(*args)
    if st != 0:
        raise SfaError(st, "sfa_window_decode")
    return out


def prepare_window_decode(*tensors, **kw) -> PreparedCall:
    """sfa_window_decode bound to these tensors (a PreparedCall returning out)."""
    args, out, keep = _marshal_window(*tensors, **kw)
    return PreparedCall([(_lib.sfa_window_decode, args, "sfa_window_decode")], out, keep)


def window_to_device(inp, device="cuda"):
    """Upload a workloads.WindowInputs instance."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    cmp = inp.cmp_indices is not None
    rope = inp.key_rope.shape[1] > 0  # zero-width rope arrays: 512-wide rows
    return {
        "query_nope": bf16(inp.query_nope),
        "query_rope": bf16(inp.query_rope) if rope else None,
        "key_nope": bf16(inp.key_nope) if inp.kv_dtype == "bf16" else torch.from_numpy(inp.key_nope).to(device),
        "key_rope": bf16(inp.key_rope) if rope else None,
        "k_nope_scales": None if inp.k_nope_scales is None else torch.from_numpy(inp.k_nope_scales).to(device),
        "cmp_indices": torch.from_numpy(inp.cmp_indices).to(device) if cmp else None,
        "block_table_ori": torch.from_numpy(inp.block_table_ori).to(device),
        "block_table_cmp": torch.from_numpy(inp.block_table_cmp).to(device) if cmp else None,
        "ori_len": torch.from_numpy(inp.ori_len).to(device),
        "cmp_len": torch.from_numpy(inp.cmp_len).to(device) if cmp else None,
    }


def _window_args(inp, d):
    return (d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"], d["cmp_indices"],
            d["block_table_ori"], d["block_table_cmp"], d["ori_len"], d["cmp_len"], inp.softmax_scale)


def run_window(inp, d=None, *, num_splits=0, out=None):
    """sfa_window_decode on an uploaded WindowInputs instance."""
    d = d if d is not None else window_to_device(inp)
    return window_decode(*_window_args(inp, d), batch=inp.batch, s1=inp.s1, window=inp.window, out=out,
                         num_splits=num_splits)


def prepare_window_run(inp, d, *, out=None, num_splits=0) -> PreparedCall:
    return prepare_window_decode(*_window_args(inp, d), batch=inp.batch, s1=inp.s1, window=inp.window, out=out,
                                 num_splits=num_splits)


def to_device(inp, device="cuda"):
    """Upload a workloads.SfaInputs instance: bf16 bit patterns become torch.bfloat16 tensors."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    kn = bf16(inp.key_nope) if inp.kv_dtype == "bf16" else torch.from_numpy(inp.key_nope).to(device)
    return {
        "query_nope": bf16(inp.query_nope),
        "query_rope": bf16(inp.query_rope),
        "key_nope": kn,
        "key_rope": bf16(inp.key_rope),
        "k_nope_scales": None if inp.k_nope_scales is None else torch.from_numpy(inp.k_nope_scales).to(device),
        "topk_indices": torch.from_numpy(inp.topk_indices).to(device),
        "block_table": torch.from_numpy(inp.block_table).to(device),
        "kv_act_seqs": torch.from_numpy(inp.kv_act_seqs).to(device),
    }


def prepare_run(inp, dev_tensors, *, prefill_mode=False, num_splits=0, out=None) -> PreparedCall:
    """prepare_decode on an uploaded instance."""
    d = dev_tensors
    return prepare_decode(d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"],
                          d["topk_indices"], d["block_table"], d["kv_act_seqs"], inp.softmax_scale, batch=inp.batch,
                          s1=inp.s1, num_splits=num_splits, out=out, prefill_mode=prefill_mode)


def run(inp, dev_tensors=None, *, prefill_mode=False, num_splits=0, out=None):
    """Run decode (or prefill) on an uploaded instance; returns the bf16 output tensor."""
    d = dev_tensors if dev_tensors is not None else to_device(inp)
    fn = prefill if prefill_mode else decode
    return fn(d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"], d["topk_indices"],
              d["block_table"], d["kv_act_seqs"], inp.softmax_scale, batch=inp.batch, s1=inp.s1,
              num_splits=num_splits, out=out)


# ---- Lightning Indexer ---------------------------------------------------------------------

INDEX_HEADS = 64
INDEX_DIM = 128


def make_indexer_dims(*, batch: int, s1: int, max_blocks_per_batch: int, num_cache_rows: int, topk: int,
                      n_heads: int = INDEX_HEADS, head_dim: int = INDEX_DIM, block_size: int = BLOCK_SIZE):
    return SfaIndexerDims(batch, s1, n_heads, head_dim, block_size, max_blocks_per_batch, num_cache_rows, topk)


def _marshal_indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs, *, batch, s1, topk=1,
                            scores=None, stream=None):
    dev = q_index.device
    t_tokens = batch * s1
    rows = k_index_cache.shape[0]
    mb = block_table.shape[1]
    _check(q_index, "q_index", (torch.bfloat16,), (t_tokens * INDEX_HEADS, INDEX_DIM), dev)
    _check(k_index_cache, "k_index_cache", (torch.bfloat16,), (rows, INDEX_DIM), dev)
    _check(weights, "weights", (torch.float32,), (t_tokens, INDEX_HEADS), dev)
    _check(block_table, "block_table", (torch.int32,), (batch, mb), dev)
    _check(kv_act_seqs, "kv_act_seqs", (torch.int32,), (batch,), dev)
    dims = make_indexer_dims(batch=batch, s1=s1, max_blocks_per_batch=mb, num_cache_rows=rows, topk=topk)
    if scores is None:
        scores = torch.empty((t_tokens, mb * BLOCK_SIZE), dtype=torch.float32, device=dev)
    _check(scores, "scores", (torch.float32,), (t_tokens, mb * BLOCK_SIZE), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (ctypes.byref(dims), _ptr(q_index), _ptr(k_index_cache), _ptr(weights), _ptr(block_table),
            _ptr(kv_act_seqs), _ptr(scores), ctypes.c_void_p(stream.cuda_stream))
    return args, scores, (dims, q_index, k_index_cache, weights, block_table, kv_act_seqs, scores, stream)


def _marshal_topk_select(scores, kv_act_seqs, *, batch, s1, topk, out=None, stream=None):
    dev = scores.device
    t_tokens = batch * s1
    n_pos = scores.shape[1]
    _check(scores, "scores", (torch.float32,), (t_tokens, n_pos), dev)
    _check(kv_act_seqs, "kv_act_seqs", (torch.int32,), (batch,), dev)
    if n_pos % BLOCK_SIZE:
        raise ValueError("scores must have a multiple of 128 columns")
    dims = make_indexer_dims(batch=batch, s1=s1, max_blocks_per_batch=n_pos // BLOCK_SIZE, num_cache_rows=0,
                             topk=topk)
    if out is None:
        out = torch.empty((t_tokens, topk), dtype=torch.int32, device=dev)
    _check(out, "topk_indices", (torch.int32,), (t_tokens, topk), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (ctypes.byref(dims), _ptr(scores), _ptr(kv_act_seqs), _ptr(out), ctypes.c_void_p(stream.cuda_stream))
    return args, out, (dims, scores, kv_act_seqs, out, stream)


def indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs, *, batch, s1, topk=1,
                   scores=None, stream=None):
    """sfa_indexer_scores: returns scores (batch*s1, max_blocks_per_batch*128) fp32."""
    args, scores, _keep = _marshal_indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs,
                                                  batch=batch, s1=s1, topk=topk, scores=scores, stream=stream)
    st = _lib.sfa_indexer_scores(*args)
    if st != 0:
        raise SfaError(st, "sfa_indexer_scores")
    return scores


def topk_select(scores, kv_act_seqs, *, batch, s1, topk, out=None, stream=None):
    """sfa_topk_select: returns topk_indices (batch*s1, topk) int32 (unsorted, -1 padded)."""
    args, out, _keep = _marshal_topk_select(scores, kv_act_seqs, batch=batch, s1=s1, topk=topk, out=out,
                                            stream=stream)
    st = _lib.sfa_topk_select(*args)
    if st != 0:
        raise SfaError(st, "sfa_topk_select")
    return out


def prepare_indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs, *, batch, s1, topk=1,
                           scores=None, stream=None) -> PreparedCall:
    """sfa_indexer_scores bound to these tensors (a PreparedCall returning the scores)."""
    args, scores, keep = _marshal_indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs,
                                                 batch=batch, s1=s1, topk=topk, scores=scores, stream=stream)
    return PreparedCall([(_lib.sfa_indexer_scores, args, "sfa_indexer_scores")], scores, keep)


def prepare_topk_select(scores, kv_act_seqs, *, batch, s1, topk, out=None, stream=None) -> PreparedCall:
    """sfa_topk_select bound to these tensors (a PreparedCall returning topk_indices)."""
    args, out, keep = _marshal_topk_select(scores, kv_act_seqs, batch=batch, s1=s1, topk=topk, out=out,
                                           stream=stream)
    return PreparedCall([(_lib.sfa_topk_select, args, "sfa_topk_select")], out, keep)


def prepare_indexer(q_index, k_index_cache, weights, block_table, kv_act_seqs, *, batch, s1, topk, scores=None,
                    out=None, stream=None) -> PreparedCall:
    """sfa_indexer_scores then sfa_topk_select bound to these tensors: a PreparedCall that queues
    both and returns topk_indices."""
    sc = prepare_indexer_scores(q_index, k_index_cache, weights, block_table, kv_act_seqs, batch=batch, s1=s1,
                                topk=topk, scores=scores, stream=stream)
    sel = prepare_topk_select(sc.out, kv_act_seqs, batch=batch, s1=s1, topk=topk, out=out, stream=stream)
    return PreparedCall(sc._calls + sel._calls, sel.out, (sc, sel))


def indexer_to_device(inp, device="cuda"):
    """Upload a workloads.IndexerInputs instance."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return {
        "q_index": bf16(inp.q_index),
        "k_index": bf16(inp.k_index),
        "weights": torch.from_numpy(np.ascontiguousarray(inp.weights)).to(device),
        "block_table": torch.from_numpy(inp.block_table).to(device),
        "kv_act_seqs": torch.from_numpy(inp.kv_act_seqs).to(device),
    }


def cache_to_device(inp, device="cuda"):
    """Upload a workloads.CacheWriteInputs instance (the cache tensors are fresh copies)."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    rope = inp.key_rope.shape[1] > 0  # zero-width rope arrays: 512-wide rows
    return {
        "new_nope": bf16(inp.new_nope),
        "new_rope": bf16(inp.new_rope) if rope else None,
        "positions": torch.from_numpy(inp.positions).to(device),
        "block_table": torch.from_numpy(inp.block_table).to(device),
        "key_nope": bf16(inp.key_nope) if inp.kv_dtype == "bf16" else torch.from_numpy(inp.key_nope).to(device),
        "key_rope": bf16(inp.key_rope) if rope else None,
        "k_nope_scales": None if inp.k_nope_scales is None else torch.from_numpy(inp.k_nope_scales).to(device),
    }


def prepare_cache_write(new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales=None, *,
                        batch, s1, stream=None) -> PreparedCall:
    """sfa_cache_write bound to these tensors (a PreparedCall returning key_nope)."""
    args, keep = _marshal_cache_write(new_nope, new_rope, positions, block_table, key_nope, key_rope, k_nope_scales,
                                      batch=batch, s1=s1, stream=stream)
    return PreparedCall([(_lib.sfa_cache_write, args, "sfa_cache_write")], key_nope, keep)


def run_cache_write(inp, d):
    """sfa_cache_write on an uploaded CacheWriteInputs instance (writes d's cache tensors)."""
    return cache_write(d["new_nope"], d["new_rope"], d["positions"], d["block_table"], d["key_nope"], d["key_rope"],
                       d["k_nope_scales"], batch=inp.batch, s1=inp.s1)


def run_indexer(inp, dev_tensors=None):
    """Scores and top-k of an uploaded IndexerInputs instance: (scores, topk_indices)."""
    d = dev_tensors if dev_tensors is not None else indexer_to_device(inp)
    sc = indexer_scores(d["q_index"], d["k_index"], d["weights"], d["block_table"], d["kv_act_seqs"],
                        batch=inp.batch, s1=inp.s1, topk=inp.topk)
    idx = topk_select(sc, d["kv_act_seqs"], batch=inp.batch, s1=inp.s1, topk=inp.topk)
    return sc, idx


# ---- compressor -------------------------------------------------------------------------

COMPRESS_CHANNELS = KV_LORA_RANK + ROPE_DIM


def _marshal_compress(kv, score, ape, gamma, eps, rope_cos, rope_sin, start_pos, kv_state, score_state,
                      block_table_cmp, key_nope, key_rope, *, batch, s1, rotate=False, stream=None):
    dev = kv.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t_tokens = batch * s1
    c = kv.shape[1]
    if c not in (COMPRESS_CHANNELS, KV_LORA_RANK, 128):
        raise ValueError("kv must have 576, 512 or 128 channels")
    ratio = ape.shape[0]
    n_pos = rope_cos.shape[0]
    rows = key_nope.shape[0]
    f32 = (torch.float32,)
    _check(kv, "kv", f32, (t_tokens, c), dev)
    _check(score, "score", f32, (t_tokens, c), dev)
    _check(ape, "ape", f32, (ratio, c), dev)
    _check(gamma, "gamma", f32, (c,), dev)
    _check(rope_cos, "rope_cos", f32, (n_pos, ROPE_DIM // 2), dev)
    _check(rope_sin, "rope_sin", f32, (n_pos, ROPE_DIM // 2), dev)
    _check(start_pos, "start_pos", (torch.int32,), (batch,), dev)
    _check(kv_state, "kv_state", f32, (batch, ratio, c), dev)
    _check(score_state, "score_state", f32, (batch, ratio, c), dev)
    _check(block_table_cmp, "block_table_cmp", (torch.int32,), None, dev)
    if block_table_cmp.dim() != 2 or block_table_cmp.shape[0] != batch:
        raise ValueError("block_table_cmp must be (batch, max_blocks)")
    if c == COMPRESS_CHANNELS:
        _check(key_nope, "key_nope", (torch.bfloat16,), (rows, KV_LORA_RANK), dev)
        _check(key_rope, "key_rope", (torch.bfloat16,), (rows, ROPE_DIM), dev)
    else:
        _check(key_nope, "key_nope", (torch.bfloat16,), (rows, c), dev)
        key_rope = None
    dims = SfaCompressDims(batch=batch, s1=s1, channels=c, ratio=ratio, rope_positions=n_pos,
                           max_blocks=block_table_cmp.shape[1], block_size=BLOCK_SIZE, rotate=int(bool(rotate)),
                           num_cache_rows=rows)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (ctypes.byref(dims), _ptr(kv), _ptr(score), _ptr(ape), _ptr(gamma), ctypes.c_float(eps), _ptr(rope_cos),
            _ptr(rope_sin), _ptr(start_pos), _ptr(kv_state), _ptr(score_state), _ptr(block_table_cmp),
            _ptr(key_nope), _ptr(key_rope), ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, kv, score, ape, gamma, rope_cos, rope_sin, start_pos, kv_state, score_state, block_table_cmp,
            key_nope, key_rope, stream)
    return args, keep


def compress(kv, score, ape, gamma, eps, rope_cos, rope_sin, start_pos, kv_state, score_state, block_table_cmp,
             key_nope, key_rope, *, batch, s1, rotate=False, stream=None):
    """sfa_compress: refreshes kv_state / score_state in place and writes the compressed entries
    of the windows the new tokens close into key_nope / key_rope (576 channels) or key_nope alone
    (512 or 128 channels; key_rope may be None). Returns key_nope."""
    args, _keep = _marshal_compress(kv, score, ape, gamma, eps, rope_cos, rope_sin, start_pos, kv_state, score_state,
                                    block_table_cmp, key_nope, key_rope, batch=batch, s1=s1, rotate=rotate,
                                    stream=stream)
    st = _lib.sfa_compress(*args)
    if st != 0:
        raise SfaError(st, "sfa_compress")
    return key_nope


def compress_to_device(inp, device="cuda"):
    """Upload a workloads.CompressInputs instance (state and pool tensors are fresh copies)."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {"kv": t(inp.kv), "score": t(inp.score), "ape": t(inp.ape), "gamma": t(inp.gamma),
            "rope_cos": t(inp.rope_cos), "rope_sin": t(inp.rope_sin), "start_pos": t(inp.start_pos),
            "kv_state": t(inp.kv_state), "score_state": t(inp.score_state),
            "block_table_cmp": t(inp.block_table_cmp), "key_nope": bf16(inp.key_nope),
            "key_rope": None if inp.key_rope is None else bf16(inp.key_rope)}


def _compress_tensors(d):
    return (d["kv"], d["score"], d["ape"], d["gamma"])


def run_compress(inp, d):
    """sfa_compress on an uploaded CompressInputs instance (updates d's state and pool tensors)."""
    return compress(*_compress_tensors(d), inp.eps, d["rope_cos"], d["rope_sin"], d["start_pos"], d["kv_state"],
                    d["score_state"], d["block_table_cmp"], d["key_nope"], d["key_rope"], batch=inp.batch, s1=inp.s1,
                    rotate=inp.rotate)


def prepare_compress(inp, d, stream=None) -> PreparedCall:
    """sfa_compress bound to an uploaded CompressInputs instance (a PreparedCall returning key_nope)."""
    args, keep = _marshal_compress(*_compress_tensors(d), inp.eps, d["rope_cos"], d["rope_sin"], d["start_pos"],
                                   d["kv_state"], d["score_state"], d["block_table_cmp"], d["key_nope"],
                                   d["key_rope"], batch=inp.batch, s1=inp.s1, rotate=inp.rotate, stream=stream)
    return PreparedCall([(_lib.sfa_compress, args, "sfa_compress")], d["key_nope"], keep)


# ---- MLA prolog -------------------------------------------------------------------------

def prolog_workspace_size(dims: SfaPrologDims) -> int:
    out = ctypes.c_size_t(0)
    st = _lib.sfa_mla_prolog_workspace_size(ctypes.byref(dims), ctypes.byref(out))
    if st != 0:
        raise SfaError(st, "sfa_mla_prolog_workspace_size")
    return out.value


def _marshal_prolog(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin, eps, *,
                    out=None, workspace=None, stream=None, cq_out=None):
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t, hidden = x.shape
    q = w_dq.shape[0]
    n_q, lat, dn = w_uk.shape
    n_pos = rope_cos.shape[0]
    b16 = (torch.bfloat16,)
    _check(x, "x", b16, (t, hidden), dev)
    _check(w_dq, "w_dq", b16, (q, hidden), dev)
    _check(gamma_cq, "gamma_cq", b16, (q,), dev)
    _check(w_uq_qr, "w_uq_qr", b16, (n_q * (dn + ROPE_DIM), q), dev)
    _check(w_uk, "w_uk", b16, (n_q, KV_LORA_RANK, dn), dev)
    _check(w_dkv_kr, "w_dkv_kr", b16, (KV_LORA_RANK + ROPE_DIM, hidden), dev)
    _check(gamma_ckv, "gamma_ckv", b16, (KV_LORA_RANK,), dev)
    _check(positions, "positions", (torch.int32,), (t,), dev)
    _check(rope_cos, "rope_cos", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    _check(rope_sin, "rope_sin", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    dims = SfaPrologDims(t, hidden, q, n_q, dn, n_pos, float(eps))
    shapes = ((t * n_q, KV_LORA_RANK), (t * n_q, ROPE_DIM), (t, KV_LORA_RANK), (t, ROPE_DIM))
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in shapes)
    for o, sh, name in zip(out, shapes, ("q_nope", "q_rope", "kv_nope", "kv_rope")):
        _check(o, name, b16, sh, dev)
    need = prolog_workspace_size(dims)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need:
        workspace = get_workspace(dev, need, stream)
    if workspace is not None:
        _check(workspace, "workspace", (torch.uint8,), None, dev)
    if cq_out is not None:
        _check(cq_out, "cq_out", b16, (t, q), dev)
    args = (ctypes.byref(dims), _ptr(x), _ptr(w_dq), _ptr(gamma_cq), _ptr(w_uq_qr), _ptr(w_uk), _ptr(w_dkv_kr),
            _ptr(gamma_ckv), _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), *[_ptr(o) for o in out], _ptr(cq_out),
            _ptr(workspace) if need else None, ctypes.c_size_t(workspace.numel() if (need and workspace is not None)
                                                            else 0),
            ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin, out,
            cq_out, workspace, stream)
    return args, out, keep


def mla_prolog(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin, eps, *,
               out=None, workspace=None, stream=None, cq_out=None):
    """sfa_mla_prolog: returns (q_nope (T*n_q, 512), q_rope (T*n_q, 64), kv_nope (T, 512),
    kv_rope (T, 64)), all bf16; cq_out (T, Q) bf16, when given, receives cq rounded to bf16."""
    args, out, _keep = _marshal_prolog(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos,
                                       rope_sin, eps, out=out, workspace=workspace, stream=stream, cq_out=cq_out)
    st = _lib.sfa_mla_prolog(*args)
    if st != 0:
        raise SfaError(st, "sfa_mla_prolog")
    return out


def prepare_mla_prolog(*tensors, **kw) -> PreparedCall:
    """sfa_mla_prolog bound to these tensors (a PreparedCall returning the output tuple)."""
    args, out, keep = _marshal_prolog(*tensors, **kw)
    return PreparedCall([(_lib.sfa_mla_prolog, args, "sfa_mla_prolog")], out, keep)


def prolog_to_device(inp, device="cuda"):
    """Upload a workloads.PrologInputs instance."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return {
        "x": bf16(inp.x), "w_dq": bf16(inp.w_dq), "gamma_cq": bf16(inp.gamma_cq), "w_uq_qr": bf16(inp.w_uq_qr),
        "w_uk": bf16(inp.w_uk), "w_dkv_kr": bf16(inp.w_dkv_kr), "gamma_ckv": bf16(inp.gamma_ckv),
        "positions": torch.from_numpy(inp.positions).to(device),
        "rope_cos": torch.from_numpy(inp.rope_cos).to(device), "rope_sin": torch.from_numpy(inp.rope_sin).to(device),
    }


def _prolog_args(inp, d):
    return (d["x"], d["w_dq"], d["gamma_cq"], d["w_uq_qr"], d["w_uk"], d["w_dkv_kr"], d["gamma_ckv"], d["positions"],
            d["rope_cos"], d["rope_sin"], inp.eps)


def run_prolog(inp, d=None, *, out=None, cq_out=None):
    """sfa_mla_prolog on an uploaded PrologInputs instance."""
    d = d if d is not None else prolog_to_device(inp)
    return mla_prolog(*_prolog_args(inp, d), out=out, cq_out=cq_out)


def prepare_prolog_run(inp, d, *, out=None) -> PreparedCall:
    return prepare_mla_prolog(*_prolog_args(inp, d), out=out)


# ---- MLA prolog, V4 form ----------------------------------------------------------------

def prolog_v4_workspace_size(dims: SfaPrologV4Dims) -> int:
    out = ctypes.c_size_t(0)
    st = _lib.sfa_mla_prolog_v4_workspace_size(ctypes.byref(dims), ctypes.byref(out))
    if st != 0:
        raise SfaError(st, "sfa_mla_prolog_v4_workspace_size")
    return out.value


def _marshal_prolog_v4(x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin, eps, *,
                       out=None, workspace=None, stream=None, cq_out=None, kv_ready=None):
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t, hidden = x.shape
    q = w_dq.shape[0]
    n_q = w_uq.shape[0] // KV_LORA_RANK
    n_pos = rope_cos.shape[0]
    b16 = (torch.bfloat16,)
    _check(x, "x", b16, (t, hidden), dev)
    _check(w_dq, "w_dq", b16, (q, hidden), dev)
    _check(gamma_cq, "gamma_cq", b16, (q,), dev)
    _check(w_uq, "w_uq", b16, (n_q * KV_LORA_RANK, q), dev)
    _check(w_dkv, "w_dkv", b16, (KV_LORA_RANK, hidden), dev)
    _check(gamma_ckv, "gamma_ckv", b16, (KV_LORA_RANK,), dev)
    _check(positions, "positions", (torch.int32,), (t,), dev)
    _check(rope_cos, "rope_cos", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    _check(rope_sin, "rope_sin", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    dims = SfaPrologV4Dims(t, hidden, q, n_q, KV_LORA_RANK, n_pos, float(eps))
    shapes = ((t * n_q, KV_LORA_RANK), (t, KV_LORA_RANK))
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in shapes)
    for o, sh, name in zip(out, shapes, ("q", "kv")):
        _check(o, name, b16, sh, dev)
    need = prolog_v4_workspace_size(dims)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need:
        workspace = get_workspace(dev, need, stream)
    if workspace is not None:
        _check(workspace, "workspace", (torch.uint8,), None, dev)
    if cq_out is not None:
        _check(cq_out, "cq_out", b16, (t, q), dev)
    args = (ctypes.byref(dims), _ptr(x), _ptr(w_dq), _ptr(gamma_cq), _ptr(w_uq), _ptr(w_dkv), _ptr(gamma_ckv),
            _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), *[_ptr(o) for o in out], _ptr(cq_out),
            _ptr(workspace), ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
            None if kv_ready is None else ctypes.c_void_p(_event_handle(kv_ready, stream)),
            ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin, out, cq_out, workspace,
            kv_ready, stream)
    return args, out, keep


def mla_prolog_v4(x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin, eps, *, out=None,
                  workspace=None, stream=None, cq_out=None):
    """sfa_mla_prolog_v4: returns (q (T*n_q, 512), kv (T, 512)) bf16, each with its rotary part in
    its last 64 channels; cq_out (T, Q) bf16, when given, receives cq rounded to bf16."""
    args, out, _keep = _marshal_prolog_v4(x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin,
                                          eps, out=out, workspace=workspace, stream=stream, cq_out=cq_out)
    st = _lib.sfa_mla_prolog_v4(*args)
    if st != 0:
        raise SfaError(st, "sfa_mla_prolog_v4")
    return out


def prolog_v4_to_device(inp, device="cuda"):
    """Upload a workloads.PrologV4Inputs instance."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return {
        "x": bf16(inp.x), "w_dq": bf16(inp.w_dq), "gamma_cq": bf16(inp.gamma_cq), "w_uq": bf16(inp.w_uq),
        "w_dkv": bf16(inp.w_dkv), "gamma_ckv": bf16(inp.gamma_ckv),
        "positions": torch.from_numpy(inp.positions).to(device),
        "rope_cos": torch.from_numpy(inp.rope_cos).to(device), "rope_sin": torch.from_numpy(inp.rope_sin).to(device),
    }


def _prolog_v4_args(inp, d):
    return (d["x"], d["w_dq"], d["gamma_cq"], d["w_uq"], d["w_dkv"], d["gamma_ckv"], d["positions"], d["rope_cos"],
            d["rope_sin"], inp.eps)


def run_prolog_v4(inp, d=None, *, out=None, cq_out=None):
    """sfa_mla_prolog_v4 on an uploaded PrologV4Inputs instance."""
    d = d if d is not None else prolog_v4_to_device(inp)
    return mla_prolog_v4(*_prolog_v4_args(inp, d), out=out, cq_out=cq_out)


def _event_handle(ev, stream) -> int:
    """The hipEvent_t of a torch.cuda.Event (recorded once on `stream` first if torch has not
    created it yet)."""
    if not ev.cuda_event:
        ev.record(stream)
    return ev.cuda_event


def prepare_prolog_v4_run(inp, d, *, out=None, cq_out=None, kv_ready=None) -> PreparedCall:
    """kv_ready: a torch.cuda.Event the call records once kv and cq_out are complete, or None."""
    args, out, keep = _marshal_prolog_v4(*_prolog_v4_args(inp, d), out=out, cq_out=cq_out, kv_ready=kv_ready)
    return PreparedCall([(_lib.sfa_mla_prolog_v4, args, "sfa_mla_prolog_v4")], out, keep)


# ---- indexer prolog ---------------------------------------------------------------------

def indexer_prolog_workspace_size(dims: SfaIndexerPrologDims) -> int:
    out = ctypes.c_size_t(0)
    st = _lib.sfa_indexer_prolog_workspace_size(ctypes.byref(dims), ctypes.byref(out))
    if st != 0:
        raise SfaError(st, "sfa_indexer_prolog_workspace_size")
    return out.value


def _marshal_indexer_prolog(x, qr, w_idx_qb, w_idx_k, ln_gamma_k, ln_beta_k, w_idx_proj, positions, rope_cos,
                            rope_sin, eps, *, rotate=True, out=None, workspace=None, stream=None):
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    t, hidden = x.shape
    q = qr.shape[1]
    d = w_idx_k.shape[0]
    nh = w_idx_proj.shape[0]
    n_pos = rope_cos.shape[0]
    b16 = (torch.bfloat16,)
    _check(x, "x", b16, (t, hidden), dev)
    _check(qr, "qr", b16, (t, q), dev)
    _check(w_idx_qb, "w_idx_qb", b16, (nh * d, q), dev)
    _check(w_idx_k, "w_idx_k", b16, (d, hidden), dev)
    _check(ln_gamma_k, "ln_gamma_k", b16, (d,), dev)
    _check(ln_beta_k, "ln_beta_k", b16, (d,), dev)
    _check(w_idx_proj, "w_idx_proj", b16, (nh, hidden), dev)
    _check(positions, "positions", (torch.int32,), (t,), dev)
    _check(rope_cos, "rope_cos", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    _check(rope_sin, "rope_sin", (torch.float32,), (n_pos, ROPE_DIM // 2), dev)
    dims = SfaIndexerPrologDims(t, hidden, q, nh, d, n_pos, int(bool(rotate)), float(eps))
    if out is None:
        out = (torch.empty((t * nh, d), dtype=torch.bfloat16, device=dev),
               torch.empty((t, d), dtype=torch.bfloat16, device=dev),
               torch.empty((t, nh), dtype=torch.float32, device=dev))
    _check(out[0], "q_index", b16, (t * nh, d), dev)
    _check(out[1], "k_index", b16, (t, d), dev)
    _check(out[2], "weights", (torch.float32,), (t, nh), dev)
    need = indexer_prolog_workspace_size(dims)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need:
        workspace = get_workspace(dev, need, stream)
    if workspace is not None:
        _check(workspace, "workspace", (torch.uint8,), None, dev)
    args = (ctypes.byref(dims), _ptr(x), _ptr(qr), _ptr(w_idx_qb), _ptr(w_idx_k), _ptr(ln_gamma_k), _ptr(ln_beta_k),
            _ptr(w_idx_proj), _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), *[_ptr(o) for o in out],
            _ptr(workspace) if need else None,
            ctypes.c_size_t(workspace.numel() if (need and workspace is not None) else 0),
            ctypes.c_void_p(stream.cuda_stream))
    keep = (dims, x, qr, w_idx_qb, w_idx_k, ln_gamma_k, ln_beta_k, w_idx_proj, positions, rope_cos, rope_sin, out,
            workspace, stream)
    return args, out, keep


def indexer_prolog(*tensors, **kw):
    """sfa_indexer_prolog: returns (q_index (T*64, 128) bf16, k_index (T, 128) bf16,
    weights (T, 64) fp32)."""
    args, out, _keep = _marshal_indexer_prolog(*tensors, **kw)
    st = _lib.sfa_indexer_prolog(*args)
    if st != 0:
        raise SfaError(st, "sfa_indexer_prolog")
    return out


def prepare_indexer_prolog(*tensors, **kw) -> PreparedCall:
    args, out, keep = _marshal_indexer_prolog(*tensors, **kw)
    return PreparedCall([(_lib.sfa_indexer_prolog, args, "sfa_indexer_prolog")], out, keep)


def indexer_prolog_to_device(inp, device="cuda"):
    """Upload a workloads.IndexerPrologInputs instance."""
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return {k: bf16(getattr(inp, k)) for k in ("x", "qr", "w_idx_qb", "w_idx_k", "ln_gamma_k", "ln_beta_k",
                                                 "w_idx_proj")} | {
        "positions": torch.from_numpy(inp.positions).to(device),
        "rope_cos": torch.from_numpy(inp.rope_cos).to(device), "rope_sin": torch.from_numpy(inp.rope_sin).to(device)}


def _indexer_prolog_args(inp, d):
    return (d["x"], d["qr"], d["w_idx_qb"], d["w_idx_k"], d["ln_gamma_k"], d["ln_beta_k"], d["w_idx_proj"],
            d["positions"], d["rope_cos"], d["rope_sin"], inp.eps)


def run_indexer_prolog(inp, d=None, *, out=None):
    d = d if d is not None else indexer_prolog_to_device(inp)
    return indexer_prolog(*_indexer_prolog_args(inp, d), rotate=inp.rotate, out=out)


def prepare_indexer_prolog_run(inp, d, *, out=None, stream=None) -> PreparedCall:
    return prepare_indexer_prolog(*_indexer_prolog_args(inp, d), rotate=inp.rotate, out=out, stream=stream)
