"""Python binding for libpkv: paged KV cache append and shared-prefix decode attention on gfx950.

Argument marshalling only.  Every step of the path (block-table gather,
split-K attention, cascade pass, partial merge, append / copy-on-write, block
pool and cascade planning) runs in the native library ``libpkv.so`` built from
``csrc/``; PyTorch only provides device memory and streams.  Importing this
package fails loudly if the library has not been built
(``python paged_kv_cache_21_amd/build.py``); there is no fallback.

The names mirror the C ABI in ``include/pkv.h``.
"""

import ctypes
import os

import numpy as np

# torch ships its own HIP runtime.  Importing it first makes libpkv.so bind to
# that same, already loaded runtime (same soname) instead of pulling a second
# HIP/HSA runtime into the process, which would then see no device.
import torch  # noqa: F401

__all__ = [
    "PkvError", "PkvInvalid", "PkvOOM", "PkvNotFound", "PkvUnsupported", "PkvWorkspaceError", "PkvHipError",
    "kv_append", "paged_decode_attn", "decode_workspace_bytes", "BlockPool", "CascadePlan",
    "ExtendPlan", "paged_extend_attn", "extend_workspace_bytes", "kv_append_fp8", "paged_decode_attn_fp8",
    "paged_decode_attn_append",
    "timing_enable", "timing_reset", "timing_read", "stream_read", "KERNELS", "lib", "LIB_PATH", "version",
    "STATUS_LEN_CLAMPED", "STATUS_BAD_BLOCK", "paged_decode_attn_noalloc", "NOALLOC_SCRATCH_BYTES",
]

# The library built in-tree next to this file (paged_kv_cache_21_amd/build.py); nothing else is loaded.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_OOM, PKV_ERR_NOT_FOUND, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP, PKV_ERR_WORKSPACE = (
    0, -1, -2, -3, -4, -5, -6)
PKV_F16, PKV_BF16 = 0, 1
STATUS_LEN_CLAMPED, STATUS_BAD_BLOCK = 1, 2  # flags of the decode calls' optional status word
NOALLOC_SCRATCH_BYTES = 64 << 20  # PKV_NOALLOC_SCRATCH_BYTES
PKV_EVICT_LRU, PKV_EVICT_RSBCM = 0, 1
KERNELS = {"append": 0, "decode_split": 1, "merge": 2, "cascade": 3}


class PkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class PkvInvalid(PkvError, ValueError):
    pass


class PkvOOM(PkvError, MemoryError):
    pass


class PkvNotFound(PkvError, KeyError):
    pass


class PkvUnsupported(PkvError, NotImplementedError):
    pass


class PkvWorkspaceError(PkvError, ValueError):
    pass


class PkvHipError(PkvError):
    pass


_ERRORS = {PKV_ERR_INVALID: PkvInvalid, PKV_ERR_OOM: PkvOOM, PKV_ERR_NOT_FOUND: PkvNotFound,
           PKV_ERR_UNSUPPORTED: PkvUnsupported, PKV_ERR_HIP: PkvHipError, PKV_ERR_WORKSPACE: PkvWorkspaceError}

_c = ctypes
_vp, _i32, _i64, _sz, _f32, _f64 = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_size_t, _c.c_float, _c.c_double

_SIGNATURES = {
    "pkv_last_error": (_c.c_char_p, []),
    "pkv_version": (_c.c_char_p, []),
    "pkv_kv_append": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pkv_paged_decode_attn": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32,
                                     _f32, _vp, _vp, _sz, _vp, _vp, _vp]),
    "pkv_paged_decode_attn_append": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _i32, _vp,
                                            _i32, _vp, _vp, _vp, _f32, _vp, _vp, _sz, _vp, _vp, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_decode_attn_noalloc": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _i32, _vp,
                                             _i32, _f32, _vp, _vp, _vp, _vp]),
    "pkv_pool_create": (_vp, [_i32, _i32, _vp]),
    "pkv_pool_destroy": (None, [_vp]),
    "pkv_seq_alloc": (_i32, [_vp, _i64, _i32]),
    "pkv_seq_alloc_prefix": (_i32, [_vp, _i64, _vp, _i32, _i32]),
    "pkv_seq_fork": (_i32, [_vp, _i64, _i64]),
    "pkv_seq_free": (_i32, [_vp, _i64]),
    "pkv_plan_append": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pkv_export_tables": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "pkv_seq_len": (_i32, [_vp, _i64]),
    "pkv_seq_table": (_i32, [_vp, _i64, _vp, _i32]),
    "pkv_refcount": (_i32, [_vp, _i32]),
    "pkv_free_count": (_i32, [_vp]),
    "pkv_num_seqs": (_i32, [_vp]),
    "pkv_free_list": (_i32, [_vp, _vp, _i32]),
    "pkv_radix_create": (_vp, [_vp, _i32]),
    "pkv_radix_destroy": (None, [_vp]),
    "pkv_radix_clear": (_i32, [_vp]),
    "pkv_radix_match": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "pkv_radix_insert": (_i32, [_vp, _vp, _i32, _vp, _i32, _f64, _i32, _vp, _vp]),
    "pkv_radix_lock": (_i32, [_vp, _i64]),
    "pkv_radix_unlock": (_i32, [_vp, _i64]),
    "pkv_radix_set_score": (_i32, [_vp, _i64, _f64]),
    "pkv_radix_evict": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp]),
    "pkv_radix_admit": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "pkv_radix_finish": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "pkv_radix_num_nodes": (_i32, [_vp]),
    "pkv_radix_cached_blocks": (_i32, [_vp]),
    "pkv_radix_evictable_blocks": (_i32, [_vp]),
    "pkv_radix_node_ids": (_i32, [_vp, _vp, _i32]),
    "pkv_radix_node_info": (_i32, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32]),
    "pkv_plan_build": (_vp, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_plan_destroy": (None, [_vp]),
    "pkv_plan_device_bytes": (_sz, [_vp]),
    "pkv_plan_upload": (_i32, [_vp, _vp, _sz, _vp]),
    "pkv_plan_num_nodes": (_i32, [_vp]),
    "pkv_plan_node": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp]),
    "pkv_plan_row": (_i32, [_vp, _i32, _vp, _vp]),
    "pkv_plan_node_pieces": (_i32, [_vp, _i32]),
    "pkv_plan_build_extend": (_vp, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_extend_workspace_bytes": (_sz, [_vp, _i32]),
    "pkv_plan_num_query_rows": (_i32, [_vp]),
    "pkv_plan_rows_per_item": (_i32, [_vp]),
    "pkv_plan_image": (_i64, [_vp, _vp, _i64, _vp]),
    "pkv_plan_item_records": (_i64, [_vp, _vp]),
    "pkv_paged_extend_attn": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _i32, _f32, _vp, _vp, _sz,
                                     _vp, _vp]),
    "pkv_paged_extend_attn_fp8": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _f32,
                                         _vp, _vp, _sz, _vp, _vp]),
    "pkv_kv_append_fp8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                                 _vp, _i32, _vp]),
    "pkv_paged_decode_attn_fp8": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _vp,
                                         _i32, _vp, _i32, _f32, _vp, _vp, _sz, _vp, _vp, _vp]),
    "pkv_stream_read": (_i32, [_vp, _i64, _vp, _i32, _vp]),
    "pkv_pool_set_host_slots": (_i32, [_vp, _i32, _vp]),
    "pkv_seq_swap_out": (_i32, [_vp, _i64, _vp, _vp, _i32, _vp]),
    "pkv_seq_swap_in": (_i32, [_vp, _i64, _vp, _vp, _i32, _vp]),
    "pkv_seq_is_swapped": (_i32, [_vp, _i64]),
    "pkv_seq_placement": (_i32, [_vp, _i64, _vp, _vp, _i32]),
    "pkv_host_free_count": (_i32, [_vp]),
    "pkv_host_free_list": (_i32, [_vp, _vp, _i32]),
    "pkv_copy_blocks": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _vp]),
    "pkv_copy_blocks_memcpy": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i32, _vp]),
    "pkv_timing_enable": (_i32, [_i32]),
    "pkv_timing_reset": (_i32, []),
    "pkv_timing_read": (_i32, [_i32, _vp, _vp]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_21_amd/build.py` "
                          "(hipcc, gfx950). There is no fallback implementation.")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


_lib = _load()


def lib():
    """The loaded ctypes handle of libpkv.so."""
    return _lib


def version():
    return _lib.pkv_version().decode()


def _check(status):
    if status != PKV_OK:
        msg = _lib.pkv_last_error().decode(errors="replace")
        raise _ERRORS.get(status, PkvError)(status, msg)


def _ptr(x):
    """Device / host address of a torch tensor or numpy array (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _dtype_code(t, dtype):
    import torch

    if dtype is not None:
        return {"f16": PKV_F16, "bf16": PKV_BF16, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}[dtype]
    if t.dtype == torch.float16:
        return PKV_F16
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise ValueError("pass dtype='f16'|'bf16' for bit-pattern (int16) tensors")


def _stream(stream, like):
    import torch

    if stream is None:
        return torch.cuda.current_stream(like.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require(cond, msg):
    if not cond:
        raise PkvInvalid(PKV_ERR_INVALID, msg)


# ---------------------------------------------------------------------------
# device operations


def kv_append(k_pages, v_pages, k_new, v_new, slot_mapping, cow_src=None, cow_dst=None, cow_rows=None,
              dtype=None, stream=None):
    """Copy-on-write the listed block prefixes, then write k_new[i]/v_new[i] to slot slot_mapping[i].

    k_pages, v_pages: [num_blocks, block_size, Hkv, d] device tensors (fp16/bf16, or int16 bits with
    ``dtype``); k_new, v_new: [N, Hkv, d]; slot_mapping int64 [N]; cow_* int32 [n_cow] (device).
    """
    _require(k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "k_pages/v_pages must be equal 4-D tensors")
    _require(k_pages.is_contiguous() and v_pages.is_contiguous(), "pages must be contiguous")
    nblk, bs, hkv, d = k_pages.shape
    n = int(slot_mapping.numel())
    _require(tuple(k_new.shape) == (n, hkv, d) and tuple(v_new.shape) == (n, hkv, d), "k_new/v_new must be [N, Hkv, d]")
    _require(k_new.is_contiguous() and v_new.is_contiguous() and slot_mapping.is_contiguous(), "inputs must be contiguous")
    import torch

    _require(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    n_cow = 0 if cow_src is None else int(cow_src.numel())
    if n_cow:
        _require(cow_src.dtype == cow_dst.dtype == cow_rows.dtype == torch.int32, "cow arrays must be int32")
        _require(cow_dst.numel() == n_cow and cow_rows.numel() == n_cow, "cow arrays must have equal length")
    _check(_lib.pkv_kv_append(_ptr(k_pages), _ptr(v_pages), nblk, bs, hkv, d, _dtype_code(k_pages, dtype),
                              _ptr(k_new), _ptr(v_new), n, _ptr(slot_mapping),
                              _ptr(cow_src) if n_cow else None, _ptr(cow_dst) if n_cow else None,
                              _ptr(cow_rows) if n_cow else None, n_cow, _stream(stream, k_pages)))


def kv_append_fp8(k_pages, v_pages, k_scales, v_scales, k_new, v_new, slot_mapping, cow_src=None, cow_dst=None,
                  cow_rows=None, src_dtype=None, stream=None):
    """FP8 pages: copy-on-write the listed block prefixes (codes and scales), then quantize
    k_new[i] / v_new[i] into slot slot_mapping[i].

    k_pages, v_pages: uint8 [num_blocks, block_size, Hkv, d]; k_scales, v_scales: float32
    [num_blocks, Hkv, block_size]; k_new, v_new: [N, Hkv, d] fp16/bf16 (or int16 bits with
    ``src_dtype``).
    """
    import torch

    _require(k_pages.dim() == 4 and v_pages.shape == k_pages.shape and k_pages.dtype == torch.uint8,
             "k_pages/v_pages must be equal uint8 [num_blocks, block_size, Hkv, d] tensors")
    nblk, bs, hkv, d = k_pages.shape
    _require(tuple(k_scales.shape) == (nblk, hkv, bs) and tuple(v_scales.shape) == (nblk, hkv, bs) and
             k_scales.dtype == v_scales.dtype == torch.float32, "scales must be float32 [num_blocks, Hkv, block_size]")
    n = int(slot_mapping.numel())
    _require(tuple(k_new.shape) == (n, hkv, d) and tuple(v_new.shape) == (n, hkv, d), "k_new/v_new must be [N, Hkv, d]")
    _require(all(t.is_contiguous() for t in (k_pages, v_pages, k_scales, v_scales, k_new, v_new, slot_mapping)),
             "inputs must be contiguous")
    _require(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    n_cow = 0 if cow_src is None else int(cow_src.numel())
    _check(_lib.pkv_kv_append_fp8(_ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), nblk, bs, hkv, d,
                                  _dtype_code(k_new, src_dtype), _ptr(k_new), _ptr(v_new), n, _ptr(slot_mapping),
                                  _ptr(cow_src) if n_cow else None, _ptr(cow_dst) if n_cow else None,
                                  _ptr(cow_rows) if n_cow else None, n_cow, _stream(stream, k_pages)))


def paged_decode_attn_fp8(q, k_pages, v_pages, k_scales, v_scales, block_tables, seq_lens, max_seq_len, scale=None,
                          plan=None, workspace=None, out=None, q_dtype=None, stream=None, status=None):
    """Decode attention over FP8 pages (codes x per-row scales); q [B, Hq, d] fp16/bf16, fp32 output.
    ``plan``: an uploaded CascadePlan of the same tables (shared blocks through the matrix-core pass).
    ``status``: as for paged_decode_attn."""
    import torch

    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape and k_pages.dtype == torch.uint8,
             "q [B, Hq, d]; uint8 pages [num_blocks, block_size, Hkv, d]")
    B, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    _require(tuple(k_scales.shape) == (nblk, hkv, bs) and tuple(v_scales.shape) == (nblk, hkv, bs) and
             k_scales.dtype == v_scales.dtype == torch.float32, "scales must be float32 [num_blocks, Hkv, block_size]")
    _require(all(t.is_contiguous() for t in (q, k_pages, v_pages, k_scales, v_scales, block_tables, seq_lens)),
             "inputs must be contiguous")
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables and lengths must be int32")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == B and seq_lens.numel() == B, "bad table shape")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    need = decode_workspace_bytes(B, hq, hkv, d, int(max_seq_len), plan)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, hq, d), "bad out tensor")
    _check(_lib.pkv_paged_decode_attn_fp8(_ptr(q), B, hq, hkv, d, _dtype_code(q, q_dtype), _ptr(k_pages),
                                          _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), nblk, bs,
                                          _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens),
                                          int(max_seq_len), float(scale), plan._handle if plan is not None else None,
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _ptr(out),
                                          _status_ptr(status), _stream(stream, q)))
    return out


def _status_ptr(status):
    """Device address of an optional int32 status word (a one-element int32 device tensor)."""
    if status is None:
        return None
    import torch

    _require(status.dtype == torch.int32 and status.numel() >= 1 and status.is_cuda, "status: int32 device tensor")
    return status.data_ptr()


def decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, plan=None):
    n = _lib.pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                        plan._handle if plan is not None else None)
    if n == 0 and batch > 0:
        msg = _lib.pkv_last_error().decode()
        if msg:
            raise PkvInvalid(PKV_ERR_INVALID, msg)
    return int(n)


def paged_decode_attn(q, k_pages, v_pages, block_tables, seq_lens, max_seq_len, scale=None, plan=None,
                      workspace=None, out=None, dtype=None, stream=None, status=None):
    """o[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the row's seq_lens[b] tokens (fp32 output).

    q: [B, Hq, d]; pages [num_blocks, 16, Hkv, d]; block_tables int32 [B, max_blocks];
    seq_lens int32 [B] (all device tensors).  ``plan``: an uploaded CascadePlan or None.
    ``workspace``: a device tensor of at least decode_workspace_bytes(...) bytes (allocated if None).
    ``status``: optional one-element int32 device tensor; the call or-s STATUS_LEN_CLAMPED /
    STATUS_BAD_BLOCK into it for inputs outside the definition's domain (never cleared by the call).
    """
    import torch

    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad q / page ranks")
    _require(q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous(), "inputs must be contiguous")
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables and lengths must be int32")
    _require(block_tables.is_contiguous() and seq_lens.is_contiguous(), "tables and lengths must be contiguous")
    B, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == B and seq_lens.numel() == B, "bad table shape")
    max_blocks = int(block_tables.shape[1])
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    hplan = plan._handle if plan is not None else None
    need = decode_workspace_bytes(B, hq, hkv, d, int(max_seq_len), plan)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, hq, d), "bad out tensor")
    _check(_lib.pkv_paged_decode_attn(_ptr(q), B, hq, hkv, d, _dtype_code(q, dtype), _ptr(k_pages), _ptr(v_pages),
                                      nblk, bs, _ptr(block_tables), max_blocks, _ptr(seq_lens), int(max_seq_len),
                                      float(scale), hplan, _ptr(workspace), ws_bytes, _ptr(out), _status_ptr(status),
                                      _stream(stream, q)))
    return out


def paged_decode_attn_noalloc(q, k_pages, v_pages, block_tables, seq_lens, max_seq_len, out, scale=None, plan=None,
                              dtype=None, stream=None, status=None):
    """paged_decode_attn with the partial results in the library's fixed per-device scratch
    (NOALLOC_SCRATCH_BYTES) instead of a workspace: the call allocates nothing.  ``out``
    (float32 [B, Hq, d]) must be given.  Calls that overlap on one device race."""
    import torch

    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad q / page ranks")
    _require(q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous(), "inputs must be contiguous")
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables and lengths must be int32")
    _require(block_tables.is_contiguous() and seq_lens.is_contiguous(), "tables and lengths must be contiguous")
    B, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == B and seq_lens.numel() == B, "bad table shape")
    _require(out is not None and out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, hq, d),
             "out: float32 [B, Hq, d] contiguous tensor required")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    _check(_lib.pkv_paged_decode_attn_noalloc(_ptr(q), B, hq, hkv, d, _dtype_code(q, dtype), _ptr(k_pages),
                                              _ptr(v_pages), nblk, bs, _ptr(block_tables),
                                              int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                              float(scale), plan._handle if plan is not None else None, _ptr(out),
                                              _status_ptr(status), _stream(stream, q)))
    return out


def paged_decode_attn_append(q, k_pages, v_pages, block_tables, seq_lens, max_seq_len, k_new, v_new, cow_src,
                             scale=None, plan=None, workspace=None, out=None, dtype=None, stream=None, status=None):
    """kv_append of one new token per row followed by paged_decode_attn, in one launch.

    The tables are those after the append; row b's new token (k_new/v_new [B, Hkv, d]) is
    its token seq_lens[b] - 1, and cow_src (int32 [B], -1 for none) names the block its
    last block was copied from on write (BlockPool.plan_append(..., row_sources=True)).  Returns out [B, Hq, d] fp32.
    """
    import torch

    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad q / page ranks")
    _require(q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous(), "inputs must be contiguous")
    _require(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables and lengths must be int32")
    _require(block_tables.is_contiguous() and seq_lens.is_contiguous(), "tables and lengths must be contiguous")
    B, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == B and seq_lens.numel() == B, "bad table shape")
    _require(tuple(k_new.shape) == (B, hkv, d) and tuple(v_new.shape) == (B, hkv, d), "k_new / v_new must be [B, Hkv, d]")
    _require(k_new.dtype == k_pages.dtype and v_new.dtype == k_pages.dtype, "new tokens must have the pages' dtype")
    _require(k_new.is_contiguous() and v_new.is_contiguous(), "new tokens must be contiguous")
    _require(cow_src.dtype == torch.int32 and cow_src.numel() == B and cow_src.is_contiguous(), "cow_src: int32 [B]")
    max_blocks = int(block_tables.shape[1])
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    hplan = plan._handle if plan is not None else None
    need = decode_workspace_bytes(B, hq, hkv, d, int(max_seq_len), plan)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, hq, d), "bad out tensor")
    _check(_lib.pkv_paged_decode_attn_append(_ptr(q), B, hq, hkv, d, _dtype_code(q, dtype), _ptr(k_pages),
                                             _ptr(v_pages), nblk, bs, _ptr(block_tables), max_blocks, _ptr(seq_lens),
                                             int(max_seq_len), _ptr(k_new), _ptr(v_new), _ptr(cow_src), float(scale),
                                             hplan, _ptr(workspace), ws_bytes, _ptr(out), _status_ptr(status),
                                             _stream(stream, q)))
    return out


# ---------------------------------------------------------------------------
# host block pool


class BlockPool:
    """Reference-counted block pool with fork / copy-on-write append / free (runs in libpkv)."""

    def __init__(self, num_blocks, block_size=16, free_order=None, num_host_slots=0, host_order=None):
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            _require(order.shape == (num_blocks,), "free_order must have num_blocks entries")
        self._order = order
        h = _lib.pkv_pool_create(int(num_blocks), int(block_size), _ptr(order))
        if not h:
            raise PkvInvalid(PKV_ERR_INVALID, _lib.pkv_last_error().decode())
        self._handle = h
        self._radix_handles = set()  # prefix caches holding references in this pool
        self._table_buf = np.empty(1024, dtype=np.int32)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.num_host_slots = int(num_host_slots)
        if num_host_slots:
            ho = None if host_order is None else np.ascontiguousarray(host_order, dtype=np.int32)
            _require(ho is None or ho.shape == (num_host_slots,), "host_order must have num_host_slots entries")
            _check(_lib.pkv_pool_set_host_slots(h, int(num_host_slots), _ptr(ho)))

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and _lib is not None:  # at interpreter exit the module globals may already be gone
            # a cache must go before its pool; garbage cycles finalize in any order
            for r in list(self._radix_handles):
                _lib.pkv_radix_destroy(r)
            self._radix_handles.clear()
            _lib.pkv_pool_destroy(h)
            self._handle = None

    def alloc(self, seq, num_tokens):
        _check(_lib.pkv_seq_alloc(self._handle, int(seq), int(num_tokens)))

    def alloc_with_prefix(self, seq, prefix_blocks, num_tokens):
        """New sequence whose table starts with the cached ``prefix_blocks``."""
        pb = np.asarray(prefix_blocks, dtype=np.int32)
        _check(_lib.pkv_seq_alloc_prefix(self._handle, int(seq), _ptr(pb), pb.shape[0], int(num_tokens)))

    def fork(self, parent, child):
        _check(_lib.pkv_seq_fork(self._handle, int(parent), int(child)))

    def free(self, seq):
        _check(_lib.pkv_seq_free(self._handle, int(seq)))

    def plan_append(self, seqs, row_sources=False):
        """Returns (slots int64 [n], cows int32 [n_cow, 3] of (src, dst, rows)); with
        ``row_sources`` also each row's copy-on-write source block (int32 [n], -1: none)."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        slots = np.empty(n, dtype=np.int64)
        src = np.empty(max(n, 1), dtype=np.int32)
        dst = np.empty(max(n, 1), dtype=np.int32)
        rows = np.empty(max(n, 1), dtype=np.int32)
        ncow = np.zeros(1, dtype=np.int32)
        row_src = np.empty(n, dtype=np.int32) if row_sources else None
        _check(_lib.pkv_plan_append(self._handle, _ptr(s), n, _ptr(slots), _ptr(src), _ptr(dst), _ptr(rows),
                                    _ptr(ncow), _ptr(row_src)))
        k = int(ncow[0])
        cows = np.stack([src[:k], dst[:k], rows[:k]], axis=1)
        return (slots, cows, row_src) if row_sources else (slots, cows)

    def export_tables(self, seqs, max_blocks):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        bt = np.empty((s.shape[0], max_blocks), dtype=np.int32)
        lens = np.empty(s.shape[0], dtype=np.int32)
        _check(_lib.pkv_export_tables(self._handle, _ptr(s), s.shape[0], int(max_blocks), _ptr(bt), _ptr(lens)))
        return bt, lens

    def table(self, seq):
        buf = self._table_buf
        n = _lib.pkv_seq_table(self._handle, int(seq), buf.ctypes.data, buf.shape[0])
        if n == -2:
            raise PkvInvalid(PKV_ERR_INVALID, f"sequence {seq} is swapped out")
        if n < 0:
            raise PkvNotFound(PKV_ERR_NOT_FOUND, f"sequence {seq} does not exist")
        if n > buf.shape[0]:
            self._table_buf = buf = np.empty(2 * n, dtype=np.int32)
            _lib.pkv_seq_table(self._handle, int(seq), buf.ctypes.data, buf.shape[0])
        return buf[:n].tolist()

    def length(self, seq):
        return int(_lib.pkv_seq_len(self._handle, int(seq)))

    def refcount(self, block):
        return int(_lib.pkv_refcount(self._handle, int(block)))

    def free_count(self):
        return int(_lib.pkv_free_count(self._handle))

    def num_seqs(self):
        return int(_lib.pkv_num_seqs(self._handle))

    def free_list(self):
        n = self.free_count()
        out = np.empty(max(n, 1), dtype=np.int32)
        _lib.pkv_free_list(self._handle, _ptr(out), n)
        return [int(x) for x in out[:n]]

    def __contains__(self, seq):
        return self.length(seq) >= 0

    # swap space
    def _swap(self, fn, seq):
        n = max(self.length(seq), 0)
        cap = max(-(-n // self.block_size), 1)
        a = np.empty(cap, dtype=np.int32)
        b = np.empty(cap, dtype=np.int32)
        cnt = np.zeros(1, dtype=np.int32)
        _check(fn(self._handle, int(seq), a.ctypes.data, b.ctypes.data, cap, cnt.ctypes.data))
        k = int(cnt[0])
        return list(zip(a[:k].tolist(), b[:k].tolist()))

    def swap_out(self, seq):
        """Plan a swap-out; returns the (device block, host slot) copies to perform."""
        return self._swap(_lib.pkv_seq_swap_out, seq)

    def swap_in(self, seq):
        """Plan a swap-in; returns the (host slot, device block) copies to perform."""
        return self._swap(_lib.pkv_seq_swap_in, seq)

    def is_swapped(self, seq):
        return _lib.pkv_seq_is_swapped(self._handle, int(seq)) == 1

    def placement(self, seq):
        n = max(self.length(seq), 0)
        cap = max(-(-n // self.block_size), 1)
        ids = np.empty(cap, dtype=np.int32)
        host = np.empty(cap, dtype=np.int8)
        k = _lib.pkv_seq_placement(self._handle, int(seq), ids.ctypes.data, host.ctypes.data, cap)
        if k < 0:
            raise PkvNotFound(PKV_ERR_NOT_FOUND, f"sequence {seq} does not exist")
        return [("host" if h else "device", int(i)) for i, h in zip(ids[:k], host[:k])]

    def host_free_count(self):
        return int(_lib.pkv_host_free_count(self._handle))

    def host_free_list(self):
        n = self.host_free_count()
        out = np.empty(max(n, 1), dtype=np.int32)
        _lib.pkv_host_free_list(self._handle, out.ctypes.data, n)
        return out[:n].tolist()


# ---------------------------------------------------------------------------
# prefix cache


class RadixCache:
    """Radix tree of cached token blocks over a BlockPool (runs in libpkv).

    ``policy`` is "lru" (least recently used unlocked leaf first) or "rsbcm"
    (lowest score / (depth + 1) first).  Keep the pool alive while the cache is.
    """

    POLICIES = {"lru": PKV_EVICT_LRU, "rsbcm": PKV_EVICT_RSBCM}

    def __init__(self, pool, policy="lru"):
        _require(policy in self.POLICIES, f"unknown policy {policy!r}")
        h = _lib.pkv_radix_create(pool._handle, self.POLICIES[policy])
        if not h:
            raise PkvInvalid(PKV_ERR_INVALID, _lib.pkv_last_error().decode())
        self._handle = h
        self._pool = pool  # the cache holds references in this pool
        pool._radix_handles.add(h)
        self.policy = policy
        self.block_size = pool.block_size
        self._i32 = np.zeros(2, dtype=np.int32)   # scratch outputs (one call at a time)
        self._i64 = np.zeros(1, dtype=np.int64)
        self._blocks = np.empty(1024, dtype=np.int32)

    def __del__(self):
        h = getattr(self, "_handle", None)
        pool = getattr(self, "_pool", None)
        if h and _lib is not None and pool is not None and h in pool._radix_handles:
            pool._radix_handles.discard(h)
            _lib.pkv_radix_destroy(h)
        self._handle = None

    @staticmethod
    def _tokens(tokens):
        return np.ascontiguousarray(tokens, dtype=np.int32)

    def match_prefix(self, tokens):
        """(matched tokens, their block ids, node id)."""
        t = self._tokens(tokens)
        nb = t.shape[0] // self.block_size
        if nb > self._blocks.shape[0]:
            self._blocks = np.empty(2 * nb, dtype=np.int32)
        i32, i64, blocks = self._i32, self._i64, self._blocks
        _check(_lib.pkv_radix_match(self._handle, t.ctypes.data, t.shape[0], i32.ctypes.data, blocks.ctypes.data,
                                    blocks.shape[0], i64.ctypes.data))
        m = int(i32[0])
        return m, blocks[:m // self.block_size].tolist(), int(i64[0])

    def insert(self, tokens, blocks, score=0.0, depth=0):
        """(node id ending at the last full block, blocks adopted)."""
        t = self._tokens(tokens)
        b = np.asarray(blocks, dtype=np.int32)
        i32, i64 = self._i32, self._i64
        _check(_lib.pkv_radix_insert(self._handle, t.ctypes.data, t.shape[0], b.ctypes.data, b.shape[0],
                                     float(score), int(depth), i64.ctypes.data, i32.ctypes.data))
        return int(i64[0]), int(i32[0])

    @staticmethod
    def _pack(requests):
        if isinstance(requests, tuple) and len(requests) == 2 and isinstance(requests[1], np.ndarray):
            return np.ascontiguousarray(requests[0], dtype=np.int32), np.ascontiguousarray(requests[1], dtype=np.int64)
        lens = np.fromiter((len(t) for t in requests), dtype=np.int64, count=len(requests))
        offsets = np.zeros(len(requests) + 1, dtype=np.int64)
        np.cumsum(lens, out=offsets[1:])
        flat = np.concatenate([np.asarray(t, dtype=np.int32) for t in requests]) if len(requests) else \
            np.zeros(1, dtype=np.int32)
        return np.ascontiguousarray(flat, dtype=np.int32), offsets

    def admit(self, requests, seqs):
        """Admit token runs (a list of token lists, or (flat tokens, offsets)) as sequences
        ``seqs``; returns [(matched tokens, locked node)] for the admitted prefix."""
        flat, offsets = self._pack(requests)
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        matched = np.empty(max(n, 1), dtype=np.int32)
        nodes = np.empty(max(n, 1), dtype=np.int64)
        count = np.zeros(1, dtype=np.int32)
        _check(_lib.pkv_radix_admit(self._handle, flat.ctypes.data, offsets.ctypes.data, n, s.ctypes.data,
                                    matched.ctypes.data, nodes.ctypes.data, count.ctypes.data))
        k = int(count[0])
        return list(zip(matched[:k].tolist(), nodes[:k].tolist()))

    def finish(self, requests, seqs, nodes, scores=None, depths=None):
        """Cache, unlock and free finished sequences (see pkv_radix_finish)."""
        flat, offsets = self._pack(requests)
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        nd = np.ascontiguousarray(nodes, dtype=np.int64)
        sc = None if scores is None else np.ascontiguousarray(scores, dtype=np.float64)
        dp = None if depths is None else np.ascontiguousarray(depths, dtype=np.int32)
        _check(_lib.pkv_radix_finish(self._handle, flat.ctypes.data, offsets.ctypes.data, s.shape[0], s.ctypes.data,
                                     nd.ctypes.data, _ptr(sc), _ptr(dp)))

    def lock(self, node):
        _check(_lib.pkv_radix_lock(self._handle, int(node)))

    def unlock(self, node):
        _check(_lib.pkv_radix_unlock(self._handle, int(node)))

    def set_score(self, node, score):
        _check(_lib.pkv_radix_set_score(self._handle, int(node), float(score)))

    def evict(self, num_blocks):
        """(blocks released to the pool's free list, evicted node ids in order)."""
        released = np.zeros(1, dtype=np.int32)
        count = np.zeros(1, dtype=np.int32)
        cap = max(self.num_nodes(), 1)
        ids = np.empty(cap, dtype=np.int64)
        _check(_lib.pkv_radix_evict(self._handle, int(num_blocks), _ptr(released), _ptr(ids), cap, _ptr(count)))
        return int(released[0]), ids[:int(count[0])].tolist()

    def clear(self):
        _check(_lib.pkv_radix_clear(self._handle))

    def num_nodes(self):
        return int(_lib.pkv_radix_num_nodes(self._handle))

    def cached_blocks(self):
        return int(_lib.pkv_radix_cached_blocks(self._handle))

    def evictable_blocks(self):
        return int(_lib.pkv_radix_evictable_blocks(self._handle))

    def node_ids(self):
        n = self.num_nodes()
        out = np.empty(n, dtype=np.int64)
        _lib.pkv_radix_node_ids(self._handle, _ptr(out), n)
        return out.tolist()

    def _info(self, node):
        parent = np.zeros(1, dtype=np.int64)
        lock = np.zeros(1, dtype=np.int32)
        last = np.zeros(1, dtype=np.int64)
        score = np.zeros(1, dtype=np.float64)
        depth = np.zeros(1, dtype=np.int32)
        nb = np.zeros(1, dtype=np.int32)
        _check(_lib.pkv_radix_node_info(self._handle, int(node), _ptr(parent), _ptr(lock), _ptr(last), _ptr(score),
                                        _ptr(depth), _ptr(nb), None, 0, None, 0))
        n = int(nb[0])
        blocks = np.empty(max(n, 1), dtype=np.int32)
        tokens = np.empty(max(n * self.block_size, 1), dtype=np.int32)
        _check(_lib.pkv_radix_node_info(self._handle, int(node), None, None, None, None, None, None, _ptr(blocks), n,
                                        _ptr(tokens), n * self.block_size))
        return (int(parent[0]), blocks[:n].tolist(), int(lock[0]), int(last[0]), float(score[0]),
                int(depth[0])), tokens[:n * self.block_size].tolist()

    def node_info(self, node):
        """(parent id, block ids, lock_ref, last access time, score, depth); parent -1 for the root."""
        return self._info(node)[0]

    def node_tokens(self, node):
        return self._info(node)[1]


# ---------------------------------------------------------------------------
# cascade plan


class CascadePlan:
    """Shared-prefix plan built on the host from block tables and lengths (numpy int32)."""

    def __init__(self, block_tables, seq_lens, num_q_heads, num_kv_heads, block_size=16, min_members=2):
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        _require(bt.ndim == 2 and sl.shape == (bt.shape[0],), "block_tables [B, max_blocks], seq_lens [B]")
        h = _lib.pkv_plan_build(_ptr(bt), _ptr(sl), bt.shape[0], bt.shape[1], int(block_size), int(num_q_heads),
                                int(num_kv_heads), int(min_members))
        if not h:
            raise PkvInvalid(PKV_ERR_INVALID, _lib.pkv_last_error().decode())
        self._handle = h
        self.batch = bt.shape[0]
        self.device_buffer = None

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and _lib is not None:  # at interpreter exit the module globals may already be gone
            _lib.pkv_plan_destroy(h)
            self._handle = None

    @property
    def device_bytes(self):
        return int(_lib.pkv_plan_device_bytes(self._handle))

    def upload(self, device="cuda", stream=None, buffer=None):
        """Copy the plan's tables to device memory (a torch buffer it keeps) and bind them."""
        import torch

        n = self.device_bytes
        if buffer is None:
            buffer = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
        _check(_lib.pkv_plan_upload(self._handle, _ptr(buffer), buffer.numel(), _stream(stream, buffer)))
        self.device_buffer = buffer
        return self

    @property
    def num_nodes(self):
        return int(_lib.pkv_plan_num_nodes(self._handle))

    def node(self, i):
        """(block ids, member rows) of shared node i."""
        nb = np.zeros(1, dtype=np.int32)
        nm = np.zeros(1, dtype=np.int32)
        _check(_lib.pkv_plan_node(self._handle, int(i), _ptr(nb), _ptr(nm), None, None))
        blocks = np.empty(max(int(nb[0]), 1), dtype=np.int32)
        members = np.empty(max(int(nm[0]), 1), dtype=np.int32)
        _check(_lib.pkv_plan_node(self._handle, int(i), None, None, _ptr(blocks), _ptr(members)))
        return blocks[: int(nb[0])].copy(), members[: int(nm[0])].copy()

    def node_pieces(self, i):
        """Token pieces node i is split into (one partial slot each)."""
        n = int(_lib.pkv_plan_node_pieces(self._handle, int(i)))
        if n < 0:
            raise PkvInvalid(PKV_ERR_INVALID, f"bad node index {i}")
        return n

    @property
    def rows_per_item(self):
        """Query rows per work item of the matrix-core pass (64 decode, 128 extend)."""
        return int(_lib.pkv_plan_rows_per_item(self._handle))

    def image(self):
        """(int32 image, {section: offset}, partial slots per query row) as uploaded to the device;
        the sections are row_info, nodes, blocks, members, items and item_recs (the work-item
        records, ``item_ints`` ints each)."""
        offs = np.zeros(6, dtype=np.int64)
        n = int(_lib.pkv_plan_image(self._handle, None, 0, _ptr(offs)))
        img = np.zeros(max(n, 1), dtype=np.int32)
        _lib.pkv_plan_image(self._handle, _ptr(img), n, _ptr(offs))
        names = ("row_info", "nodes", "blocks", "members", "items")
        sections = dict(zip(names, offs[:5].tolist()))
        ints = np.zeros(1, dtype=np.int32)
        sections["item_recs"] = int(_lib.pkv_plan_item_records(self._handle, _ptr(ints)))
        sections["item_ints"] = int(ints[0])
        return img[:n], sections, int(offs[5])

    def row(self, b):
        """(shared tokens, partial slots used by the row's nodes) of row b."""
        st = np.zeros(1, dtype=np.int32)
        dp = np.zeros(1, dtype=np.int32)
        _check(_lib.pkv_plan_row(self._handle, int(b), _ptr(st), _ptr(dp)))
        return int(st[0]), int(dp[0])


class ExtendPlan(CascadePlan):
    """Plan for multi-token (extend) attention: block tables, lengths and the number of new query
    tokens per row (numpy int32); query rows are packed in row order."""

    def __init__(self, block_tables, seq_lens, q_lens, num_q_heads, num_kv_heads, block_size=16, min_members=2):
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        ql = np.ascontiguousarray(q_lens, dtype=np.int32)
        _require(bt.ndim == 2 and sl.shape == (bt.shape[0],) and ql.shape == sl.shape,
                 "block_tables [B, max_blocks], seq_lens [B], q_lens [B]")
        h = _lib.pkv_plan_build_extend(_ptr(bt), _ptr(sl), _ptr(ql), bt.shape[0], bt.shape[1], int(block_size),
                                       int(num_q_heads), int(num_kv_heads), int(min_members))
        if not h:
            raise PkvInvalid(PKV_ERR_INVALID, _lib.pkv_last_error().decode())
        self._handle = h
        self.batch = bt.shape[0]
        self.device_buffer = None

    @property
    def num_query_rows(self):
        return int(_lib.pkv_plan_num_query_rows(self._handle))


def extend_workspace_bytes(plan, head_dim):
    n = _lib.pkv_extend_workspace_bytes(plan._handle, int(head_dim))
    if n == 0:
        raise PkvInvalid(PKV_ERR_INVALID, _lib.pkv_last_error().decode())
    return int(n)


def paged_extend_attn(q, k_pages, v_pages, plan, scale=None, workspace=None, out=None, dtype=None, stream=None):
    """Causal multi-token attention: query row r (token i of row b, at position
    seq_lens[b] - q_lens[b] + i) attends to its row's tokens [0, position] (fp32 output).

    q: [num_query_rows, Hq, d] device tensor; pages [num_blocks, 16, Hkv, d]; ``plan``: an uploaded ExtendPlan.
    """
    import torch

    _require(isinstance(plan, ExtendPlan) and plan.device_buffer is not None, "plan must be an uploaded ExtendPlan")
    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad q / page ranks")
    _require(q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous(), "inputs must be contiguous")
    nq, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    need = extend_workspace_bytes(plan, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((nq, hq, d), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (nq, hq, d), "bad out tensor")
    _check(_lib.pkv_paged_extend_attn(_ptr(q), nq, hq, hkv, d, _dtype_code(q, dtype), _ptr(k_pages), _ptr(v_pages),
                                      nblk, bs, float(scale), plan._handle, _ptr(workspace), ws_bytes, _ptr(out),
                                      _stream(stream, q)))
    return out


def paged_extend_attn_fp8(q, k_pages, v_pages, k_scales, v_scales, plan, scale=None, workspace=None, out=None,
                          q_dtype=None, stream=None):
    """``paged_extend_attn`` over FP8 pages (uint8 codes, float32 scales [num_blocks, Hkv, 16])."""
    import torch

    _require(isinstance(plan, ExtendPlan) and plan.device_buffer is not None, "plan must be an uploaded ExtendPlan")
    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape and k_pages.dtype == torch.uint8,
             "q [NQ, Hq, d]; uint8 pages [num_blocks, block_size, Hkv, d]")
    nq, hq, d = q.shape
    nblk, bs, hkv, dk = k_pages.shape
    _require(dk == d, "head_dim of q and pages differ")
    _require(tuple(k_scales.shape) == (nblk, hkv, bs) and tuple(v_scales.shape) == (nblk, hkv, bs) and
             k_scales.dtype == v_scales.dtype == torch.float32, "scales must be float32 [num_blocks, Hkv, block_size]")
    _require(all(t.is_contiguous() for t in (q, k_pages, v_pages, k_scales, v_scales)), "inputs must be contiguous")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    need = extend_workspace_bytes(plan, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((nq, hq, d), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (nq, hq, d), "bad out tensor")
    _check(_lib.pkv_paged_extend_attn_fp8(_ptr(q), nq, hq, hkv, d, _dtype_code(q, q_dtype), _ptr(k_pages),
                                          _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), nblk, bs, float(scale),
                                          plan._handle, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _ptr(out), _stream(stream, q)))
    return out


# ---------------------------------------------------------------------------
# timing


def copy_blocks(dst, src, dst_ids, src_ids, stream=None, max_workgroups=0):
    """Block copies between block arrays (device tensors or pinned host tensors):
    block dst_ids[i] of each dst[k] = block src_ids[i] of src[k].  dst and src are
    equal-length lists of tensors whose first dimension counts blocks; the id
    tensors are int32 on the device (or pinned host memory).  ``max_workgroups``
    caps the launch (0: one work-group per block and array)."""
    _require(len(dst) == len(src) and 1 <= len(dst) <= 4, "1..4 destination / source arrays")
    n = int(dst_ids.numel())
    _require(int(src_ids.numel()) == n, "dst_ids and src_ids differ in length")
    for t in (dst_ids, src_ids):
        _require(str(t.dtype) == "torch.int32" and t.is_contiguous(), "ids must be contiguous int32 tensors")
    nd, ns = int(dst[0].shape[0]), int(src[0].shape[0])
    bb = []
    for d, s in zip(dst, src):
        _require(d.is_contiguous() and s.is_contiguous(), "block arrays must be contiguous")
        _require(d.shape[0] == nd and s.shape[0] == ns, "every array of one side must hold the same block count")
        b = d[0].numel() * d.element_size() if nd else s[0].numel() * s.element_size()
        _require(s[0].numel() * s.element_size() == b if ns else True, "block sizes differ between dst and src")
        bb.append(b)
    dp = (_vp * len(dst))(*[t.data_ptr() for t in dst])
    sp = (_vp * len(src))(*[t.data_ptr() for t in src])
    bytes_ = (_i64 * len(dst))(*bb)
    dev = dst_ids if dst_ids.is_cuda else (dst[0] if dst[0].is_cuda else src[0])
    _check(_lib.pkv_copy_blocks(len(dst), dp, sp, bytes_, nd, ns, _ptr(dst_ids), _ptr(src_ids), n,
                                int(max_workgroups), _stream(stream, dev)))


def copy_blocks_memcpy(dst, src, dst_ids, src_ids, stream=None):
    """``copy_blocks`` as one runtime copy per run of consecutive ids; ids are host sequences of ints."""
    _require(len(dst) == len(src) and 1 <= len(dst) <= 4, "1..4 destination / source arrays")
    di = np.ascontiguousarray(dst_ids, dtype=np.int32)
    si = np.ascontiguousarray(src_ids, dtype=np.int32)
    _require(di.shape == si.shape and di.ndim == 1, "dst_ids and src_ids differ in shape")
    nd, ns = int(dst[0].shape[0]), int(src[0].shape[0])
    bb = []
    for d, s in zip(dst, src):
        _require(d.is_contiguous() and s.is_contiguous(), "block arrays must be contiguous")
        _require(d.shape[0] == nd and s.shape[0] == ns, "every array of one side must hold the same block count")
        b = d[0].numel() * d.element_size() if nd else s[0].numel() * s.element_size()
        _require(s[0].numel() * s.element_size() == b if ns else True, "block sizes differ between dst and src")
        bb.append(b)
    dp = (_vp * len(dst))(*[t.data_ptr() for t in dst])
    sp = (_vp * len(src))(*[t.data_ptr() for t in src])
    bytes_ = (_i64 * len(dst))(*bb)
    dev = dst[0] if dst[0].is_cuda else src[0]
    _check(_lib.pkv_copy_blocks_memcpy(len(dst), dp, sp, bytes_, nd, ns, di.ctypes.data, si.ctypes.data, di.shape[0],
                                    _stream(stream, dev)))


def stream_read(buf, sink, grid=0, stream=None):
    """Plain streaming read of a device tensor (the read-bandwidth yardstick); sink: int32 [1] device."""
    _check(_lib.pkv_stream_read(_ptr(buf), buf.numel() * buf.element_size() // 16 * 16, _ptr(sink), int(grid),
                                _stream(stream, buf)))


def timing_enable(on=True):
    _check(_lib.pkv_timing_enable(1 if on else 0))


def timing_reset():
    _check(_lib.pkv_timing_reset())


def timing_read(kernel):
    """(total milliseconds, launches) for kernel name or id since the last reset."""
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    ms = np.zeros(1, dtype=np.float64)
    cnt = np.zeros(1, dtype=np.int64)
    _check(_lib.pkv_timing_read(k, _ptr(ms), _ptr(cnt)))
    return float(ms[0]), int(cnt[0])
