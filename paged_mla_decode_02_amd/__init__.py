"""Python binding of libmla_decode.so (paged MLA decode for MI355X / gfx950).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels; torch supplies device memory and streams. The entry points mirror the
C ABI in include/mla_decode.h:

    plan(kv_lens, heads, q_len_max, kv_dtype, mode, num_cus) -> int32 numpy words
    workspace_size(plan_words) -> bytes
    decode_fwd(...)        enqueue decode (+ merge) on the current stream
    debug_gather(...)      the decode kernel's gather, written to a dense tensor

``MlaDecoder`` wraps the per-batch steps a caller repeats (build the plan on the
host, upload it, size the workspace, launch). If the library is missing or a
call fails, an error is raised; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")

MLA_BF16, MLA_FP8_E4M3 = 0, 1
PLAN_AUTO, PLAN_UNIFORM, PLAN_LENGTH_AWARE = 0, 1, 2
D_LATENT, D_V = 576, 512
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "WORKSPACE", -4: "PLAN_MISMATCH",
          -5: "HIP"}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load the shared library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} not found: build it first (python -m paged_mla_decode_02_amd.build)")
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.mla_decode_plan_capacity.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i64)]
    lib.mla_decode_plan_capacity.restype = i32
    lib.mla_decode_plan.argtypes = [p32, i32, i32, i32, i32, i32, i32, p32, i64]
    lib.mla_decode_plan.restype = i32
    lib.mla_decode_workspace_size.argtypes = [p32, ctypes.POINTER(i64)]
    lib.mla_decode_workspace_size.restype = i32
    lib.mla_decode_workspace_init.argtypes = [p32, vp, i64, vp]
    lib.mla_decode_workspace_init.restype = i32
    lib.mla_decode_fwd.argtypes = [vp, i32, vp, vp, i32, vp, i64, vp, vp, vp, p32, vp, i32, i32,
                                   i32, i32, ctypes.c_float, vp, vp, vp, i64, vp]
    lib.mla_decode_fwd.restype = i32
    lib.mla_decode_fwd_noalloc.argtypes = [vp, i32, vp, vp, i32, vp, i64, vp, vp, vp, p32, vp, i32, i32,
                                           i32, i32, ctypes.c_float, vp, vp, vp]
    lib.mla_decode_fwd_noalloc.restype = i32
    lib.mla_debug_gather.argtypes = [vp, i32, i64, vp, vp, p32, vp, i32, vp, vp]
    lib.mla_debug_gather.restype = i32
    lib.mla_decode_fwd_dcp.argtypes = [vp, i32, vp, vp, i32, vp, i64, vp, vp, vp, p32, vp, i32, i32,
                                       i32, i32, ctypes.c_float, vp, vp, vp, i64, i32, i32, vp, vp]
    lib.mla_decode_fwd_dcp.restype = i32
    lib.mla_merge_shards.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.mla_merge_shards.restype = i32
    lib.mla_cache_write.argtypes = [vp, i32, i64, vp, i32, i64, vp, i32, vp, i32, vp, i64, vp]
    lib.mla_cache_write.restype = i32
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = i32
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().mla_last_error().decode()


def _check(status: int):
    if status != 0:
        raise MlaError(status, last_error())


def _dtype_code(name_or_code) -> int:
    if name_or_code in (MLA_BF16, MLA_FP8_E4M3):
        return int(name_or_code)
    return {"bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}[name_or_code]


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def plan_capacity(rows: int, num_cus: int, heads: int, q_len_max: int) -> int:
    n = ctypes.c_int64(0)
    _check(load_library().mla_decode_plan_capacity(rows, num_cus, heads, q_len_max, ctypes.byref(n)))
    return n.value


def plan(kv_lens, heads: int, q_len_max: int, kv_dtype, mode: int = PLAN_AUTO,
         num_cus: int = 256) -> np.ndarray:
    """Host split plan (int32 words) for these per-row KV lengths."""
    lens = _host_i32(kv_lens)
    rows = int(lens.shape[0])
    cap = plan_capacity(max(rows, 1), num_cus, heads, q_len_max) if rows >= 1 and 1 <= heads <= 128 \
        and 1 <= q_len_max <= 16 and num_cus >= 1 else 64
    out = np.zeros(cap, dtype=np.int32)
    _check(load_library().mla_decode_plan(
        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), rows, heads, q_len_max,
        _dtype_code(kv_dtype), int(mode), num_cus,
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap))
    return out[:int(out[19])].copy()


def workspace_size(plan_words: np.ndarray) -> int:
    w = _host_i32(plan_words)
    n = ctypes.c_int64(0)
    _check(load_library().mla_decode_workspace_size(w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                   ctypes.byref(n)))
    return n.value


PLAN_MERGE_IN_KERNEL = 0x100
PLAN_FP8_PV = 0x200   # fp8 PV products (fp8 KV; not with PLAN_MERGE_IN_KERNEL)


def workspace_init(plan_words: np.ndarray, workspace, stream=None):
    """Enqueue mla_decode_workspace_init (zero the split counters)."""
    w = _host_i32(plan_words)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().mla_decode_workspace_init(w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                    _ptr(workspace), nbytes, _stream_handle(stream)))


def alloc_workspace(plan_words: np.ndarray, device="cuda", min_bytes: int = 16):
    """A zeroed workspace tensor (uint8) for this plan, ready for decode_fwd."""
    import torch
    return torch.zeros(max(workspace_size(plan_words), min_bytes), dtype=torch.uint8, device=device)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


_EMPTY_STANDIN = {}


def _ptr_any(t) -> int:
    """The address of a device tensor that may have no elements. An empty
    tensor has no storage (address 0), while the library wants a valid
    address even for an argument it will not touch: every query block or
    index list empty. A small aligned buffer per device stands in for it."""
    if t.numel() > 0:
        return int(t.data_ptr())
    import torch
    key = str(t.device)
    if key not in _EMPTY_STANDIN:
        _EMPTY_STANDIN[key] = torch.zeros(64, dtype=torch.int32, device=t.device)
    return int(_EMPTY_STANDIN[key].data_ptr())


def _stream_handle(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


_CODE_DTYPES = None


def _code_dtypes():
    """torch dtypes accepted as the stored codes of each format: bf16 bits
    (bfloat16 or int16), fp8 OCP e4m3fn codes (float8_e4m3fn or uint8)."""
    global _CODE_DTYPES
    if _CODE_DTYPES is None:
        import torch
        _CODE_DTYPES = {MLA_BF16: (torch.bfloat16, torch.int16),
                        MLA_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}
    return _CODE_DTYPES


def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def _check_device_tensor(name, t, device, dtypes, dim=None):
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor", TypeError)
    _need(t.is_cuda and t.device == device, f"{name} must be on {device}, got {t.device}")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}; expected one of {list(dtypes)}", TypeError)
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dim is not None:
        _need(t.dim() == dim, f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")


def _check_decode_tensors(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr,
                          kv_indices, rows, heads, q_len_max, o, lse, workspace=None):
    """Host-side checks of everything the C ABI cannot see: tensor dtypes,
    shapes, contiguity and device. The ABI then checks sizes, alignment and
    the plan. Raises TypeError / ValueError; nothing is launched."""
    import torch
    codes = _code_dtypes()
    dev = q.device if isinstance(q, torch.Tensor) else None
    _check_device_tensor("q", q, dev, codes[q_dtype], 3)
    _need(q.shape[1] == heads and q.shape[2] == D_LATENT,
          f"q must be [tokens, {heads}, {D_LATENT}], got {tuple(q.shape)}")
    _check_device_tensor("kv_pool", kv_pool, dev, codes[kv_dtype], 2)
    _need(kv_pool.shape[1] == D_LATENT and kv_pool.shape[0] >= 1,
          f"kv_pool must be [num_slots >= 1, {D_LATENT}], got {tuple(kv_pool.shape)}")
    for name, t in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if t is not None:
            _check_device_tensor(name, t, dev, (torch.float32,))
            _need(t.numel() >= 1, f"{name} must hold one float32")
    for name, t, n in (("qo_indptr", qo_indptr, rows + 1), ("kv_indptr", kv_indptr, rows + 1),
                       ("kv_indices", kv_indices, None)):
        _check_device_tensor(name, t, dev, (torch.int32,), 1)
        _need(n is None or t.numel() == n, f"{name} must have {n} entries, got {t.numel()}")
    tokens = min(int(q.shape[0]), rows * q_len_max)    # at most q_len_max tokens per row
    _check_device_tensor("o", o, dev, codes[MLA_BF16], 3)
    _need(o.shape[1] == heads and o.shape[2] == D_V and o.shape[0] >= tokens,
          f"o must be [>= {tokens}, {heads}, {D_V}] bf16, got {tuple(o.shape)}")
    _check_device_tensor("lse", lse, dev, (torch.float32,), 2)
    _need(lse.shape[1] == heads and lse.shape[0] >= tokens,
          f"lse must be [>= {tokens}, {heads}] float32, got {tuple(lse.shape)}")
    if workspace is not None:
        _check_device_tensor("workspace", workspace, dev, (torch.uint8, torch.int8))


def decode_fwd(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr, kv_indices,
               plan_host: np.ndarray, plan_dev, rows: int, heads: int, q_len_max: int, causal: bool,
               softmax_scale: float, o, lse, workspace=None, stream=None):
    """Enqueue mla_decode_fwd. Tensors are device tensors; q/kv_pool hold the
    stored codes (bf16 as int16/bfloat16, fp8 as uint8/float8_e4m3fn);
    q_scale/kv_scale are 1-element float32 device tensors or None."""
    q_dtype, kv_dtype = _dtype_code(q_dtype), _dtype_code(kv_dtype)
    _check_decode_tensors(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr,
                          kv_indices, rows, heads, q_len_max, o, lse, workspace)
    ph = _host_i32(plan_host)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().mla_decode_fwd(
        _ptr_any(q), _dtype_code(q_dtype), _ptr(q_scale), _ptr(kv_pool), _dtype_code(kv_dtype),
        _ptr(kv_scale), int(kv_pool.shape[0]), _ptr(qo_indptr), _ptr(kv_indptr), _ptr_any(kv_indices),
        ph.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(plan_dev), rows, heads, q_len_max,
        1 if causal else 0, float(softmax_scale), _ptr_any(o), _ptr_any(lse), _ptr(workspace), ws_bytes,
        _stream_handle(stream))
    _check(st)


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_fwd_noalloc(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr,
                       kv_indices, plan_host: np.ndarray, plan_dev, rows: int, heads: int,
                       q_len_max: int, causal: bool, softmax_scale: float, o, lse, stream=None):
    """Enqueue mla_decode_fwd_noalloc: decode_fwd with the split partials in
    the library's static per-GPU scratch (no workspace, nothing allocated).
    Calls that overlap on one GPU race."""
    q_dtype, kv_dtype = _dtype_code(q_dtype), _dtype_code(kv_dtype)
    _check_decode_tensors(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr,
                          kv_indices, rows, heads, q_len_max, o, lse)
    ph = _host_i32(plan_host)
    st = load_library().mla_decode_fwd_noalloc(
        _ptr_any(q), _dtype_code(q_dtype), _ptr(q_scale), _ptr(kv_pool), _dtype_code(kv_dtype),
        _ptr(kv_scale), int(kv_pool.shape[0]), _ptr(qo_indptr), _ptr(kv_indptr), _ptr_any(kv_indices),
        ph.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(plan_dev), rows, heads, q_len_max,
        1 if causal else 0, float(softmax_scale), _ptr_any(o), _ptr_any(lse), _stream_handle(stream))
    _check(st)


def decode_fwd_dcp(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr, kv_indices,
                   plan_host: np.ndarray, plan_dev, rows: int, heads: int, q_len_max: int, causal: bool,
                   softmax_scale: float, o, lse, dcp_world: int, dcp_rank: int, kv_len_global,
                   workspace=None, stream=None):
    """Enqueue mla_decode_fwd_dcp for shard dcp_rank of dcp_world (its own
    index lists and plan); kv_len_global is an int32 device tensor [rows]."""
    import torch
    q_dtype, kv_dtype = _dtype_code(q_dtype), _dtype_code(kv_dtype)
    _check_decode_tensors(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, qo_indptr, kv_indptr,
                          kv_indices, rows, heads, q_len_max, o, lse, workspace)
    _check_device_tensor("kv_len_global", kv_len_global, q.device, (torch.int32,), 1)
    _need(kv_len_global.numel() == rows, f"kv_len_global must have {rows} entries")
    ph = _host_i32(plan_host)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().mla_decode_fwd_dcp(
        _ptr_any(q), _dtype_code(q_dtype), _ptr(q_scale), _ptr(kv_pool), _dtype_code(kv_dtype),
        _ptr(kv_scale), int(kv_pool.shape[0]), _ptr(qo_indptr), _ptr(kv_indptr), _ptr_any(kv_indices),
        ph.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(plan_dev), rows, heads, q_len_max,
        1 if causal else 0, float(softmax_scale), _ptr_any(o), _ptr_any(lse), _ptr(workspace), ws_bytes,
        int(dcp_world), int(dcp_rank), _ptr(kv_len_global), _stream_handle(stream))
    _check(st)


def merge_shards(o_parts, lse_parts, o, lse, stream=None):
    """Enqueue mla_merge_shards: o_parts bf16 [W, T, H, 512], lse_parts fp32
    [W, T, H] -> o bf16 [T, H, 512], lse fp32 [T, H]."""
    W, T, H = int(o_parts.shape[0]), int(o_parts.shape[1]), int(o_parts.shape[2])
    if tuple(lse_parts.shape) != (W, T, H) or tuple(o.shape) != (T, H, 512) or tuple(lse.shape) != (T, H):
        raise ValueError("shape mismatch between o_parts, lse_parts, o and lse")
    for t in (o_parts, lse_parts, o, lse):
        if not t.is_contiguous():
            raise ValueError("merge_shards needs contiguous tensors")
    _check(load_library().mla_merge_shards(_ptr(o_parts), _ptr(lse_parts), W, T, H, _ptr(o), _ptr(lse),
                                           _stream_handle(stream)))


def debug_gather(kv_pool, kv_dtype, kv_indptr, kv_indices, plan_host: np.ndarray, plan_dev,
                 rows: int, dense_out, stream=None):
    """Enqueue mla_debug_gather: the decode kernel's gather of every split,
    written as bf16 bits to dense_out [kv_indptr[rows] - kv_indptr[0], 576]."""
    import torch
    kv_dtype = _dtype_code(kv_dtype)
    dev = kv_pool.device
    _check_device_tensor("kv_pool", kv_pool, dev, _code_dtypes()[kv_dtype], 2)
    _need(kv_pool.shape[1] == D_LATENT, f"kv_pool must be [num_slots, {D_LATENT}]")
    for name, t in (("kv_indptr", kv_indptr), ("kv_indices", kv_indices)):
        _check_device_tensor(name, t, dev, (torch.int32,), 1)
    _need(kv_indptr.numel() == rows + 1, f"kv_indptr must have {rows + 1} entries")
    _check_device_tensor("dense_out", dense_out, dev, _code_dtypes()[MLA_BF16], 2)
    _need(dense_out.shape[1] == D_LATENT, f"dense_out must be [keys, {D_LATENT}]")
    ph = _host_i32(plan_host)
    st = load_library().mla_debug_gather(
        _ptr(kv_pool), _dtype_code(kv_dtype), int(kv_pool.shape[0]), _ptr(kv_indptr),
        _ptr(kv_indices), ph.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(plan_dev), rows,
        _ptr(dense_out), _stream_handle(stream))
    _check(st)


MLA_SRC_BF16, MLA_SRC_FP16, MLA_SRC_FP32 = 0, 1, 2


def cache_write(kv_c, k_pe, slot_mapping, kv_pool, kv_dtype, kv_scale=None, stream=None):
    """Enqueue mla_cache_write. kv_c [T, 512] and k_pe [T, 64] are device
    tensors of bfloat16, float16 or float32 (rows may be strided, elements
    contiguous); each is passed with its own dtype. slot_mapping is an int64
    device tensor [T] (negative = skip); kv_pool holds the stored codes
    [num_slots, 576]; kv_scale a 1-element float32 device tensor or None."""
    import torch
    src = {torch.bfloat16: MLA_SRC_BF16, torch.float16: MLA_SRC_FP16, torch.float32: MLA_SRC_FP32}
    for name, t, width in (("kv_c", kv_c, 512), ("k_pe", k_pe, 64)):
        if t.dtype not in src:
            raise TypeError(f"{name} must be bfloat16, float16 or float32, got {t.dtype}")
        if t.dim() != 2 or t.shape[1] != width or t.stride(1) != 1:
            raise ValueError(f"{name} must be [tokens, {width}] with contiguous rows")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int64 tensor")
    tokens = int(slot_mapping.shape[0])
    if kv_c.shape[0] != tokens or k_pe.shape[0] != tokens:
        raise ValueError("kv_c, k_pe and slot_mapping must have the same number of tokens")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != 576 or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be a contiguous [num_slots, 576] tensor")
    st = load_library().mla_cache_write(
        _ptr(kv_c), src[kv_c.dtype], int(kv_c.stride(0)), _ptr(k_pe), src[k_pe.dtype],
        int(k_pe.stride(0)), _ptr(slot_mapping), tokens, _ptr(kv_pool), _dtype_code(kv_dtype),
        _ptr(kv_scale), int(kv_pool.shape[0]), _stream_handle(stream))
    _check(st)


class MlaDecoder:
    """Holds the device tensors of one decode batch and runs the hot path:
    host plan -> plan upload (pinned, async) -> decode kernel -> merge kernel.

    ``inputs`` is a dict of device tensors: q, kv_pool, qo_indptr, kv_indptr,
    kv_indices, and optional q_scale / kv_scale (float32, 1 element)."""

    def __init__(self, heads: int, q_len_max: int, q_dtype, kv_dtype, causal: bool,
                 softmax_scale: float, mode: int = PLAN_AUTO, num_cus: Optional[int] = None,
                 device=None):
        import torch
        self.torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.heads, self.q_len_max = heads, q_len_max
        self.q_dtype, self.kv_dtype = _dtype_code(q_dtype), _dtype_code(kv_dtype)
        self.causal, self.softmax_scale, self.mode = causal, softmax_scale, mode
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        self.num_cus = num_cus
        self._plan_pinned = None
        self._plan_dev = None
        self._plan_copied = None   # event: the last host->device plan copy finished reading
        self._ws = None

    def make_plan(self, kv_lens) -> np.ndarray:
        return plan(kv_lens, self.heads, self.q_len_max, self.kv_dtype, self.mode, self.num_cus)

    def upload_plan(self, words: np.ndarray):
        torch = self.torch
        n = int(words.shape[0])
        if self._plan_pinned is None or self._plan_pinned.numel() < n:
            self._plan_pinned = torch.empty(max(n, 1024), dtype=torch.int32, pin_memory=True)
            self._plan_dev = torch.empty(max(n, 1024), dtype=torch.int32, device=self.device)
        if self._plan_copied is not None:
            self._plan_copied.synchronize()   # the pinned buffer may still be in flight
        self._plan_pinned[:n].copy_(torch.from_numpy(words))
        self._plan_dev[:n].copy_(self._plan_pinned[:n], non_blocking=True)
        self._plan_copied = torch.cuda.Event()
        self._plan_copied.record()
        return self._plan_dev

    def workspace(self, words: np.ndarray):
        nbytes = workspace_size(words)
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes:
            # zeroed: the counter region must start at zero; calls keep it so
            self._ws = self.torch.zeros(nbytes, dtype=self.torch.uint8, device=self.device)
        return self._ws

    def run(self, inputs: dict, kv_lens, o, lse, words: Optional[np.ndarray] = None):
        """One pass of the hot path; returns the plan words used."""
        if words is None:
            words = self.make_plan(kv_lens)
        plan_dev = self.upload_plan(words)
        ws = self.workspace(words)
        rows = int(len(kv_lens))
        decode_fwd(inputs["q"], self.q_dtype, inputs.get("q_scale"), inputs["kv_pool"],
                   self.kv_dtype, inputs.get("kv_scale"), inputs["qo_indptr"], inputs["kv_indptr"],
                   inputs["kv_indices"], words, plan_dev, rows, self.heads, self.q_len_max,
                   self.causal, self.softmax_scale, o, lse, ws)
        return words


def device_inputs(q_codes: np.ndarray, q_scale, pool_codes: np.ndarray, kv_scale,
                  qo_indptr, kv_indptr, kv_indices, device="cuda") -> dict:
    """Copy stored host arrays (bf16 bit patterns as uint16, fp8 codes as uint8,
    int32 CSR lists, float scales or None) to device tensors."""
    import torch

    def codes(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device)
        if a.dtype == np.uint8:
            return torch.from_numpy(a).to(device)
        raise TypeError(f"stored codes must be uint16 (bf16) or uint8 (fp8), got {a.dtype}")

    def scale(x):
        return None if x is None else torch.tensor([float(x)], dtype=torch.float32, device=device)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)

    return {"q": codes(q_codes), "q_scale": scale(q_scale), "kv_pool": codes(pool_codes),
            "kv_scale": scale(kv_scale), "qo_indptr": i32(qo_indptr), "kv_indptr": i32(kv_indptr),
            "kv_indices": i32(kv_indices)}
