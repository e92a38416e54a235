"""libvqkv: decode attention over a vector-quantized KV cache on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/vqkv.h``.  Every function
here only checks and marshals arguments (torch tensors supply device memory
and the current HIP stream); all computation runs in the HIP kernels of
``libvqkv.so``.  There is no CPU fallback: if the library is missing, importing
this package raises.

Method (VecInfer, arXiv 2510.06175; research.elamur.ai summary card): keys are
smoothed per channel and Hadamard-rotated, keys and values are stored as
K-Means codebook indices (2^8 x 4 for 2 bits, 2^12 x 8 for 1.5 bits), the
query gets the inverse transform, and attention dequantizes inside the kernel.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqkv.so")

FMT_2BIT = 0
FMT_1P5BIT = 1
FMT_3BIT = 2                      # 4096 x 4: a third width inside the pages' 1.25-4 bit range
FMT_1P25BIT = 3                   # 1024 x 8: the low end of that range
FMT_4BIT = 4                      # 256 x 2: the high end
FMT_VALUE_TRANSFORM = 0x100      # OR'ed into a format: values smoothed and rotated too
DTYPE_BF16 = 0
DTYPE_FP32 = 1
HEAD_DIM = 128
ENTRIES = {FMT_2BIT: 256, FMT_1P5BIT: 4096, FMT_3BIT: 4096, FMT_1P25BIT: 1024, FMT_4BIT: 256}
DSUB = {FMT_2BIT: 4, FMT_1P5BIT: 8, FMT_3BIT: 4, FMT_1P25BIT: 8, FMT_4BIT: 2}
# Kernels selectable for measurement (measure_decode_attention).
DECODE_PATHS = {"default": 0, "table": 1, "gather": 2, "mfma": 3}

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP runtime error"}


class VqkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("fmt", ctypes.c_int32)]


def make_shape(batch: int, num_q_heads: int, num_kv_heads: int, max_tokens: int, fmt: int,
               head_dim: int = HEAD_DIM) -> Shape:
    return Shape(batch, num_q_heads, num_kv_heads, head_dim, max_tokens, fmt)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvqkv.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m vector_quantized_bit_vqkv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    SP = ctypes.POINTER(Shape)
    sig = {
        "vqkv_code_bytes_per_token": (SZ, [I32]),
        "vqkv_cache_bytes": (SZ, [SP]),
        "vqkv_workspace_bytes": (SZ, [SP, I32]),
        "vqkv_suggest_splits": (I32, [SP, I32]),
        "vqkv_status_string": (ctypes.c_char_p, [I32]),
        "vqkv_last_error": (ctypes.c_char_p, []),
        "vqkv_transform_query": (I32, [SP, P, I32, P, P, P]),
        "vqkv_quantize_append": (I32, [SP, P, P, I32, I32, I32, P, P, P, P, P, P]),
        "vqkv_decode_attention": (I32, [SP, P, P, P, P, P, I32, F32, I32, P, P]),
        "vqkv_combine": (I32, [SP, I32, P, P, P]),
        "vqkv_step_workspace_bytes": (SZ, [SP, I32]),
        "vqkv_value_output_transform": (I32, [SP, P, P, P]),
        "vqkv_decode_step": (I32, [SP, P, P, P, I32, I32, P, P, P, P, P, F32, I32, P, P, P]),
        "vqkv_decode_step_static": (I32, [SP, P, P, P, I32, I32, P, P, P, P, P, F32, I32, P, P]),
        "vqkv_decode_step_varlen": (I32, [SP, P, P, P, I32, P, I32, P, P, P, P, P, F32, I32, P, P, P]),
        "vqkv_decode_step_paged": (I32, [SP, P, P, P, I32, P, I32, P, P, P, P, P, I32, P, F32, I32, P, P, P]),
        "vqkv_decode_attention_varlen": (I32, [SP, P, P, P, P, P, P, I32, F32, I32, P, P]),
        "vqkv_quantize_append_varlen": (I32, [SP, P, P, I32, P, P, P, P, P, P, P]),
        "vqkv_decode_attention_paged": (I32, [SP, P, P, P, P, P, I32, P, P, I32, F32, I32, P, P]),
        "vqkv_quantize_append_paged": (I32, [SP, P, P, I32, P, P, P, P, P, P, I32, P, P]),
        "vqkv_smooth_scales": (I32, [I32, I32, P, I32, P, P]),
        "vqkv_train_workspace_bytes": (SZ, [I32, I32]),
        "vqkv_train_codebook": (I32, [I32, I32, P, I32, I32, P, P, I32, P, P, P, P]),
        "vqkv_measure_decode_attention": (I32, [SP, P, P, P, P, P, I32, F32, I32, P, I32, P]),
        "vqkv_baseline_bf16_decode": (I32, [SP, P, P, P, I32, F32, I32, P, P]),
        "vqkv_baseline_read_stream": (I32, [P, SZ, P, I32, P]),
        "vqkv_baseline_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise VqkvError(status, lib().vqkv_last_error().decode())


def _ptr(t) -> ctypes.c_void_p | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------------- sizes

def code_bytes_per_token(fmt: int) -> int:
    return int(lib().vqkv_code_bytes_per_token(fmt))


def cache_bytes(shape: Shape) -> int:
    return int(lib().vqkv_cache_bytes(ctypes.byref(shape)))


def workspace_bytes(shape: Shape, num_splits: int) -> int:
    return int(lib().vqkv_workspace_bytes(ctypes.byref(shape), num_splits))


def step_workspace_bytes(shape: Shape, num_splits: int) -> int:
    return int(lib().vqkv_step_workspace_bytes(ctypes.byref(shape), num_splits))


def suggest_splits(shape: Shape, seq_len: int) -> int:
    return int(lib().vqkv_suggest_splits(ctypes.byref(shape), seq_len))


# ---------------------------------------------------------------------- hot path

def transform_query(shape: Shape, q, smooth, q_prime) -> None:
    """q' = H (q * s): q [B][Hq][128] bf16/fp32, smooth fp32 [Hkv][128], q_prime fp32 out."""
    _check(lib().vqkv_transform_query(ctypes.byref(shape), _ptr(q), _dtype_code(q), _ptr(smooth),
                                      _ptr(q_prime), _stream(q)))


def quantize_append(shape: Shape, k_new, v_new, start_pos: int, smooth, k_book, v_book, k_codes, v_codes) -> None:
    """Codes for positions [start_pos, start_pos + n) from k_new, v_new [B][Hkv][n][128]."""
    n_new = k_new.shape[2]
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    _check(lib().vqkv_quantize_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), n_new,
                                      start_pos, _ptr(smooth), _ptr(k_book), _ptr(v_book), _ptr(k_codes),
                                      _ptr(v_codes), _stream(k_new)))


def decode_attention(shape: Shape, q_prime, k_book, v_book, k_codes, v_codes, seq_len: int, num_splits: int,
                     workspace, sm_scale: float | None = None) -> None:
    """Split-context attention over the codes; partials go to `workspace`."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(lib().vqkv_decode_attention(ctypes.byref(shape), _ptr(q_prime), _ptr(k_book), _ptr(v_book),
                                       _ptr(k_codes), _ptr(v_codes), seq_len, sm_scale, num_splits,
                                       _ptr(workspace), _stream(q_prime)))


def measure_decode_attention(shape: Shape, q_prime, k_book, v_book, k_codes, v_codes, seq_len: int,
                             num_splits: int, workspace, path: str, sm_scale: float | None = None) -> None:
    """decode_attention on a kernel chosen for measurement: 'default', 'table', 'gather' or 'mfma'."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if path not in DECODE_PATHS:
        raise ValueError(f"unknown decode path {path!r}")
    _check(lib().vqkv_measure_decode_attention(ctypes.byref(shape), _ptr(q_prime), _ptr(k_book), _ptr(v_book),
                                               _ptr(k_codes), _ptr(v_codes), seq_len, sm_scale, num_splits,
                                               _ptr(workspace), DECODE_PATHS[path], _stream(q_prime)))


def decode_attention_varlen(shape: Shape, q_prime, k_book, v_book, k_codes, v_codes, seq_lens, max_seq_len: int,
                            num_splits: int, workspace, sm_scale: float | None = None) -> None:
    """Ragged batch: sequence b holds seq_lens[b] tokens (int32 device tensor [B])."""
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    _check(lib().vqkv_decode_attention_varlen(ctypes.byref(shape), _ptr(q_prime), _ptr(k_book), _ptr(v_book),
                                              _ptr(k_codes), _ptr(v_codes), _ptr(seq_lens), max_seq_len, sm_scale,
                                              num_splits, _ptr(workspace), _stream(q_prime)))


def quantize_append_varlen(shape: Shape, k_new, v_new, positions, smooth, k_book, v_book, k_codes, v_codes) -> None:
    """One new token per sequence [B][Hkv][1][128], sequence b's at positions[b] (int32 device tensor)."""
    import torch
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype or k_new.shape[2] != 1:
        raise ValueError("k_new and v_new must both be [B][Hkv][1][128] of one dtype")
    if positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    _check(lib().vqkv_quantize_append_varlen(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                             _ptr(positions), _ptr(smooth), _ptr(k_book), _ptr(v_book),
                                             _ptr(k_codes), _ptr(v_codes), _stream(k_new)))


def decode_attention_paged(shape: Shape, q_prime, k_book, v_book, k_pool, v_pool, block_table, seq_lens,
                           max_seq_len: int, num_splits: int, workspace, sm_scale: float | None = None) -> None:
    """Paged cache: pools [num_blocks][64 * W] bytes, block_table int32 [B][Hkv][max_tokens / 64]."""
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    W = code_bytes_per_token(shape.fmt)
    num_blocks = k_pool.numel() // (64 * W)
    if v_pool.numel() // (64 * W) != num_blocks:
        raise ValueError("k_pool and v_pool must hold the same number of blocks")
    _check(lib().vqkv_decode_attention_paged(ctypes.byref(shape), _ptr(q_prime), _ptr(k_book), _ptr(v_book),
                                             _ptr(k_pool), _ptr(v_pool), num_blocks, _ptr(block_table),
                                             _ptr(seq_lens), max_seq_len, sm_scale, num_splits, _ptr(workspace),
                                             _stream(q_prime)))


def quantize_append_paged(shape: Shape, k_new, v_new, positions, smooth, k_book, v_book, k_pool, v_pool,
                          block_table) -> None:
    """One new token per sequence into a paged cache (see decode_attention_paged)."""
    import torch
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype or k_new.shape[2] != 1:
        raise ValueError("k_new and v_new must both be [B][Hkv][1][128] of one dtype")
    if positions.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("positions and block_table must be int32")
    W = code_bytes_per_token(shape.fmt)
    num_blocks = k_pool.numel() // (64 * W)
    _check(lib().vqkv_quantize_append_paged(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                            _ptr(positions), _ptr(smooth), _ptr(k_book), _ptr(v_book),
                                            _ptr(k_pool), _ptr(v_pool), num_blocks, _ptr(block_table),
                                            _stream(k_new)))


def combine(shape: Shape, num_splits: int, workspace, out) -> None:
    """Log-sum-exp merge of the splits into out [B][Hq][128] fp32."""
    _check(lib().vqkv_combine(ctypes.byref(shape), num_splits, _ptr(workspace), _ptr(out), _stream(out)))


def decode_step(shape: Shape, q, k_new, v_new, position: int, smooth, k_book, v_book, k_codes, v_codes,
                num_splits: int, workspace, out, sm_scale: float | None = None) -> None:
    """Append one token per sequence at `position`, then attention over [0, position] into out
    (one to three launches: the 2-bit attention appends the token itself, and with several splits a
    combine launch follows; bit-identical to quantize_append + transform_query + decode_attention +
    combine)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype or q.dtype != k_new.dtype:
        raise ValueError("q, k_new and v_new must share a dtype; k_new and v_new a shape")
    if k_new.shape[2] != 1:
        raise ValueError("decode_step appends one token per sequence")
    _check(lib().vqkv_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                  position, _ptr(smooth), _ptr(k_book), _ptr(v_book), _ptr(k_codes),
                                  _ptr(v_codes), sm_scale, num_splits, _ptr(workspace), _ptr(out), _stream(q)))


# Bytes of the static device workspace behind decode_step_static, on each GPU.
STATIC_SCRATCH_BYTES = 8 << 20


def decode_step_static(shape: Shape, q, k_new, v_new, position: int, smooth, k_book, v_book, k_codes, v_codes,
                       num_splits: int, out, sm_scale: float | None = None) -> None:
    """decode_step without a workspace argument: the library's static per-GPU scratch serves as
    the workspace, so nothing is allocated (calls overlapping on one GPU race on it)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _step_inputs(q, k_new, v_new)
    _check(lib().vqkv_decode_step_static(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                         position, _ptr(smooth), _ptr(k_book), _ptr(v_book), _ptr(k_codes),
                                         _ptr(v_codes), sm_scale, num_splits, _ptr(out), _stream(q)))


def torch_int32():
    import torch
    return torch.int32


def _step_inputs(q, k_new, v_new):
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype or q.dtype != k_new.dtype:
        raise ValueError("q, k_new and v_new must share a dtype; k_new and v_new a shape")
    if k_new.shape[2] != 1:
        raise ValueError("a decode step appends one token per sequence")


def decode_step_varlen(shape: Shape, q, k_new, v_new, positions, max_seq_len: int, smooth, k_book, v_book,
                       k_codes, v_codes, num_splits: int, workspace, out, sm_scale: float | None = None) -> None:
    """Ragged batches: sequence b appends at positions[b] (device int32) and attends to [0, positions[b]]."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _step_inputs(q, k_new, v_new)
    if positions.dtype != torch_int32():
        raise ValueError("positions must be int32")
    _check(lib().vqkv_decode_step_varlen(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                         _ptr(positions), max_seq_len, _ptr(smooth), _ptr(k_book), _ptr(v_book),
                                         _ptr(k_codes), _ptr(v_codes), sm_scale, num_splits, _ptr(workspace),
                                         _ptr(out), _stream(q)))


def decode_step_paged(shape: Shape, q, k_new, v_new, positions, max_seq_len: int, smooth, k_book, v_book,
                      k_pool, v_pool, block_table, num_splits: int, workspace, out,
                      sm_scale: float | None = None) -> None:
    """decode_step_varlen over a pool of 64-token code blocks named by block_table [B][Hkv][max_tokens / 64]."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _step_inputs(q, k_new, v_new)
    if positions.dtype != torch_int32() or block_table.dtype != torch_int32():
        raise ValueError("positions and block_table must be int32")
    W = code_bytes_per_token(shape.fmt)
    num_blocks = k_pool.numel() // (64 * W)
    if v_pool.numel() // (64 * W) != num_blocks:
        raise ValueError("k_pool and v_pool must hold the same number of blocks")
    _check(lib().vqkv_decode_step_paged(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                        _ptr(positions), max_seq_len, _ptr(smooth), _ptr(k_book), _ptr(v_book),
                                        _ptr(k_pool), _ptr(v_pool), num_blocks, _ptr(block_table), sm_scale,
                                        num_splits, _ptr(workspace), _ptr(out), _stream(q)))


def value_output_transform(shape: Shape, smooth, out) -> None:
    """Value-transform variant: out [B][Hq][128] <- s_v * (H out) in place (smooth [2][Hkv][128])."""
    _check(lib().vqkv_value_output_transform(ctypes.byref(shape), _ptr(smooth), _ptr(out), _stream(out)))


# ------------------------------------------------------------------- calibration

def smooth_scales(k_cal, smooth) -> None:
    """s[h][c] = sqrt(max_t |k_cal[h][t][c]|) for k_cal [Hkv][n][128]; smooth fp32 [Hkv][128] out."""
    hkv, n = k_cal.shape[0], k_cal.shape[1]
    _check(lib().vqkv_smooth_scales(hkv, n, _ptr(k_cal), _dtype_code(k_cal), _ptr(smooth), _stream(k_cal)))


def train_workspace_bytes(fmt: int, n_cal: int) -> int:
    return int(lib().vqkv_train_workspace_bytes(fmt, n_cal))


def train_codebook(fmt: int, rows, is_key: bool, smooth, init_idx, iters: int, book, workspace,
                   centroids=None) -> None:
    """K-Means codebook for one KV head from calibration rows [n][128] (see vqkv.h)."""
    n = rows.shape[0]
    _check(lib().vqkv_train_codebook(fmt, n, _ptr(rows), _dtype_code(rows), int(bool(is_key)),
                                     _ptr(smooth) if is_key else None, _ptr(init_idx), iters, _ptr(book),
                                     _ptr(centroids), _ptr(workspace), _stream(rows)))


# ------------------------------------------------------------------ a whole cache

@dataclass
class VQCache:
    """Device buffers of one layer's quantized cache plus the decode scratch.

    A convenience holder: it allocates with torch and calls the functions above.
    """
    shape: Shape
    smooth: "object"        # fp32 [Hkv][128]
    k_book: "object"        # fp16 bits (int16 tensor) [Hkv][E][dsub]
    v_book: "object"
    k_codes: "object"       # uint8 [B][Hkv][max_tokens * W]
    v_codes: "object"

    @staticmethod
    def allocate(shape: Shape, smooth, k_book, v_book, device) -> "VQCache":
        import torch
        W = code_bytes_per_token(shape.fmt)
        dims = (shape.batch, shape.num_kv_heads, shape.max_tokens * W)
        return VQCache(shape, smooth, k_book, v_book,
                       torch.zeros(dims, dtype=torch.uint8, device=device),
                       torch.zeros(dims, dtype=torch.uint8, device=device))

    def append(self, k_new, v_new, start_pos: int) -> None:
        quantize_append(self.shape, k_new, v_new, start_pos, self.smooth, self.k_book, self.v_book,
                        self.k_codes, self.v_codes)

    def attend(self, q, seq_len: int, num_splits: int | None = None, out=None, q_prime=None, workspace=None):
        import torch
        if num_splits is None:
            num_splits = suggest_splits(self.shape, seq_len)
        B, Hq = self.shape.batch, self.shape.num_q_heads
        if q_prime is None:
            q_prime = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(workspace_bytes(self.shape, num_splits), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
        transform_query(self.shape, q, self.smooth, q_prime)
        decode_attention(self.shape, q_prime, self.k_book, self.v_book, self.k_codes, self.v_codes, seq_len,
                         num_splits, workspace)
        combine(self.shape, num_splits, workspace, out)
        if self.shape.fmt & FMT_VALUE_TRANSFORM:
            value_output_transform(self.shape, self.smooth, out)
        return out

    def step(self, q, k_new, v_new, position: int, num_splits: int | None = None, out=None, workspace=None):
        """One decode step (decode_step's one to three launches): append k_new, v_new [B][Hkv][1][128] at `position`,
        then attend with q over tokens [0, position] (decode_step)."""
        import torch
        if num_splits is None:
            num_splits = suggest_splits(self.shape, position + 1)
        B, Hq = self.shape.batch, self.shape.num_q_heads
        if workspace is None:
            workspace = torch.empty(step_workspace_bytes(self.shape, num_splits), dtype=torch.uint8,
                                    device=q.device)
        if out is None:
            out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
        decode_step(self.shape, q, k_new, v_new, position, self.smooth, self.k_book, self.v_book, self.k_codes,
                    self.v_codes, num_splits, workspace, out)
        return out


# ------------------------------------------------------------- measurement only

def baseline_bf16_decode(shape: Shape, q, k, v, seq_len: int, num_splits: int, workspace,
                         sm_scale: float | None = None) -> None:
    """Unquantized bf16 decode (same splits and workspace format; merge with combine())."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    st = lib().vqkv_baseline_bf16_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), seq_len, sm_scale,
                                         num_splits, _ptr(workspace), _stream(q))
    if st != 0:
        raise VqkvError(st, lib().vqkv_baseline_last_error().decode())


def baseline_read_stream(buf, sink, blocks: int = 4096) -> None:
    """Read every byte of `buf` once (HBM read-bandwidth probe)."""
    nbytes = buf.numel() * buf.element_size()
    st = lib().vqkv_baseline_read_stream(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(buf))
    if st != 0:
        raise VqkvError(st, lib().vqkv_baseline_last_error().decode())
