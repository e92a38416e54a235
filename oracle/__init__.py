"""CPU oracle for decode attention over a vector-quantized KV cache (VecInfer).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  The arithmetic lives in
``vqkv_oracle.c`` (plain fp64 C, built with ``-ffp-contract=off``); this module
only marshals numpy arrays into it.  See that file's header for the passages of
the VecInfer pages each function follows and for the readings taken where the
pages are silent.

Parity status: every function here is pinned by CPU tests against something
other than itself (closed forms, textbook/library routines, brute force,
invariants); see ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vqkv_oracle.c")
_LIB = os.path.join(_HERE, "libvqkv_oracle.so")

HEAD_DIM = 128
FORMATS = {0: (256, 4), 1: (4096, 8), 2: (4096, 4), 3: (1024, 8), 4: (256, 2)}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        sig = {
            "vqo_format": (I, [P, P]),
            "vqo_half_to_double": (D, [ctypes.c_uint16]),
            "vqo_double_to_half": (ctypes.c_uint16, [D]),
            "vqo_hadamard": (None, [P]),
            "vqo_fwht": (None, [P]),
            "vqo_smooth_scales": (None, [P, I64, P]),
            "vqo_transform_key": (None, [P, P, P]),
            "vqo_transform_query": (None, [P, P, P]),
            "vqo_nearest": (I, [P, P, I, I]),
            "vqo_quantize": (I, [I, I64, P, P, P, P, P, P, P, P, I]),
            "vqo_kmeans": (None, [I64, I, I, P, P, I, P, P, I]),
            "vqo_attention": (I, [I, I, I, I, I64, P, P, P, P, P, P, P, D, P, I]),
            "vqo_value_output_transform": (None, [P, P]),
            "vqo_attention_fp": (I, [I, I, I, I64, P, P, P, D, P, I]),
            "vqo_pack_k": (I, [I, I64, P, P]),
            "vqo_unpack_k": (I, [I, I64, P, P]),
            "vqo_pack_v": (I, [I, I64, P, P]),
            "vqo_unpack_v": (I, [I, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def default_threads() -> int:
    """Threads for the oracle's parallel loops: the CPUs this process may run
    on, capped by a cgroup CPU quota and by OMP_NUM_THREADS when they are set."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, -(-int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint16))


# ------------------------------------------------------------------ scalar helpers

def half_to_double(bits: int) -> float:
    return lib().vqo_half_to_double(int(bits))


def double_to_half(x: float) -> int:
    return int(lib().vqo_double_to_half(float(x)))


def doubles_to_half(x: np.ndarray) -> np.ndarray:
    flat = np.asarray(x, dtype=np.float64).ravel()
    f = lib().vqo_double_to_half
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


# ---------------------------------------------------------------------- transforms

def hadamard() -> np.ndarray:
    H = np.zeros((HEAD_DIM, HEAD_DIM), dtype=np.float64)
    lib().vqo_hadamard(_p(H))
    return H


def fwht(x) -> np.ndarray:
    out = _f64(x).copy()
    lib().vqo_fwht(_p(out))
    return out


def smooth_scales(k_cal) -> np.ndarray:
    """k_cal: [n][128] -> s: [128] float32."""
    k = _f64(k_cal)
    s = np.zeros(HEAD_DIM, dtype=np.float32)
    lib().vqo_smooth_scales(_p(k), k.shape[0], _p(s))
    return s


def transform_key(k, s) -> np.ndarray:
    k, s = _f64(k), _f32(s)
    out = np.zeros(HEAD_DIM, dtype=np.float64)
    lib().vqo_transform_key(_p(k), _p(s), _p(out))
    return out


def transform_query(q, s) -> np.ndarray:
    q, s = _f64(q), _f32(s)
    out = np.zeros(HEAD_DIM, dtype=np.float64)
    lib().vqo_transform_query(_p(q), _p(s), _p(out))
    return out


def transform_keys(k, s) -> np.ndarray:
    """Row-wise transform_key for k [n][128]."""
    k = _f64(k)
    return np.stack([transform_key(row, s) for row in k]) if len(k) else np.zeros((0, HEAD_DIM))


# ---------------------------------------------------------------- nearest centroid

def nearest(x, book) -> int:
    """book: fp64 [E][dsub]."""
    x, book = _f64(x), _f64(book)
    return lib().vqo_nearest(_p(x), _p(book), book.shape[0], book.shape[1])


def quantize(fmt: int, k, v, s, kbook16, vbook16, nthreads: int | None = None, sv=None):
    """k, v: [n][128]; s: [128]; books fp16 bits [E][dsub].  Returns (kcodes, vcodes) [n][J] uint16.
    sv: [128] value scales of the value-transform variant (values quantized as H (v / sv)), or None."""
    E, dsub = FORMATS[fmt]
    k, v, s = _f64(k), _f64(v), _f32(s)
    sv = None if sv is None else _f32(sv)
    kb, vb = _u16(kbook16), _u16(vbook16)
    assert kb.shape == (E, dsub) and vb.shape == (E, dsub)
    n = k.shape[0]
    J = HEAD_DIM // dsub
    kc = np.zeros((n, J), dtype=np.uint16)
    vc = np.zeros((n, J), dtype=np.uint16)
    rc = lib().vqo_quantize(fmt, n, _p(k), _p(v), _p(s), None if sv is None else _p(sv), _p(kb), _p(vb),
                            _p(kc), _p(vc),
                            nthreads or default_threads())
    assert rc == 0
    return kc, vc


def kmeans(points, init_idx, iters: int = 20, nthreads: int | None = None):
    """Lloyd's K-Means from the given initial point indices.  Returns (fp64 centroids, assignment)."""
    pts = _f64(points)
    init = np.ascontiguousarray(np.asarray(init_idx, dtype=np.int64))
    n, dsub = pts.shape
    E = init.shape[0]
    cent = np.zeros((E, dsub), dtype=np.float64)
    assign = np.zeros(n, dtype=np.int32)
    lib().vqo_kmeans(n, dsub, E, _p(pts), _p(init), iters, _p(cent), _p(assign),
                     nthreads or default_threads())
    return cent, assign


# ----------------------------------------------------------------------- attention

def attention(fmt: int, q, s, kbook16, vbook16, kcodes, vcodes, sm_scale: float | None = None,
              nthreads: int | None = None, sv=None) -> np.ndarray:
    """q [B][Hq][128]; s [Hkv][128]; books [Hkv][E][dsub] fp16 bits; codes [B][Hkv][T][J].
    sv: [Hkv][128] value scales of the value-transform variant (output mapped back), or None."""
    q, s = _f64(q), _f32(s)
    sv = None if sv is None else _f32(sv)
    kb, vb, kc, vc = _u16(kbook16), _u16(vbook16), _u16(kcodes), _u16(vcodes)
    B, Hq, _ = q.shape
    _, Hkv, T, J = kc.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    out = np.zeros((B, Hq, HEAD_DIM), dtype=np.float64)
    rc = lib().vqo_attention(fmt, B, Hq, Hkv, T, _p(q), _p(s), None if sv is None else _p(sv), _p(kb), _p(vb),
                             _p(kc), _p(vc),
                             float(sm_scale), _p(out), nthreads or default_threads())
    assert rc == 0
    return out


def value_output_transform(o, sv) -> np.ndarray:
    """o [128] -> sv * (H o): the inverse of the value transform v' = H (v / sv)."""
    x = np.array(_f64(o), dtype=np.float64, copy=True)
    lib().vqo_value_output_transform(_p(x), _p(_f32(sv)))
    return x


def attention_fp(q, k, v, sm_scale: float | None = None, nthreads: int | None = None) -> np.ndarray:
    """Full-precision attention on raw k, v [B][Hkv][T][128]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, _ = q.shape
    _, Hkv, T, _ = k.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    out = np.zeros((B, Hq, HEAD_DIM), dtype=np.float64)
    rc = lib().vqo_attention_fp(B, Hq, Hkv, T, _p(q), _p(k), _p(v), float(sm_scale), _p(out),
                                nthreads or default_threads())
    assert rc == 0
    return out


# ------------------------------------------------------------------------- layouts

def code_bytes_per_token(fmt: int) -> int:
    return {0: 32, 1: 24, 2: 48, 3: 20, 4: 64}[fmt]


def pack_k(fmt: int, codes, cap: int, out: np.ndarray | None = None) -> np.ndarray:
    """codes [T][J] -> the library's key-code bytes for one (b, h) stream of capacity cap."""
    c = _u16(codes)
    if out is None:
        out = np.zeros(cap * code_bytes_per_token(fmt), dtype=np.uint8)
    assert lib().vqo_pack_k(fmt, c.shape[0], _p(c), _p(out)) == 0
    return out


def unpack_k(fmt: int, data, T: int) -> np.ndarray:
    E, dsub = FORMATS[fmt]
    d = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    out = np.zeros((T, HEAD_DIM // dsub), dtype=np.uint16)
    assert lib().vqo_unpack_k(fmt, T, _p(d), _p(out)) == 0
    return out


def pack_v(fmt: int, codes, cap: int, out: np.ndarray | None = None) -> np.ndarray:
    c = _u16(codes)
    if out is None:
        out = np.zeros(cap * code_bytes_per_token(fmt), dtype=np.uint8)
    assert lib().vqo_pack_v(fmt, c.shape[0], _p(c), _p(out)) == 0
    return out


def unpack_v(fmt: int, data, T: int) -> np.ndarray:
    E, dsub = FORMATS[fmt]
    d = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    out = np.zeros((T, HEAD_DIM // dsub), dtype=np.uint16)
    assert lib().vqo_unpack_v(fmt, T, _p(d), _p(out)) == 0
    return out


def pack_stream(fmt: int, kcodes, vcodes, cap: int):
    """codes [B][Hkv][T][J] -> (k bytes, v bytes) shaped [B][Hkv][cap * W]."""
    kc, vc = _u16(kcodes), _u16(vcodes)
    B, H, T, _ = kc.shape
    W = code_bytes_per_token(fmt)
    kb = np.zeros((B, H, cap * W), dtype=np.uint8)
    vb = np.zeros((B, H, cap * W), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            pack_k(fmt, kc[b, h], cap, kb[b, h])
            pack_v(fmt, vc[b, h], cap, vb[b, h])
    return kb, vb


# ----------------------------------------------------------------------- codebooks

def train_codebooks(fmt: int, k_cal, v_cal, s, init_k, init_v, iters: int = 20,
                    nthreads: int | None = None):
    """Offline codebooks for one KV head: K-Means on the transformed key sub-vectors
    and on the raw value sub-vectors; returns fp16 bit patterns [E][dsub] for K and V."""
    E, dsub = FORMATS[fmt]
    xk = transform_keys(k_cal, s).reshape(-1, dsub)
    xv = _f64(v_cal).reshape(-1, dsub)
    ck, _ = kmeans(xk, init_k, iters, nthreads)
    cv, _ = kmeans(xv, init_v, iters, nthreads)
    return doubles_to_half(ck), doubles_to_half(cv)
