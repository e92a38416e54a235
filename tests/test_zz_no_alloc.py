"""The allocation-free decode step (vqkv_decode_step_static) against
vqkv_decode_step with a caller's workspace: the same output bits and the same
cache bytes, on consecutive calls that share the static scratch (the second
smaller than the first, so it runs over what the first left there), and the
refusal of a step whose workspace exceeds the scratch."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import vector_quantized_bit_vqkv_amd as vq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _case(fmt, B, Hq, Hkv, pos, seed):
    """A cache of pos + 1 tokens' random codes plus one step's inputs."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    cap = ((pos + 1 + 63) // 64) * 64
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.5, 4.0, (Hkv, D)).astype(np.float32)
    kb = synth.random_fp16_book(seed, (Hkv, E, dsub), 0.6)
    vb = synth.random_fp16_book(seed + 1, (Hkv, E, dsub), 1.0)
    kc = synth.random_codes(seed, (B, Hkv, pos + 1, J), E)
    vc = synth.random_codes(seed + 1, (B, Hkv, pos + 1, J), E)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    q = _dev(rng.standard_normal((B, Hq, D)).astype(np.float32), torch.bfloat16)
    k_new = _dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    v_new = _dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    books = (_dev(kb.view(np.int16)), _dev(vb.view(np.int16)))
    return vq.make_shape(B, Hq, Hkv, cap, fmt), _dev(s), books, kbytes, vbytes, q, k_new, v_new


# Consecutive calls: (fmt, B, Hq, Hkv, position, splits); each list runs in order.
SEQUENCES = [
    [(0, 2, 32, 8, 4098, 9), (0, 1, 8, 2, 700, 3), (0, 1, 8, 2, 700, 1)],
    [(1, 2, 40, 8, 4098, 9), (1, 1, 10, 2, 700, 3)],
    [(2, 2, 32, 8, 3000, 5), (0, 1, 16, 2, 1000, 2), (1, 1, 5, 1, 129, 2)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["2bit", "1p5bit", "mixed"])
def test_static_step_equals_step_with_workspace(seq):
    for i, (fmt, B, Hq, Hkv, pos, S) in enumerate(seq):
        print(f"\n[case] static step call {i}: fmt{fmt} B{B} Hq{Hq} Hkv{Hkv} pos{pos} S{S}", flush=True)
        shape, sm, books, kbytes, vbytes, q, k_new, v_new = _case(fmt, B, Hq, Hkv, pos, 900 + 10 * i + fmt)
        assert vq.step_workspace_bytes(shape, S) <= vq.STATIC_SCRATCH_BYTES
        ref_k, ref_v, got_k, got_v = _dev(kbytes), _dev(vbytes), _dev(kbytes), _dev(vbytes)
        ws = torch.full((vq.step_workspace_bytes(shape, S),), 0xFF, dtype=torch.uint8, device=DEV)
        want = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        vq.decode_step(shape, q, k_new, v_new, pos, sm, books[0], books[1], ref_k, ref_v, S, ws, want)
        vq.decode_step_static(shape, q, k_new, v_new, pos, sm, books[0], books[1], got_k, got_v, S, got)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.isfinite(w).all()
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"call {i}: max diff {np.abs(g - w).max()}"
        assert torch.equal(got_k, ref_k) and torch.equal(got_v, ref_v), f"call {i}: cache bytes differ"


def test_static_step_refuses_a_workspace_beyond_the_scratch():
    """A batch-32, 32-head step at 64 splits needs ~34 MB of workspace: refused on
    the host with VQKV_ERR_UNSUPPORTED, before any device work."""
    B, Hq, Hkv, cap = 32, 32, 8, 8192
    shape = vq.make_shape(B, Hq, Hkv, cap, vq.FMT_2BIT)
    assert vq.step_workspace_bytes(shape, 64) > vq.STATIC_SCRATCH_BYTES
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    codes = torch.zeros((B, Hkv, cap * 32), dtype=torch.uint8, device=DEV)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
    sm = torch.ones((Hkv, D), dtype=torch.float32, device=DEV)
    book = torch.zeros((Hkv, 256, 4), dtype=torch.int16, device=DEV)
    with pytest.raises(vq.VqkvError) as e:
        vq.decode_step_static(shape, q, kv, kv, cap - 1, sm, book, book, codes, codes, 64, out)
    assert e.value.status == 2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and not codes.any()
    # The C ABI directly: the same status.
    st = vq.lib().vqkv_decode_step_static(ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(kv.data_ptr()), 0,
                                          cap - 1, ctypes.c_void_p(sm.data_ptr()), ctypes.c_void_p(book.data_ptr()),
                                          ctypes.c_void_p(book.data_ptr()), ctypes.c_void_p(codes.data_ptr()),
                                          ctypes.c_void_p(codes.data_ptr()), 0.088, 64,
                                          ctypes.c_void_p(out.data_ptr()), None)
    assert st == 2
