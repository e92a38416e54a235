"""GPU parity of the product path at the benchmark's full sizes.

The cache is built exactly as the benchmark builds it (``bench.Workload``):
keys, values, queries and calibration rows drawn on the device by ``synth``'s
seeded generator, smoothing scales and 20-iteration K-Means codebooks
calibrated on the GPU, every token of the context bulk-coded by
``vqkv_quantize_append``.  The bytes of the last token are then overwritten
with a fixed pattern and one ``vqkv_decode_step`` at the last position runs in
the benchmark's launch configuration (``vqkv_suggest_splits``), on the same
cache buffer and workspace the benchmark times: one launch at batch 32, the
fused-append attention plus the combine launch at batch 1 (32 splits), the
append launch plus the attention with its counter-fused combine for the
1.5-bit Qwen-shaped cache (4 splits).

For a seeded sample of (b, KV head) slices the oracle then recomputes
everything from the drawn inputs alone (arXiv 2510.06175 page, technical
framework stages 2-3; VecInfer card, Summary): the smoothing scales and the
codebooks (bit-exact against the GPU's), the codes of every token of the
slice, the step's appended token included (bit-exact against the cache), and
the attention of the step's queries over the whole context (within 2e-3 of the
step's output).  No oracle input comes from the library: the GPU's scales and
books are compared with the oracle's, and the oracle then runs on its own.

Runtime on the GPU machine (16 host threads for the oracle): about 20 s for the
whole file, most of it the oracle's 1.5-bit codebooks and codes.
"""
import os
import time

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import bench  # noqa: E402
import vector_quantized_bit_vqkv_amd as vq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
D = 128
PATTERN = 0xA5


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def rel_err(got, ref):
    """Per (b, g): max|got - ref| / max|ref|; returns the worst."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())


def last_token_value_bits(fmt, E, J):
    """Bytes, inside a 64-token value block, that hold bits of the block's last
    token, and the mask of its bits in each: what the oracle's packing sets
    when only that token has nonzero codes (E - 1 sets every bit of each of
    its codes).  In the 1.25-bit layout a byte can hold bits of two tokens."""
    probe = np.zeros((64, J), dtype=np.uint16)
    probe[63] = E - 1
    packed = oracle.pack_v(fmt, probe, 64)
    pos = np.nonzero(packed)[0]
    return pos, packed[pos]


# (workload, number of sampled (b, KV head) slices)
PRODUCT = [("llama8b_b32_t196k", 4), ("llama8b_b1_t196k", 8), ("llama8b_b1_t32k", 8),
           ("qwen14b_b8_t128k_1p5", 2), ("qwen14b_b8_t128k_1p25", 2), ("llama8b_b8_t196k_4bit", 2)]


@pytest.mark.parametrize("name,nsamp", PRODUCT)
def test_product_step_at_full_size(name, nsamp):
    say(f"product step at full size: {name}")
    t_start = time.time()
    torch.cuda.set_device(DEV)
    wk = bench.Workload(name, torch.device(DEV), keep_bf16=False, keep_inputs=True)
    wl, case, seed = wk.wl, wk.case, wk.seed
    fmt, B, Hq, Hkv, T = wl.fmt, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len
    E, dsub = oracle.FORMATS[fmt]
    J, G = D // dsub, Hq // Hkv
    W = vq.code_bytes_per_token(fmt)
    kc_dev, vc_dev = wk.caches[0]

    # The step must write the new token's codes itself: overwrite its bits
    # (only its own: other tokens' bits sharing a byte keep their values).
    kc_dev[:, :, (T - 1) * W:] = PATTERN
    pos, bits = last_token_value_bits(fmt, E, J)
    vpos = torch.from_numpy(pos + (T - 64) * W).to(DEV)
    mask = torch.from_numpy(bits).to(DEV)
    vc_dev[:, :, vpos] = (vc_dev[:, :, vpos] & ~mask) | (PATTERN & mask)
    torch.cuda.synchronize()
    wk.fused_step(0)                 # decode_step on caches[0], as the timed loop calls it
    torch.cuda.synchronize()
    out = wk.out.cpu().numpy()
    smooth_gpu = wk.smooth.cpu().numpy()
    kb_gpu = wk.k_book.cpu().numpy().view(np.uint16)
    vb_gpu = wk.v_book.cpu().numpy().view(np.uint16)
    gpu_s = time.time() - t_start
    print(f"  S={wk.S}; cache built and stepped in {gpu_s:.1f} s", flush=True)

    # The oracle from the drawn inputs alone.
    t0 = time.time()
    k_cal = case["k_cal"].float().cpu().numpy()
    v_cal = case["v_cal"].float().cpu().numpy()
    q = case["q"].float().cpu().numpy()
    n_cal = k_cal.shape[1]
    s_ref = np.stack([oracle.smooth_scales(k_cal[h]) for h in range(Hkv)])
    assert np.array_equal(smooth_gpu, s_ref), "smoothing scales differ from the oracle's"
    slices = [(b, h) for b in range(B) for h in range(Hkv)]
    pick = [slices[i] for i in np.random.default_rng(seed).permutation(len(slices))[:nsamp]]
    books = {}
    worst = 0.0
    for b, h in pick:
        if h not in books:
            ik = synth.kmeans_init_indices(seed + 2 * h, n_cal * J, E)
            iv = synth.kmeans_init_indices(seed + 2 * h + 1, n_cal * J, E)
            kb_ref, vb_ref = oracle.train_codebooks(fmt, k_cal[h], v_cal[h], s_ref[h], ik, iv, iters=20)
            assert np.array_equal(kb_gpu[h], kb_ref), f"key codebook of head {h} differs from the oracle's"
            assert np.array_equal(vb_gpu[h], vb_ref), f"value codebook of head {h} differs from the oracle's"
            books[h] = (kb_ref, vb_ref)
        kb_ref, vb_ref = books[h]
        k = case["k"][b, h].float().cpu().numpy()
        v = case["v"][b, h].float().cpu().numpy()
        kc_ref, vc_ref = oracle.quantize(fmt, k, v, s_ref[h], kb_ref, vb_ref)
        del k, v
        gk = oracle.unpack_k(fmt, kc_dev[b, h].cpu().numpy(), T)
        gv = oracle.unpack_v(fmt, vc_dev[b, h].cpu().numpy(), T)
        bad_k = np.nonzero((gk != kc_ref).any(axis=1))[0]
        bad_v = np.nonzero((gv != vc_ref).any(axis=1))[0]
        assert bad_k.size == 0, f"(b={b}, h={h}): key codes differ at {bad_k.size} tokens, first {bad_k[:8]}"
        assert bad_v.size == 0, f"(b={b}, h={h}): value codes differ at {bad_v.size} tokens, first {bad_v[:8]}"
        ref = oracle.attention(fmt, q[b:b + 1, h * G:(h + 1) * G], s_ref[h:h + 1], kb_ref[None], vb_ref[None],
                               kc_ref[None, None], vc_ref[None, None])
        err = rel_err(out[b:b + 1, h * G:(h + 1) * G], ref)
        worst = max(worst, err)
        print(f"  (b={b}, h={h}): {T} tokens' codes bit-exact, step output error {err:.3e}", flush=True)
    print(f"  worst {worst:.3e} over {len(pick)} slices; oracle {time.time() - t0:.1f} s", flush=True)
    assert worst <= TOL
    del wk, case
    torch.cuda.empty_cache()
