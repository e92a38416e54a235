"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: codes, smoothing scales and codebooks bit-exact; attention outputs
within 2e-3 max relative error, measured per (b, q-head) as
max|o_gpu - o_ref| / max|o_ref|; the query transform within the fp32 bound
derived below.  Inputs come from ``synth`` (seeded) or from torch's seeded
device generator; no oracle input comes from the HIP path.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import vector_quantized_bit_vqkv_amd as vq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
D = 128


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def book_dev(bits):
    return dev(np.ascontiguousarray(bits).view(np.int16))


def rel_err(got, ref):
    """Per (b, g): max|got - ref| / max|ref|; returns the worst."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())


def run_decode(shape, q_prime, kb, vb, kc, vc, T, S, path=None):
    ws = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    out = torch.empty((shape.batch, shape.num_q_heads, D), dtype=torch.float32, device=DEV)
    if path:
        vq.measure_decode_attention(shape, q_prime, kb, vb, kc, vc, T, S, ws, path)
    else:
        vq.decode_attention(shape, q_prime, kb, vb, kc, vc, T, S, ws)
    vq.combine(shape, S, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()



def _oracle_step_codes(fmt, kc, vc, pos, k_new, v_new, s, kb, vb, sv=None):
    """The oracle's codes of each sequence's appended token (k_new, v_new
    [B][Hkv][1][128] device tensors, the drawn inputs), written into the
    oracle-side code arrays kc, vc [B][Hkv][T][J] at position pos[b]; a
    position outside [0, T) is skipped."""
    kn, vn = k_new.float().cpu().numpy(), v_new.float().cpu().numpy()
    for b, p in enumerate(pos):
        if p < 0 or p >= kc.shape[2]:
            continue
        for h in range(kn.shape[1]):
            a, c = oracle.quantize(fmt, kn[b, h], vn[b, h], s[h], kb[h], vb[h], sv=None if sv is None else sv[h])
            kc[b, h, p], vc[b, h, p] = a[0], c[0]


def _assert_cache_codes(fmt, gk, gv, kc, vc, lens):
    """The cache bytes gk, gv [B][Hkv][cap * W] (host) hold the oracle's codes
    kc, vc for tokens [0, lens[b]) of every sequence."""
    for b, T in enumerate(lens):
        for h in range(kc.shape[1]):
            if T <= 0:
                continue
            assert np.array_equal(oracle.unpack_k(fmt, gk[b, h], T), kc[b, h, :T]), f"key codes b={b} h={h}"
            assert np.array_equal(oracle.unpack_v(fmt, gv[b, h], T), vc[b, h, :T]), f"value codes b={b} h={h}"


# ------------------------------------------------------------------ query transform

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,Hq,Hkv", [(1, 4, 1), (3, 32, 8), (2, 40, 8), (1, 8, 8)])
def test_transform_query(dtype, B, Hq, Hkv):
    say(f"transform_query {dtype} B{B} Hq{Hq} Hkv{Hkv}")
    rng = np.random.default_rng(B * 100 + Hq)
    q = synth.normal_numpy(rng, (B, Hq, D), dtype)
    s = rng.uniform(0.3, 8.0, (Hkv, D)).astype(np.float32)
    shape = vq.make_shape(B, Hq, Hkv, 64, 0)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q, torch.bfloat16 if dtype == "bf16" else torch.float32), dev(s), qp)
    got = qp.cpu().numpy()
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hq):
            h = g // G
            ref = oracle.transform_query(q[b, g], s[h])
            # fp32: one rounding in q*s, seven butterfly stages and the scale, each
            # at most 2^-24 relative, and H is orthogonal, so the error norm stays
            # below 10 * 2^-24 * ||q * s||.
            bound = 10 * 2.0 ** -24 * np.linalg.norm(q[b, g].astype(np.float64) * s[h])
            assert np.abs(got[b, g] - ref).max() <= bound


# ------------------------------------------------------------------- calibration

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_smooth_scales_bit_exact(dtype):
    say(f"smooth_scales {dtype}")
    case = synth.make_cpu_case(synth.dataclasses.replace(synth.WORKLOADS["llama8b_b1_t32k"], dtype=dtype), 3,
                               seq_len=1, n_cal=777)
    out = torch.empty((8, D), dtype=torch.float32, device=DEV)
    vq.smooth_scales(dev(case.k_cal, torch.bfloat16 if dtype == "bf16" else torch.float32), out)
    got = out.cpu().numpy()
    for h in range(8):
        assert np.array_equal(got[h], oracle.smooth_scales(case.k_cal[h]))


@pytest.mark.parametrize("fmt,n_cal,iters", [(0, 1024, 20), (1, 512, 4), (2, 256, 4), (3, 256, 6), (4, 512, 8)])
@pytest.mark.parametrize("is_key", [True, False])
def test_train_codebook_bit_exact(fmt, n_cal, iters, is_key):
    say(f"train_codebook fmt{fmt} n_cal{n_cal} iters{iters} key{is_key}")
    E, dsub = oracle.FORMATS[fmt]
    case = synth.make_cpu_case(synth.WORKLOADS["llama8b_b1_t32k"], 4, seq_len=1, n_cal=n_cal)
    rows = case.k_cal[0] if is_key else case.v_cal[0]
    s = oracle.smooth_scales(case.k_cal[0])
    init = synth.kmeans_init_indices(5 + fmt, n_cal * (D // dsub), E)
    pts = (oracle.transform_keys(rows, s) if is_key else rows.astype(np.float64)).reshape(-1, dsub)
    cent_ref, _ = oracle.kmeans(pts, init, iters)
    book_ref = oracle.doubles_to_half(cent_ref)
    book = torch.empty((E, dsub), dtype=torch.int16, device=DEV)
    cent = torch.empty((E, dsub), dtype=torch.float64, device=DEV)
    ws = torch.empty(vq.train_workspace_bytes(fmt, n_cal), dtype=torch.uint8, device=DEV)
    vq.train_codebook(fmt, dev(rows, torch.bfloat16), is_key, dev(s), dev(init), iters, book, ws, cent)
    torch.cuda.synchronize()
    assert np.array_equal(cent.cpu().numpy().view(np.uint64), cent_ref.view(np.uint64))
    assert np.array_equal(book.cpu().numpy().view(np.uint16), book_ref)


# -------------------------------------------------------------------- quantizer

def _quant_case(fmt, B, Hkv, n, dtype, seed):
    E, dsub = oracle.FORMATS[fmt]
    wl = synth.dataclasses.replace(synth.WORKLOADS["llama8b_b1_t32k"], num_kv_heads=Hkv, num_q_heads=Hkv,
                                   dtype=dtype)
    case = synth.make_cpu_case(wl, seed, seq_len=n, n_cal=256, batch=B)
    s = np.stack([oracle.smooth_scales(case.k_cal[h]) for h in range(Hkv)])
    # Books drawn near the data's scale; parity does not depend on book quality.
    kb = synth.random_fp16_book(seed, (Hkv, E, dsub), 0.5)
    vb = synth.random_fp16_book(seed + 1, (Hkv, E, dsub), 1.0)
    return case, s, kb, vb


def _oracle_codes(fmt, case, s, kb, vb):
    B, Hkv, n, _ = case.k.shape
    J = D // oracle.FORMATS[fmt][1]
    kc = np.zeros((B, Hkv, n, J), np.uint16)
    vc = np.zeros((B, Hkv, n, J), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            kc[b, h], vc[b, h] = oracle.quantize(fmt, case.k[b, h], case.v[b, h], s[h], kb[h], vb[h])
    return kc, vc


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_append_bit_exact_with_ragged_appends(fmt, dtype):
    """A prefill of 37 tokens at 0, then appends of 1, 2, 1, 17 and 64 tokens at
    odd and even positions; every code bit-exact and every byte outside the
    appended positions untouched (the 1.5-bit value rows share a byte between
    neighbouring tokens)."""
    say(f"quantize_append fmt{fmt} {dtype}")
    B, Hkv, cap = 2, 3, 192
    pieces = [(0, 37), (37, 1), (38, 2), (40, 1), (41, 17), (58, 64)]
    n = 122
    case, s, kb, vb = _quant_case(fmt, B, Hkv, n, dtype, 40 + fmt)
    kc_ref, vc_ref = _oracle_codes(fmt, case, s, kb, vb)
    shape = vq.make_shape(B, Hkv, Hkv, cap, fmt)
    W = vq.code_bytes_per_token(fmt)
    sentinel = np.random.default_rng(1).integers(0, 256, (B, Hkv, cap * W), dtype=np.uint8)
    kcodes, vcodes = dev(sentinel), dev(sentinel)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for start, cnt in pieces:
        k_new = dev(case.k[:, :, start:start + cnt], tdt).contiguous()
        v_new = dev(case.v[:, :, start:start + cnt], tdt).contiguous()
        vq.quantize_append(shape, k_new, v_new, start, dev(s), book_dev(kb), book_dev(vb), kcodes, vcodes)
    torch.cuda.synchronize()
    gk, gv = kcodes.cpu().numpy(), vcodes.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            assert np.array_equal(oracle.unpack_k(fmt, gk[b, h], n), kc_ref[b, h])
            assert np.array_equal(oracle.unpack_v(fmt, gv[b, h], n), vc_ref[b, h])
            # Bytes of positions >= n keep the sentinel: repack the reference over it.
            expect_k = oracle.pack_k(fmt, kc_ref[b, h], cap, sentinel[b, h].copy())
            expect_v = oracle.pack_v(fmt, vc_ref[b, h], cap, sentinel[b, h].copy())
            assert np.array_equal(gk[b, h], expect_k)
            assert np.array_equal(gv[b, h], expect_v)


VT = vq.FMT_VALUE_TRANSFORM


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_value_transform_append_bit_exact(fmt):
    """Value-transform variant: bulk appends (2-bit exact scan, 1.5-bit screen)
    and one-token appends code the values as H (v / s_v), bit-exact against the
    oracle (and not equal to the untransformed codes)."""
    say(f"value-transform append fmt{fmt}")
    B, Hkv, cap, n = 2, 3, 128, 70
    case, s, kb, vb = _quant_case(fmt, B, Hkv, n, "bf16", 60 + fmt)
    sv = np.stack([oracle.smooth_scales(case.v_cal[h]) for h in range(Hkv)])
    J = D // oracle.FORMATS[fmt][1]
    kc_ref = np.zeros((B, Hkv, n, J), np.uint16)
    vc_ref = np.zeros_like(kc_ref)
    vc_plain = np.zeros_like(kc_ref)
    for b in range(B):
        for h in range(Hkv):
            kc_ref[b, h], vc_ref[b, h] = oracle.quantize(fmt, case.k[b, h], case.v[b, h], s[h], kb[h], vb[h],
                                                         sv=sv[h])
            _, vc_plain[b, h] = oracle.quantize(fmt, case.k[b, h], case.v[b, h], s[h], kb[h], vb[h])
    assert not np.array_equal(vc_ref, vc_plain)
    shape = vq.make_shape(B, Hkv, Hkv, cap, fmt | VT)
    W = vq.code_bytes_per_token(fmt)
    kcodes = torch.zeros((B, Hkv, cap * W), dtype=torch.uint8, device=DEV)
    vcodes = torch.zeros_like(kcodes)
    smooth2 = dev(np.concatenate([s, sv]))
    for start, cnt in [(0, 64), (64, 1), (65, 5)]:
        k_new = dev(case.k[:, :, start:start + cnt], torch.bfloat16).contiguous()
        v_new = dev(case.v[:, :, start:start + cnt], torch.bfloat16).contiguous()
        vq.quantize_append(shape, k_new, v_new, start, smooth2, book_dev(kb), book_dev(vb), kcodes, vcodes)
    torch.cuda.synchronize()
    gk, gv = kcodes.cpu().numpy(), vcodes.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            assert np.array_equal(oracle.unpack_k(fmt, gk[b, h], n), kc_ref[b, h])
            assert np.array_equal(oracle.unpack_v(fmt, gv[b, h], n), vc_ref[b, h])


@pytest.mark.parametrize("fmt,S", [(0, 1), (0, 7), (1, 3), (2, 4), (3, 2), (4, 3)])
def test_value_transform_attention_matches_oracle(fmt, S):
    """Value-transform variant: transform_query + decode_attention + combine +
    value_output_transform against the oracle's attention with the output map."""
    say(f"value-transform attention fmt{fmt} S{S}")
    B, Hq, Hkv, T = 2, 8, 2, 1000
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 7000 + 10 * fmt + S)
    sv = np.random.default_rng(S).uniform(0.5, 3.0, (Hkv, D)).astype(np.float32)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt | VT)
    smooth2 = dev(np.concatenate([s, sv]))
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q), smooth2, qp)
    ws = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.decode_attention(shape, qp, book_dev(kb), book_dev(vb), dev(kbytes), dev(vbytes), T, S, ws)
    vq.combine(shape, S, ws, out)
    vq.value_output_transform(shape, smooth2, out)
    torch.cuda.synchronize()
    ref = oracle.attention(fmt, q, s, kb, vb, kc, vc, sv=sv)
    err = rel_err(out.cpu().numpy(), ref)
    print(f"  max relative error {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("fmt,S,paged", [(0, 1, False), (0, 6, False), (1, 1, False), (1, 4, False),
                                         (0, 5, True), (1, 3, True), (2, 3, False), (0, 1, True),
                                         (3, 1, False), (3, 4, True), (4, 1, False), (4, 3, True)])
def test_value_transform_step_equals_the_calls(fmt, S, paged):
    """Value-transform variant: decode_step (uniform) or decode_step_paged
    (ragged positions) against append + transform_query + decode + combine +
    value_output_transform: the same output bits and cache bytes; then the
    oracle with the output map on the cache as it ends up."""
    say(f"value-transform step fmt{fmt} S{S} paged={paged}")
    B, Hq, Hkv = 3, 8, 2
    pos = [777, 1500, 64] if paged else [1500] * B
    cap = ((max(pos) + 1 + 63) // 64) * 64
    W = vq.code_bytes_per_token(fmt)
    q, s, kb, vb, kc, vc, _ = _attn_inputs(fmt, B, Hq, Hkv, max(pos) + 1, 7100 + 10 * fmt + S, cap)
    sv = np.random.default_rng(S + 5).uniform(0.5, 3.0, (Hkv, D)).astype(np.float32)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt | VT)
    smooth2 = dev(np.concatenate([s, sv]))
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    if paged:
        kpool, vpool, table = _paged_pool(kbytes, vbytes, W, 71 + S)
        tab = torch.from_numpy(table).to(DEV)
        ref_k, ref_v, got_k, got_v = dev(kpool), dev(vpool), dev(kpool), dev(vpool)
    else:
        ref_k, ref_v, got_k, got_v = dev(kbytes), dev(vbytes), dev(kbytes), dev(vbytes)
    rng = np.random.default_rng(S)
    books = (book_dev(kb), book_dev(vb))
    qd = dev(rng.standard_normal((B, Hq, D)).astype(np.float32), torch.bfloat16)
    k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws_ref = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    ws = torch.full((vq.step_workspace_bytes(shape, S),), 0xFF, dtype=torch.uint8, device=DEV)
    want = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    mx = max(pos) + 1
    if paged:
        pos_d = torch.tensor(pos, dtype=torch.int32, device=DEV)
        lens_d = torch.tensor([p + 1 for p in pos], dtype=torch.int32, device=DEV)
        vq.quantize_append_paged(shape, k_new, v_new, pos_d, smooth2, books[0], books[1], ref_k, ref_v, tab)
        vq.transform_query(shape, qd, smooth2, qp)
        vq.decode_attention_paged(shape, qp, books[0], books[1], ref_k, ref_v, tab, lens_d, mx, S, ws_ref)
        vq.decode_step_paged(shape, qd, k_new, v_new, pos_d, mx, smooth2, books[0], books[1], got_k, got_v, tab, S,
                             ws, got)
    else:
        vq.quantize_append(shape, k_new, v_new, pos[0], smooth2, books[0], books[1], ref_k, ref_v)
        vq.transform_query(shape, qd, smooth2, qp)
        vq.decode_attention(shape, qp, books[0], books[1], ref_k, ref_v, mx, S, ws_ref)
        vq.decode_step(shape, qd, k_new, v_new, pos[0], smooth2, books[0], books[1], got_k, got_v, S, ws, got)
    vq.combine(shape, S, ws_ref, want)
    vq.value_output_transform(shape, smooth2, want)
    torch.cuda.synchronize()
    g, w = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"max diff {np.abs(g - w).max()}"
    assert torch.equal(got_k, ref_k) and torch.equal(got_v, ref_v)
    gk, gv = got_k.cpu().numpy(), got_v.cpu().numpy()
    if paged:
        nb = cap // 64
        gk = np.stack([np.stack([np.concatenate([gk[table[b, h, i]] for i in range(nb)]) for h in range(Hkv)])
                       for b in range(B)])
        gv = np.stack([np.stack([np.concatenate([gv[table[b, h, i]] for i in range(nb)]) for h in range(Hkv)])
                       for b in range(B)])
    # The oracle codes the appended tokens itself; the cache must hold its codes.
    _oracle_step_codes(fmt, kc, vc, pos, k_new, v_new, s, kb, vb, sv)
    _assert_cache_codes(fmt, gk, gv, kc, vc, [p + 1 for p in pos])
    qf = qd.float().cpu().numpy()
    for b, p in enumerate(pos):
        T = p + 1
        ref = oracle.attention(fmt, qf[b:b + 1], s, kb, vb, kc[b:b + 1, :, :T], vc[b:b + 1, :, :T], sv=sv)
        err = rel_err(g[b:b + 1], ref)
        print(f"  b={b} T={T} max relative error {err:.3e}", flush=True)
        assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_ties_go_to_lowest_index(fmt):
    """Duplicate codebook entries and values exactly halfway between two entries."""
    say(f"quantize ties fmt{fmt}")
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(7)
    kb = synth.random_fp16_book(3, (1, E, dsub), 0.5)
    kb[0, 200] = kb[0, 17]                                      # duplicate: 17 must win over 200
    vb = np.zeros((1, E, dsub), np.float16)
    vb[0, :, 0] = np.arange(E, dtype=np.float64) * 0.25          # entries 0, .25, .5, ... on dim 0
    vb[0, E - 1] = vb[0, 5]                                     # the last entry duplicates entry 5
    vb = vb.view(np.uint16)
    n = 64
    v = np.zeros((n, D), np.float32)
    v[:, ::dsub] = (rng.integers(0, 200, (n, J)) * 0.25 + 0.125).astype(np.float32)   # exact midpoints
    v[:4, 0] = 1.25                                             # exactly entries 5 and E - 1: 5 wins
    k = rng.standard_normal((n, D)).astype(np.float32)
    s = np.ones(D, np.float32)
    kc_ref, vc_ref = oracle.quantize(fmt, k, v, s, kb[0], vb[0])
    shape = vq.make_shape(1, 1, 1, 64, fmt)
    kcodes = torch.zeros((1, 1, 64 * vq.code_bytes_per_token(fmt)), dtype=torch.uint8, device=DEV)
    vcodes = torch.zeros_like(kcodes)
    vq.quantize_append(shape, dev(k[None, None]), dev(v[None, None]), 0, dev(s[None]), book_dev(kb),
                       book_dev(vb), kcodes, vcodes)
    torch.cuda.synchronize()
    gk = oracle.unpack_k(fmt, kcodes[0, 0].cpu().numpy(), n)
    gv = oracle.unpack_v(fmt, vcodes[0, 0].cpu().numpy(), n)
    assert np.array_equal(gk, kc_ref) and np.array_equal(gv, vc_ref)
    assert not np.any(gk == 200)
    # Halfway between entries m and m+1 the lower index wins; of two equal entries, the lower.
    expect = (v[:, ::dsub] / 0.25 - 0.5).astype(np.uint16)
    expect[:4, 0] = 5
    assert np.array_equal(gv, expect)
    # The same tokens appended one at a time (the per-step append path).
    kcodes1 = torch.zeros_like(kcodes)
    vcodes1 = torch.zeros_like(kcodes)
    for t in range(9):
        vq.quantize_append(shape, dev(k[None, None, t:t + 1]), dev(v[None, None, t:t + 1]), t, dev(s[None]),
                           book_dev(kb), book_dev(vb), kcodes1, vcodes1)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.unpack_k(fmt, kcodes1[0, 0].cpu().numpy(), 9), kc_ref[:9])
    assert np.array_equal(oracle.unpack_v(fmt, vcodes1[0, 0].cpu().numpy(), 9), vc_ref[:9])


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_near_ties_below_fp32_resolution(fmt):
    """Keys whose rotated sub-vectors sit at the midpoint of two codebook
    entries one fp16 ulp apart (up to the fp32 rounding of k): the two
    distances agree to far below fp32 resolution, so only fp64 tells them
    apart.  The codes, one token at a time and in bulk, equal the oracle's;
    a plain fp32 argmin would miss many of them (counted on the host)."""
    say(f"quantize near ties fmt{fmt}")
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(31 + fmt)
    half = E // 2
    base = (rng.standard_normal((half, dsub)) * 0.5).astype(np.float16)
    base[:, 0] = np.abs(base[:, 0]) + np.float16(0.25)           # positive: next entry up is one ulp larger
    up = base.copy()
    up[:, 0] = np.nextafter(base[:, 0], np.float16(np.inf))
    kb = np.concatenate([base, up]).view(np.uint16)[None]         # entry e + E/2 = entry e, one ulp up on dim 0
    n = 48
    pick = rng.integers(0, half, (n, J))
    xt = base[pick].astype(np.float64)                            # (n, J, dsub)
    xt[:, :, 0] = 0.5 * (base[pick, 0].astype(np.float64) + up[pick, 0].astype(np.float64))
    H = np.array([[1.0]])
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    H /= math.sqrt(D)
    s = rng.uniform(0.5, 2.0, D).astype(np.float32)
    k = ((xt.reshape(n, D) @ H) * s).astype(np.float32)          # H is symmetric and orthogonal
    v = rng.standard_normal((n, D)).astype(np.float32)
    vb = synth.random_fp16_book(41, (1, E, dsub), 1.0)
    kc_ref, vc_ref = oracle.quantize(fmt, k, v, s, kb[0], vb[0])
    # How many codes a plain fp32 argmin gets wrong: x rounded to fp32, fp32 distances.
    x32 = ((k.astype(np.float64) / s) @ H).reshape(n, J, dsub).astype(np.float32)
    cb32 = kb[0].view(np.float16).astype(np.float32)
    d32 = np.zeros((n, J, E), np.float32)
    for i in range(dsub):
        t = x32[:, :, None, i] - cb32[None, None, :, i]
        d32 = d32 + t * t
    miss = int(np.sum(np.argmin(d32, axis=-1) != kc_ref))
    print(f"  fp32 argmin differs from the exact code on {miss} of {n * J} sub-vectors", flush=True)
    assert miss >= 20
    shape = vq.make_shape(1, 1, 1, 64, fmt)
    W = vq.code_bytes_per_token(fmt)
    for mode in ("bulk", "one-token"):
        kcodes = torch.zeros((1, 1, 64 * W), dtype=torch.uint8, device=DEV)
        vcodes = torch.zeros_like(kcodes)
        if mode == "bulk":
            vq.quantize_append(shape, dev(k[None, None]), dev(v[None, None]), 0, dev(s[None]), book_dev(kb),
                               book_dev(vb), kcodes, vcodes)
        else:
            for t in range(n):
                vq.quantize_append(shape, dev(k[None, None, t:t + 1]), dev(v[None, None, t:t + 1]), t, dev(s[None]),
                                   book_dev(kb), book_dev(vb), kcodes, vcodes)
        torch.cuda.synchronize()
        assert np.array_equal(oracle.unpack_k(fmt, kcodes[0, 0].cpu().numpy(), n), kc_ref), mode
        assert np.array_equal(oracle.unpack_v(fmt, vcodes[0, 0].cpu().numpy(), n), vc_ref), mode


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_fallbacks_match_oracle(fmt):
    """Points the distance screen cannot take (coordinates beyond the fp16 range,
    NaN) go through the exact scan: codes still equal the oracle's, in the bulk
    and in the one-token path.  A NaN makes every distance NaN, so the lowest
    index, 0, is the code (the oracle's rule)."""
    say(f"quantize fallbacks fmt{fmt}")
    E, dsub = oracle.FORMATS[fmt]
    rng = np.random.default_rng(11 + fmt)
    n = 40
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    k[3] *= 3.0e5                     # |x| far beyond 2^15 after the transform
    v[5] *= 1.0e5
    v[7, 9] = np.nan                  # one value sub-vector
    k[11, 4] = np.nan                 # spreads over the whole rotated key
    v[13, :dsub] = 40000.0            # just past the fp16-safe range
    s = rng.uniform(0.5, 2.0, D).astype(np.float32)
    kb = synth.random_fp16_book(21, (1, E, dsub), 0.8)
    vb = synth.random_fp16_book(22, (1, E, dsub), 1.0)
    kc_ref, vc_ref = oracle.quantize(fmt, k, v, s, kb[0], vb[0])
    assert np.all(kc_ref[11] == 0) and vc_ref[7, 9 // dsub] == 0
    shape = vq.make_shape(1, 1, 1, 64, fmt)
    W = vq.code_bytes_per_token(fmt)
    for mode in ("bulk", "one-token"):
        kcodes = torch.zeros((1, 1, 64 * W), dtype=torch.uint8, device=DEV)
        vcodes = torch.zeros_like(kcodes)
        if mode == "bulk":
            vq.quantize_append(shape, dev(k[None, None]), dev(v[None, None]), 0, dev(s[None]), book_dev(kb),
                               book_dev(vb), kcodes, vcodes)
        else:
            for t in range(n):
                vq.quantize_append(shape, dev(k[None, None, t:t + 1]), dev(v[None, None, t:t + 1]), t, dev(s[None]),
                                   book_dev(kb), book_dev(vb), kcodes, vcodes)
        torch.cuda.synchronize()
        assert np.array_equal(oracle.unpack_k(fmt, kcodes[0, 0].cpu().numpy(), n), kc_ref), mode
        assert np.array_equal(oracle.unpack_v(fmt, vcodes[0, 0].cpu().numpy(), n), vc_ref), mode


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_degenerate_scales_match_oracle(fmt):
    """Smoothing scales are device data the library does not inspect (that would
    need a synchronizing copy).  A negative and an infinite scale (that channel
    becomes 0), a tiny one (rotated coordinates near 1e5: past the fp16 range of
    the screen, so the exact scan decides), and a zero one (infinite or NaN
    coordinates: every key code is 0, the lowest index) give the oracle's codes
    in the bulk and in the one-token path; values are not divided and keep
    ordinary codes."""
    say(f"quantize degenerate scales fmt{fmt}")
    E, dsub = oracle.FORMATS[fmt]
    rng = np.random.default_rng(31 + fmt)
    n = 24
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    k[4, 5] = 0.0                     # 0 / 0 = NaN in the second set
    base = rng.uniform(0.5, 2.0, D).astype(np.float32)
    s1, s2, s3 = base.copy(), base.copy(), base.copy()
    s1[9], s1[20] = -1.5, np.inf
    s2[33] = 1e-6
    s3[5] = 0.0
    kb = synth.random_fp16_book(41, (1, E, dsub), 0.8)
    vb = synth.random_fp16_book(42, (1, E, dsub), 1.0)
    shape = vq.make_shape(1, 1, 1, 64, fmt)
    W = vq.code_bytes_per_token(fmt)
    for s_ in (s1, s2, s3):
        kc_ref, vc_ref = oracle.quantize(fmt, k, v, s_, kb[0], vb[0])
        for mode in ("bulk", "one-token"):
            kcodes = torch.zeros((1, 1, 64 * W), dtype=torch.uint8, device=DEV)
            vcodes = torch.zeros_like(kcodes)
            if mode == "bulk":
                vq.quantize_append(shape, dev(k[None, None]), dev(v[None, None]), 0, dev(s_[None]), book_dev(kb),
                                   book_dev(vb), kcodes, vcodes)
            else:
                for t in range(n):
                    vq.quantize_append(shape, dev(k[None, None, t:t + 1]), dev(v[None, None, t:t + 1]), t,
                                       dev(s_[None]), book_dev(kb), book_dev(vb), kcodes, vcodes)
            torch.cuda.synchronize()
            assert np.array_equal(oracle.unpack_k(fmt, kcodes[0, 0].cpu().numpy(), n), kc_ref), mode
            assert np.array_equal(oracle.unpack_v(fmt, vcodes[0, 0].cpu().numpy(), n), vc_ref), mode


# ---------------------------------------------------------------------- attention

def _attn_inputs(fmt, B, Hq, Hkv, T, seed, cap=None):
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    cap = cap or ((T + 63) // 64) * 64
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    s = rng.uniform(0.5, 4.0, (Hkv, D)).astype(np.float32)
    kb = synth.random_fp16_book(seed, (Hkv, E, dsub), 0.6)
    vb = synth.random_fp16_book(seed + 1, (Hkv, E, dsub), 1.0)
    kc = synth.random_codes(seed, (B, Hkv, T, J), E)
    vc = synth.random_codes(seed + 1, (B, Hkv, T, J), E)
    return q, s, kb, vb, kc, vc, cap


def _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, S, path=None):
    B, Hq, _ = q.shape
    _, Hkv, T, _ = kc.shape
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q), dev(s), qp)
    return run_decode(shape, qp, book_dev(kb), book_dev(vb), dev(kbytes), dev(vbytes), T, S, path)


ATTN_CASES = [
    # fmt, B, Hq, Hkv, T, S, path
    (0, 1, 4, 1, 2048, 1, "table"),
    (0, 1, 4, 1, 2048, 32, "table"),
    (0, 1, 4, 1, 2048, 4, "gather"),
    (0, 2, 32, 8, 1, 1, None),
    (0, 2, 32, 8, 65, 2, None),
    (0, 1, 8, 8, 777, 5, "table"),
    (0, 1, 8, 8, 777, 5, "gather"),
    (0, 1, 6, 2, 1000, 3, "table"),
    (0, 2, 12, 4, 4099, 9, "table"),
    (0, 2, 12, 4, 4099, 9, "gather"),
    (0, 1, 16, 2, 333, 2, "gather"),       # G = 8
    (0, 1, 10, 2, 129, 3, "gather"),       # G = 5
    (0, 1, 4, 1, 2048, 1, "mfma"),
    (0, 1, 4, 1, 2048, 32, "mfma"),
    (0, 1, 8, 8, 777, 5, "mfma"),          # G = 1
    (0, 1, 6, 2, 1000, 3, "mfma"),         # G = 3
    (0, 2, 12, 4, 4099, 9, "mfma"),
    (0, 1, 16, 2, 333, 2, "mfma"),         # G = 8: two head blocks
    (0, 1, 10, 2, 129, 3, "mfma"),         # G = 5
    (0, 2, 32, 8, 1, 1, "mfma"),
    (1, 1, 40, 8, 1000, 4, None),          # G = 5: two head blocks
    (1, 2, 5, 1, 64, 1, None),
    (1, 1, 8, 1, 129, 3, None),            # G = 8
    (1, 1, 2, 2, 3001, 7, None),           # G = 1
    (1, 2, 12, 4, 4099, 9, None),          # G = 3, ragged tail
    (1, 1, 40, 8, 1000, 4, "gather"),
    (1, 1, 8, 1, 129, 3, "gather"),
    (1, 1, 2, 2, 3001, 7, "gather"),
    (2, 1, 4, 1, 2048, 1, None),           # 3-bit
    (2, 2, 32, 8, 4099, 9, None),          # ragged tail
    (2, 1, 8, 8, 777, 5, None),            # G = 1
    (2, 1, 16, 2, 333, 2, None),           # G = 8
    (2, 1, 10, 2, 129, 3, None),           # G = 5
    (2, 2, 32, 8, 1, 1, None),
    (3, 1, 40, 8, 1000, 4, None),          # 1.25-bit, G = 5: two head blocks
    (3, 2, 5, 1, 64, 1, None),
    (3, 1, 8, 1, 129, 3, None),            # G = 8
    (3, 1, 2, 2, 3001, 7, None),           # G = 1
    (3, 2, 12, 4, 4099, 9, None),          # G = 3, ragged tail
    (3, 2, 32, 8, 1, 1, None),
    (4, 1, 4, 1, 2048, 1, None),           # 4-bit
    (4, 2, 32, 8, 4099, 9, None),          # ragged tail
    (4, 1, 8, 8, 777, 5, None),            # G = 1
    (4, 1, 16, 2, 333, 2, None),           # G = 8
    (4, 1, 10, 2, 129, 3, None),           # G = 5
    (4, 2, 32, 8, 1, 1, None),
    (0, 1, 12, 2, 300, 2, None),           # G = 6
    (1, 1, 14, 2, 300, 3, None),           # G = 7
    (2, 1, 12, 2, 300, 1, None),           # G = 6
    (3, 1, 14, 2, 300, 2, None),           # G = 7
    (4, 1, 14, 2, 300, 3, None),           # G = 7
]


@pytest.mark.parametrize("fmt,B,Hq,Hkv,T,S,path", ATTN_CASES)
def test_decode_matches_oracle(fmt, B, Hq, Hkv, T, S, path):
    say(f"decode fmt{fmt} B{B} Hq{Hq} Hkv{Hkv} T{T} S{S} path={path}")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 1000 + T + Hq)
    got = _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, S, path)
    ref = oracle.attention(fmt, q, s, kb, vb, kc, vc)
    err = rel_err(got, ref)
    print(f"  max relative error {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("fmt,Hq,Hkv", [(0, 8, 2), (1, 10, 2), (2, 8, 2), (3, 10, 2), (4, 8, 2)])
@pytest.mark.parametrize("S", [1, 5, 64])
def test_decode_varlen_matches_oracle(fmt, Hq, Hkv, S):
    """Ragged batch: each sequence its own length (1, a ragged tail, the longest,
    and 0); the codes past a sequence's length belong to other data and must be
    ignored; a zero-length sequence gives a zero output."""
    lens = [1, 777, 4099, 0]
    B, T = len(lens), max(lens)
    say(f"decode varlen fmt{fmt} Hq{Hq} Hkv{Hkv} S{S} lens {lens}")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 500 + fmt)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q), dev(s), qp)
    ws = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    vq.decode_attention_varlen(shape, qp, book_dev(kb), book_dev(vb), dev(kbytes), dev(vbytes), seq, T, S, ws)
    vq.combine(shape, S, ws, out)
    got = out.cpu().numpy()
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(got[b] == 0.0)
            continue
        ref = oracle.attention(fmt, q[b:b + 1], s, kb, vb, kc[b:b + 1, :, :L], vc[b:b + 1, :, :L])
        err = rel_err(got[b:b + 1], ref)
        print(f"  b={b} L={L} max relative error {err:.3e}", flush=True)
        assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_append_varlen_bit_exact(fmt):
    """One token per sequence at its own position (odd, even, block edges);
    a position outside the cache leaves that sequence untouched; every other
    byte keeps its sentinel."""
    say(f"quantize_append varlen fmt{fmt}")
    B, Hkv, cap = 4, 2, 192
    positions = [0, 65, 130, cap]
    case, s, kb, vb = _quant_case(fmt, B, Hkv, 1, "bf16", 70 + fmt)
    kc_ref, vc_ref = _oracle_codes(fmt, case, s, kb, vb)
    shape = vq.make_shape(B, Hkv, Hkv, cap, fmt)
    W = vq.code_bytes_per_token(fmt)
    sentinel = np.random.default_rng(4).integers(0, 256, (B, Hkv, cap * W), dtype=np.uint8)
    kcodes, vcodes = dev(sentinel), dev(sentinel)
    pos = torch.tensor(positions, dtype=torch.int32, device=DEV)
    vq.quantize_append_varlen(shape, dev(case.k, torch.bfloat16), dev(case.v, torch.bfloat16), pos, dev(s),
                              book_dev(kb), book_dev(vb), kcodes, vcodes)
    torch.cuda.synchronize()
    gk, gv = kcodes.cpu().numpy(), vcodes.cpu().numpy()
    for b, t in enumerate(positions):
        for h in range(Hkv):
            if t >= cap:
                assert np.array_equal(gk[b, h], sentinel[b, h]) and np.array_equal(gv[b, h], sentinel[b, h])
                continue
            # Expected: the sentinel with this token's codes packed at position t.
            J = kc_ref.shape[-1]
            full_k = oracle.unpack_k(fmt, sentinel[b, h], cap)
            full_v = oracle.unpack_v(fmt, sentinel[b, h], cap)
            full_k[t] = kc_ref[b, h, 0]
            full_v[t] = vc_ref[b, h, 0]
            expect_k = oracle.pack_k(fmt, full_k, cap, sentinel[b, h].copy())
            expect_v = oracle.pack_v(fmt, full_v, cap, sentinel[b, h].copy())
            assert np.array_equal(gk[b, h], expect_k), (b, h)
            assert np.array_equal(gv[b, h], expect_v), (b, h)
            assert J > 0


def _paged_pool(kbytes, vbytes, W, seed, spare=3):
    """Scatter the 64-token blocks of contiguous streams [B][Hkv][cap * W] into a
    shuffled pool with a few unused blocks; returns pools and the block table."""
    B, H, n = kbytes.shape
    nb = n // (64 * W)
    total = B * H * nb + spare
    perm = np.random.default_rng(seed).permutation(total)[:B * H * nb].reshape(B, H, nb).astype(np.int32)
    kpool = np.random.default_rng(seed + 1).integers(0, 256, (total, 64 * W), dtype=np.uint8)
    vpool = kpool.copy()
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                kpool[perm[b, h, i]] = kbytes[b, h, i * 64 * W:(i + 1) * 64 * W]
                vpool[perm[b, h, i]] = vbytes[b, h, i * 64 * W:(i + 1) * 64 * W]
    return kpool, vpool, perm


@pytest.mark.parametrize("fmt,Hq,Hkv", [(0, 8, 2), (1, 10, 2), (2, 8, 2), (3, 10, 2), (4, 8, 2)])
@pytest.mark.parametrize("S", [1, 7])
@pytest.mark.parametrize("lens", [(1000, 700), (20000, 13001)])
def test_decode_paged_equals_contiguous(fmt, Hq, Hkv, S, lens):
    """A cache scattered over a shuffled block pool gives bitwise the same output
    as the contiguous cache (same arithmetic in the same order).  The long case
    gives every wave about 20 tiles (table lookups for tiles loaded ahead) and
    ragged last tiles."""
    lens = list(lens)
    B, T = len(lens), max(lens)
    say(f"decode paged fmt{fmt} S{S} lens{lens}")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 600 + fmt)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    W = vq.code_bytes_per_token(fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    kpool, vpool, table = _paged_pool(kbytes, vbytes, W, 9)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q), dev(s), qp)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    outs = []
    for paged in (False, True):
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        if paged:
            vq.decode_attention_paged(shape, qp, book_dev(kb), book_dev(vb), dev(kpool), dev(vpool),
                                      torch.from_numpy(table).to(DEV), seq, T, S, ws)
        else:
            vq.decode_attention_varlen(shape, qp, book_dev(kb), book_dev(vb), dev(kbytes), dev(vbytes), seq, T, S, ws)
        vq.combine(shape, S, ws, out)
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    ref = oracle.attention(fmt, q[1:2], s, kb, vb, kc[1:2, :, :lens[1]], vc[1:2, :, :lens[1]])
    assert rel_err(outs[1][1:2], ref) <= TOL


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_append_paged_bit_exact(fmt):
    """One token per sequence into a paged cache lands in the pool block its table
    names, byte for byte as in the contiguous cache; other pool bytes untouched."""
    say(f"quantize_append paged fmt{fmt}")
    B, Hkv, cap = 3, 2, 192
    positions = [5, 64 + 33, 191]
    case, s, kb, vb = _quant_case(fmt, B, Hkv, 1, "bf16", 80 + fmt)
    shape = vq.make_shape(B, Hkv, Hkv, cap, fmt)
    W = vq.code_bytes_per_token(fmt)
    base = np.random.default_rng(6).integers(0, 256, (B, Hkv, cap * W), dtype=np.uint8)
    kpool, vpool, table = _paged_pool(base, base, W, 12)
    kc_c, vc_c = dev(base), dev(base)
    kp, vp = dev(kpool), dev(vpool)
    pos = torch.tensor(positions, dtype=torch.int32, device=DEV)
    k_new, v_new = dev(case.k, torch.bfloat16), dev(case.v, torch.bfloat16)
    vq.quantize_append_varlen(shape, k_new, v_new, pos, dev(s), book_dev(kb), book_dev(vb), kc_c, vc_c)
    vq.quantize_append_paged(shape, k_new, v_new, pos, dev(s), book_dev(kb), book_dev(vb), kp, vp,
                             torch.from_numpy(table).to(DEV))
    torch.cuda.synchronize()
    want_k, want_v, _ = _paged_pool(kc_c.cpu().numpy(), vc_c.cpu().numpy(), W, 12)
    assert np.array_equal(kp.cpu().numpy(), want_k)
    assert np.array_equal(vp.cpu().numpy(), want_v)
    assert not np.array_equal(kc_c.cpu().numpy(), base)            # the appends did write


STEP_CASES = [
    # fmt, B, Hq, Hkv, position, S, dtype
    (0, 2, 32, 8, 0, 1, "bf16"),          # the first token: attention over one token
    (0, 2, 32, 8, 4098, 1, "bf16"),       # one split: the attention kernel writes out itself
    (0, 2, 32, 8, 4098, 9, "bf16"),       # ragged tail, fused combine
    (0, 1, 16, 2, 700, 11, "fp32"),       # G = 8: eight combine groups
    (0, 1, 8, 8, 2000, 32, "fp32"),       # G = 1
    (1, 1, 40, 8, 1000, 4, "bf16"),       # G = 5
    (1, 2, 12, 4, 4098, 9, "fp32"),       # G = 3
    (1, 1, 2, 2, 3000, 47, "bf16"),       # G = 1, many splits
    (2, 2, 32, 8, 4098, 9, "bf16"),       # 3-bit
    (2, 1, 8, 8, 700, 1, "fp32"),
    (3, 1, 40, 8, 1000, 4, "bf16"),       # 1.25-bit, G = 5
    (3, 2, 12, 4, 4098, 9, "fp32"),       # G = 3
    (3, 1, 8, 8, 700, 1, "bf16"),         # one split
    (0, 1, 12, 2, 2000, 3, "bf16"),       # G = 6
    (0, 1, 14, 2, 2000, 1, "fp32"),       # G = 7, one split
    (4, 1, 40, 8, 1000, 4, "bf16"),       # 4-bit, G = 5
    (4, 2, 12, 4, 4098, 9, "fp32"),       # G = 3
    # 2-bit, one split: the append runs inside the attention kernel (one launch).
    (0, 1, 16, 2, 700, 1, "fp32"),        # G = 8
    (0, 3, 8, 8, 2000, 1, "fp32"),        # G = 1
    (0, 2, 12, 4, 63, 1, "bf16"),         # G = 3, the last position of a block
    (0, 1, 40, 8, 64, 1, "bf16"),         # G = 5, the first position of a block
    (0, 1, 8, 2, 20000, 1, "bf16"),       # ~20 tiles per wave: the waves' in-step barriers
    (0, 2, 8, 2, 17000, 3, "fp32"),       # two launches, three splits of ~5.7k tokens
]


@pytest.mark.parametrize("fmt,B,Hq,Hkv,pos,S,dtype", STEP_CASES)
def test_decode_step_equals_the_four_calls(fmt, B, Hq, Hkv, pos, S, dtype):
    """decode_step (two launches, fused combine) against quantize_append +
    transform_query + decode_attention + combine: the same output bits and the
    same cache bytes, on two steps in a row that share a workspace filled with
    0xFF bytes beforehand (the counters need no initialization), and the
    output within the tolerance of the oracle on the cache as it ends up."""
    say(f"decode_step fmt{fmt} B{B} Hq{Hq} Hkv{Hkv} pos{pos} S{S} {dtype}")
    cap = ((pos + 2 + 63) // 64) * 64
    q, s, kb, vb, kc, vc, _ = _attn_inputs(fmt, B, Hq, Hkv, pos + 2, 5000 + pos + Hq, cap)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(pos + S)
    books, sm = (book_dev(kb), book_dev(vb)), dev(s)
    ref_k, ref_v = dev(kbytes), dev(vbytes)
    got_k, got_v = dev(kbytes), dev(vbytes)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws_ref = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    ws = torch.full((vq.step_workspace_bytes(shape, S),), 0xFF, dtype=torch.uint8, device=DEV)
    assert ws.numel() > ws_ref.numel()
    for p in (pos, pos + 1):
        qd = dev(rng.standard_normal((B, Hq, D)).astype(np.float32), tdt)
        k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32) * 2.0, tdt)
        v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), tdt)
        want = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        vq.quantize_append(shape, k_new, v_new, p, sm, books[0], books[1], ref_k, ref_v)
        vq.transform_query(shape, qd, sm, qp)
        vq.decode_attention(shape, qp, books[0], books[1], ref_k, ref_v, p + 1, S, ws_ref)
        vq.combine(shape, S, ws_ref, want)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        vq.decode_step(shape, qd, k_new, v_new, p, sm, books[0], books[1], got_k, got_v, S, ws, got)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"position {p}: max diff {np.abs(g - w).max()}"
        assert torch.equal(got_k, ref_k) and torch.equal(got_v, ref_v)
        _oracle_step_codes(fmt, kc, vc, [p] * B, k_new, v_new, s, kb, vb)
    # The cache after the second step holds the oracle's codes; the oracle's
    # attention over them.
    T = pos + 2
    _assert_cache_codes(fmt, got_k.cpu().numpy(), got_v.cpu().numpy(), kc, vc, [T] * B)
    ref = oracle.attention(fmt, qd.float().cpu().numpy(), s, kb, vb, kc, vc)
    err = rel_err(got.cpu().numpy(), ref)
    print(f"  max relative error {err:.3e}", flush=True)
    assert err <= TOL


def _hadamard():
    H = np.array([[1.0]])
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H / math.sqrt(D)


@pytest.mark.parametrize("S", [1, 3])
def test_fused_step_append_hard_cases_match_oracle(S):
    """The 2-bit step appends inside the attention kernel (one split: every
    work-group, three: the one whose split holds the token) with an fp32
    distance screen and the pinned fp64 distance for the survivors.  Tokens
    appended one step at a time must get the oracle's codes on: a duplicated
    entry (the lower index wins), midpoints of fp16 neighbours one ulp apart
    (below fp32 resolution), exact value midpoints, a negative, an infinite and
    a tiny scale (coordinates near 1e5), a zero scale (infinite or NaN
    coordinates), NaN elements, and values past the fp32 range of squares."""
    say(f"fused step append hard cases S{S}")
    fmt, B, Hq, Hkv, cap, p0, n = 0, 1, 8, 2, 256, 192, 16
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    H = _hadamard()
    rng = np.random.default_rng(77 + S)

    def near_tie_book(seed):
        r = np.random.default_rng(seed)
        base = (r.standard_normal((E // 2, dsub)) * 0.5).astype(np.float16)
        base[:, 0] = np.abs(base[:, 0]) + np.float16(0.25)
        up = base.copy()
        up[:, 0] = np.nextafter(base[:, 0], np.float16(np.inf))
        return base, up, np.concatenate([base, up]).view(np.uint16)

    scenarios = []
    # 1. Head 0: near ties one fp16 ulp apart; head 1: a duplicated entry hit exactly.
    base, up, ntb = near_tie_book(5)
    kb = np.stack([ntb, synth.random_fp16_book(6, (1, E, dsub), 0.5)[0]])
    kb[1, 200] = kb[1, 17]
    s = rng.uniform(0.5, 2.0, (Hkv, D)).astype(np.float32)
    pick = rng.integers(0, E // 2, (n, J))
    xt = base[pick].astype(np.float64)
    xt[:, :, 0] = 0.5 * (base[pick, 0].astype(np.float64) + up[pick, 0].astype(np.float64))
    k = np.empty((n, Hkv, D), np.float32)
    k[:, 0] = (xt.reshape(n, D) @ H) * s[0]
    c17 = kb[1, 17].view(np.float16).astype(np.float64)
    k[:, 1] = (np.tile(c17, J)[None] @ H) * s[1]
    vb = np.zeros((Hkv, E, dsub), np.float16)
    vb[:, :, 0] = np.arange(E, dtype=np.float64) * 0.25
    vb[:, E - 1] = vb[:, 5]
    v = np.zeros((n, Hkv, D), np.float32)
    v[:, :, ::dsub] = (rng.integers(0, 200, (n, Hkv, J)) * 0.25 + 0.125).astype(np.float32)
    v[:3, :, 0] = 1.25                                           # entries 5 and E - 1: 5 wins
    scenarios.append(("ties", k, v, s, kb, vb.view(np.uint16)))
    # 2. Degenerate scales: negative and infinite (head 0), tiny (head 1).
    s = rng.uniform(0.5, 2.0, (Hkv, D)).astype(np.float32)
    s[0, 9], s[0, 20], s[1, 33] = -1.5, np.inf, 1e-6
    k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    scenarios.append(("scales", k, v, s, synth.random_fp16_book(8, (Hkv, E, dsub), 0.8),
                      synth.random_fp16_book(9, (Hkv, E, dsub), 1.0)))
    # 3. Fallbacks: a zero scale (0 / 0 = NaN and x / 0 = inf), NaN elements,
    #    huge keys and values (squares past the fp32 range).
    s = rng.uniform(0.5, 2.0, (Hkv, D)).astype(np.float32)
    s[0, 5] = 0.0
    k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    k[::2, 0, 5] = 0.0
    k[1, 1] *= 3.0e5
    k[3, 1] *= 1.0e19
    k[5, 1, 7] = np.nan
    v[2, 0, 9] = np.nan
    v[4, 1, :dsub] = 2.0e19
    v[6, 0] *= 1.0e25
    scenarios.append(("fallbacks", k, v, s, synth.random_fp16_book(10, (Hkv, E, dsub), 0.8),
                      synth.random_fp16_book(11, (Hkv, E, dsub), 1.0)))

    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    for name, k, v, s, kb, vb in scenarios:
        kc0 = synth.random_codes(12, (B, Hkv, cap, J), E)
        vc0 = synth.random_codes(13, (B, Hkv, cap, J), E)
        kbytes, vbytes = oracle.pack_stream(fmt, kc0, vc0, cap)
        kcodes, vcodes = dev(kbytes), dev(vbytes)
        books, sm = (book_dev(kb), book_dev(vb)), dev(s)
        ws = torch.empty(vq.step_workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        qd = dev(rng.standard_normal((B, Hq, D)).astype(np.float32))
        for t in range(n):
            vq.decode_step(shape, qd, dev(k[None, t, :, None]), dev(v[None, t, :, None]), p0 + t, sm, books[0],
                           books[1], kcodes, vcodes, S, ws, out)
        torch.cuda.synchronize()
        for h in range(Hkv):
            kc_ref, vc_ref = oracle.quantize(fmt, k[:, h], v[:, h], s[h], kb[h], vb[h])
            gk = oracle.unpack_k(fmt, kcodes[0, h].cpu().numpy(), p0 + n)[p0:]
            gv = oracle.unpack_v(fmt, vcodes[0, h].cpu().numpy(), p0 + n)[p0:]
            assert np.array_equal(gk, kc_ref), (name, h, np.argwhere(gk != kc_ref)[:5])
            assert np.array_equal(gv, vc_ref), (name, h, np.argwhere(gv != vc_ref)[:5])
            if name == "ties" and h == 1:
                assert np.all(gk == 17)
            # The cache outside the appended rows is untouched.
            assert np.array_equal(oracle.unpack_k(fmt, kcodes[0, h].cpu().numpy(), p0), kc0[0, h, :p0])


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_step_captured_in_a_graph_replays_exactly(fmt):
    """One decode step (append of one token per sequence, query transform,
    decode, combine) captured in a HIP graph: every replay, with eager work and
    synchronizations between replays, equals the eager step bit for bit (the
    library launches only kernels on the caller's stream, no memsets or
    allocations)."""
    say(f"graph capture fmt{fmt}")
    B, Hq, Hkv, T = 2, 8, 2, 900
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 700 + fmt)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    rng = np.random.default_rng(3)
    k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))
    v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))
    S = 3
    books = (book_dev(kb), book_dev(vb))
    sm = dev(s)
    qd = dev(q)

    def make_state():
        return {"kc": dev(kbytes), "vc": dev(vbytes), "qp": torch.empty((B, Hq, D), dtype=torch.float32, device=DEV),
                "ws": torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV),
                "out": torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)}

    def step(st):
        vq.quantize_append(shape, k_new, v_new, T, sm, books[0], books[1], st["kc"], st["vc"])
        vq.transform_query(shape, qd, sm, st["qp"])
        vq.decode_attention(shape, st["qp"], books[0], books[1], st["kc"], st["vc"], T + 1, S, st["ws"])
        vq.combine(shape, S, st["ws"], st["out"])

    eager = make_state()
    step(eager)
    torch.cuda.synchronize()
    want = eager["out"].cpu().numpy()
    want_k, want_v = eager["kc"].cpu().numpy(), eager["vc"].cpu().numpy()

    g_state = make_state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm up outside the capture
        step(g_state)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_state)
    for r in range(3):
        g_state["out"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g_state["out"].cpu().numpy().view(np.uint32), want.view(np.uint32)), r
        assert np.array_equal(g_state["kc"].cpu().numpy(), want_k) and np.array_equal(g_state["vc"].cpu().numpy(), want_v)
        step(eager)                                     # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,Hq,Hkv,S,paged", [(0, 8, 2, 1, False), (0, 8, 2, 7, False), (1, 10, 2, 5, False),
                                                (0, 8, 2, 7, True), (1, 10, 2, 3, True), (0, 32, 8, 64, True),
                                                (2, 8, 2, 5, True), (0, 40, 8, 1, True), (0, 8, 8, 1, True),
                                                (3, 10, 2, 5, False), (3, 40, 8, 3, True), (4, 8, 2, 4, False),
                                                (4, 40, 8, 3, True)])
def test_decode_step_ragged_equals_the_four_calls(fmt, Hq, Hkv, S, paged):
    """decode_step_varlen / decode_step_paged against append (varlen / paged) +
    transform_query + decode (varlen / paged, lengths positions + 1) + combine:
    the same output bits and cache bytes on two steps in a row (positions: the
    first token, a ragged tail, the longest, a skipped sequence at -1 that must
    give zeros, a block start), then the oracle per sequence."""
    say(f"decode_step ragged fmt{fmt} Hq{Hq} Hkv{Hkv} S{S} paged={paged}")
    pos0 = [0, 776, 4098, -1, 64]
    B = len(pos0)
    cap = ((max(pos0) + 2 + 63) // 64) * 64
    W = vq.code_bytes_per_token(fmt)
    q, s, kb, vb, kc, vc, _ = _attn_inputs(fmt, B, Hq, Hkv, max(pos0) + 2, 6100 + S, cap)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    if paged:
        kpool, vpool, table = _paged_pool(kbytes, vbytes, W, 61 + S)
        tab = torch.from_numpy(table).to(DEV)
        ref_k, ref_v, got_k, got_v = dev(kpool), dev(vpool), dev(kpool), dev(vpool)
    else:
        ref_k, ref_v, got_k, got_v = dev(kbytes), dev(vbytes), dev(kbytes), dev(vbytes)
    rng = np.random.default_rng(S)
    books, sm = (book_dev(kb), book_dev(vb)), dev(s)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws_ref = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    ws = torch.full((vq.step_workspace_bytes(shape, S),), 0xFF, dtype=torch.uint8, device=DEV)
    for step in range(2):
        pos = [p + step if p >= 0 else p for p in pos0]
        mx = max(pos) + 1
        pos_d = torch.tensor(pos, dtype=torch.int32, device=DEV)
        lens_d = torch.tensor([max(p + 1, 0) for p in pos], dtype=torch.int32, device=DEV)
        qd = dev(rng.standard_normal((B, Hq, D)).astype(np.float32), torch.bfloat16)
        k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
        v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
        want = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        if paged:
            vq.quantize_append_paged(shape, k_new, v_new, pos_d, sm, books[0], books[1], ref_k, ref_v, tab)
            vq.transform_query(shape, qd, sm, qp)
            vq.decode_attention_paged(shape, qp, books[0], books[1], ref_k, ref_v, tab, lens_d, mx, S, ws_ref)
            vq.decode_step_paged(shape, qd, k_new, v_new, pos_d, mx, sm, books[0], books[1], got_k, got_v, tab, S,
                                 ws, got)
        else:
            vq.quantize_append_varlen(shape, k_new, v_new, pos_d, sm, books[0], books[1], ref_k, ref_v)
            vq.transform_query(shape, qd, sm, qp)
            vq.decode_attention_varlen(shape, qp, books[0], books[1], ref_k, ref_v, lens_d, mx, S, ws_ref)
            vq.decode_step_varlen(shape, qd, k_new, v_new, pos_d, mx, sm, books[0], books[1], got_k, got_v, S,
                                  ws, got)
        vq.combine(shape, S, ws_ref, want)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"step {step}: max diff {np.abs(g - w).max()}"
        assert torch.equal(got_k, ref_k) and torch.equal(got_v, ref_v)
        assert np.all(g[3] == 0.0)
        _oracle_step_codes(fmt, kc, vc, pos, k_new, v_new, s, kb, vb)
    # The cache after the second step holds the oracle's codes; the oracle's
    # attention per sequence over them.
    gk, gv = got_k.cpu().numpy(), got_v.cpu().numpy()
    if paged:
        nb = cap // 64
        gk = np.stack([np.stack([np.concatenate([gk[table[b, h, i]] for i in range(nb)]) for h in range(Hkv)])
                       for b in range(B)])
        gv = np.stack([np.stack([np.concatenate([gv[table[b, h, i]] for i in range(nb)]) for h in range(Hkv)])
                       for b in range(B)])
    _assert_cache_codes(fmt, gk, gv, kc, vc, [p + 1 for p in pos])
    qf = qd.float().cpu().numpy()
    for b, p in enumerate(pos):
        if p < 0:
            continue
        T = p + 1
        ref = oracle.attention(fmt, qf[b:b + 1], s, kb, vb, kc[b:b + 1, :, :T], vc[b:b + 1, :, :T])
        err = rel_err(g[b:b + 1], ref)
        print(f"  b={b} T={T} max relative error {err:.3e}", flush=True)
        assert err <= TOL


@pytest.mark.parametrize("fmt,S", [(0, 1), (0, 3), (1, 3), (3, 2), (4, 2)])
def test_decode_step_varlen_appends_past_max_seq_len(fmt, S):
    """A ragged step whose max_seq_len is below positions[b] + 1: the token is
    still appended (by the last split's work-group in the one-launch 2-bit
    step) and no split attends to it, exactly as the separate calls do; the
    cache then holds the oracle's codes for it."""
    say(f"decode_step_varlen with a position past max_seq_len, fmt{fmt} S{S}")
    B, Hq, Hkv = 2, 8, 2
    pos, mx = [100, 3000], 1000
    cap = 3072
    q, s, kb, vb, kc, vc, _ = _attn_inputs(fmt, B, Hq, Hkv, cap, 8100 + S + fmt, cap)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    ref_k, ref_v, got_k, got_v = dev(kbytes), dev(vbytes), dev(kbytes), dev(vbytes)
    rng = np.random.default_rng(31 + S)
    books, sm = (book_dev(kb), book_dev(vb)), dev(s)
    qd = dev(rng.standard_normal((B, Hq, D)).astype(np.float32), torch.bfloat16)
    k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    pos_d = torch.tensor(pos, dtype=torch.int32, device=DEV)
    lens_d = torch.tensor([p + 1 for p in pos], dtype=torch.int32, device=DEV)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws_ref = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    ws = torch.full((vq.step_workspace_bytes(shape, S),), 0xFF, dtype=torch.uint8, device=DEV)
    want = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    vq.quantize_append_varlen(shape, k_new, v_new, pos_d, sm, books[0], books[1], ref_k, ref_v)
    vq.transform_query(shape, qd, sm, qp)
    vq.decode_attention_varlen(shape, qp, books[0], books[1], ref_k, ref_v, lens_d, mx, S, ws_ref)
    vq.combine(shape, S, ws_ref, want)
    vq.decode_step_varlen(shape, qd, k_new, v_new, pos_d, mx, sm, books[0], books[1], got_k, got_v, S, ws, got)
    torch.cuda.synchronize()
    g, w = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"max diff {np.abs(g - w).max()}"
    assert torch.equal(got_k, ref_k) and torch.equal(got_v, ref_v)
    _oracle_step_codes(fmt, kc, vc, pos, k_new, v_new, s, kb, vb)
    _assert_cache_codes(fmt, got_k.cpu().numpy(), got_v.cpu().numpy(), kc, vc, [p + 1 for p in pos])


@pytest.mark.parametrize("fmt,S", [(0, 3), (1, 4), (0, 1), (2, 2), (3, 3), (4, 1), (4, 4)])
def test_decode_step_captured_in_a_graph(fmt, S):
    """decode_step captured in a HIP graph: the prologue clears the arrival
    counters with ordinary stores (no memset node), so every replay, with eager
    steps on another workspace between replays, equals the eager step bit for
    bit."""
    say(f"decode_step graph fmt{fmt} S{S}")
    B, Hq, Hkv, T = 2, 8, 2, 1500
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, B, Hq, Hkv, T, 900 + fmt)
    shape = vq.make_shape(B, Hq, Hkv, cap, fmt)
    kbytes, vbytes = oracle.pack_stream(fmt, kc, vc, cap)
    rng = np.random.default_rng(4)
    k_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    v_new = dev(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32), torch.bfloat16)
    qd = dev(q, torch.bfloat16)
    books, sm = (book_dev(kb), book_dev(vb)), dev(s)

    def make_state():
        return {"kc": dev(kbytes), "vc": dev(vbytes),
                "ws": torch.empty(vq.step_workspace_bytes(shape, S), dtype=torch.uint8, device=DEV),
                "out": torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)}

    def step(st):
        vq.decode_step(shape, qd, k_new, v_new, T - 1, sm, books[0], books[1], st["kc"], st["vc"], S, st["ws"],
                       st["out"])

    eager = make_state()
    step(eager)
    torch.cuda.synchronize()
    want = eager["out"].cpu().numpy()
    g_state = make_state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(g_state)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_state)
    for r in range(3):
        g_state["out"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g_state["out"].cpu().numpy().view(np.uint32), want.view(np.uint32)), r
        step(eager)
        torch.cuda.synchronize()


def test_decode_single_token_returns_its_value():
    say("decode T=1")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(0, 1, 8, 2, 1, 77, cap=128)
    got = _gpu_attention(0, q, s, kb, vb, kc, vc, cap, 1)
    for g in range(8):
        h = g // 4
        v0 = vb[h].view(np.float16).astype(np.float64)[vc[0, h, 0]].reshape(D)
        assert np.abs(got[0, g] - v0).max() <= 1e-6 * np.abs(v0).max()


@pytest.mark.parametrize("fmt,Hq,Hkv,S", [(0, 8, 2, 3), (1, 10, 2, 3), (2, 8, 2, 1), (3, 10, 2, 4), (4, 8, 2, 3)])
def test_decode_query_beyond_fp16_range(fmt, Hq, Hkv, S):
    """Queries whose elements times sm_scale * log2(e) pass the fp16 maximum
    (65504): the matrix-core path scales such a head's query operand by a
    power of two and takes its scores back in the exponents.  With unit
    smoothing scales and a constant query row, q' = H q is that constant
    times sqrt(128) on dim 0 and exactly zero elsewhere, so the softmax puts
    equal weights on the tokens whose sub-vector-0 centroid has the largest
    (first head) or smallest (last head) dim 0; the other heads stay normal."""
    say(f"decode with fp16-overflowing queries, fmt {fmt} Hq{Hq} Hkv{Hkv} S{S}")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, 1, Hq, Hkv, 1000, 4242 + fmt)
    s = np.ones_like(s)
    q[0, 0, :] = 5.0e5          # q'_0 * sm_scale * log2(e) ~ 7.2e5
    q[0, Hq - 1, :] = -3.0e6    # ~ -4.3e6
    got = _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, S)
    ref = oracle.attention(fmt, q, s, kb, vb, kc, vc)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  max relative error {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("fmt,path", [(0, "table"), (0, "gather"), (0, "mfma"), (1, "mfma"), (1, "gather"), (2, "mfma"),
                                      (3, "mfma"), (4, "mfma")])
def test_decode_split_invariance_and_determinism(fmt, path):
    """1 split vs 64 splits, and a rerun.  Every path rounds each weight to fp16
    (round to nearest, relative error <= 2^-11) against a running maximum that
    depends on the split, and normalizes by the sum of the same rounded weights;
    two split counts give two independent roundings, so the outputs may differ
    by up to about 2 * 2^-11 of the value range: 1e-3.  Reruns are bitwise equal."""
    say(f"decode splits 1 vs 64, rerun, fmt {fmt} {path}")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(fmt, 1, 32, 8, 4096, 5)
    a = _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, 1, path)
    b = _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, 64, path)
    c = _gpu_attention(fmt, q, s, kb, vb, kc, vc, cap, 64, path)
    assert rel_err(b, a) < 1e-3
    assert np.array_equal(b.view(np.uint32), c.view(np.uint32))


def test_decode_ignores_bytes_past_seq_len():
    """Codes beyond seq_len (inside the capacity) must not change the result."""
    say("decode garbage past seq_len")
    q, s, kb, vb, kc, vc, cap = _attn_inputs(0, 1, 4, 1, 100, 9, cap=256)
    shape = vq.make_shape(1, 4, 1, cap, 0)
    kbytes, vbytes = oracle.pack_stream(0, kc, vc, cap)
    noise = np.random.default_rng(3).integers(0, 256, kbytes.shape, dtype=np.uint8)
    # The bytes that hold tokens [0, 100): pack an all-ones code array (unused
    # bytes stay 0), whatever the layout is.
    ones = np.ones((1, 1, 100, 32), dtype=np.uint16)
    kmask, vmask = (m != 0 for m in oracle.pack_stream(0, ones, ones, cap))
    assert kmask.sum() == vmask.sum() == 100 * 32
    kb2 = np.where(kmask, kbytes, noise)
    vb2 = np.where(vmask, vbytes, noise)
    qp = torch.empty((1, 4, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q), dev(s), qp)
    a = run_decode(shape, qp, book_dev(kb), book_dev(vb), dev(kbytes), dev(vbytes), 100, 2)
    b = run_decode(shape, qp, book_dev(kb), book_dev(vb), dev(kb2), dev(vb2), 100, 2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_end_to_end_tiny_workload():
    """The tiny 2-bit workload end to end: GPU calibration (scales, 20-iteration
    K-Means books) equals the oracle's, GPU codes equal the oracle's, and the
    GPU decode is within 2e-3 of the oracle's attention."""
    wl = synth.WORKLOADS["tiny_g4_t2048"]
    say(wl.name)
    case = synth.make_cpu_case(wl, synth.seed_for(wl.name))
    s_ref = oracle.smooth_scales(case.k_cal[0])
    init_k = synth.kmeans_init_indices(11, synth.N_CALIB * 32, 256)
    init_v = synth.kmeans_init_indices(12, synth.N_CALIB * 32, 256)
    kb_ref, vb_ref = oracle.train_codebooks(0, case.k_cal[0], case.v_cal[0], s_ref, init_k, init_v, iters=20)

    smooth = torch.empty((1, D), dtype=torch.float32, device=DEV)
    vq.smooth_scales(dev(case.k_cal), smooth)
    ws = torch.empty(vq.train_workspace_bytes(0, synth.N_CALIB), dtype=torch.uint8, device=DEV)
    k_book = torch.empty((1, 256, 4), dtype=torch.int16, device=DEV)
    v_book = torch.empty((1, 256, 4), dtype=torch.int16, device=DEV)
    vq.train_codebook(0, dev(case.k_cal[0]), True, smooth[0], dev(init_k), 20, k_book[0], ws)
    vq.train_codebook(0, dev(case.v_cal[0]), False, None, dev(init_v), 20, v_book[0], ws)
    torch.cuda.synchronize()
    assert np.array_equal(smooth.cpu().numpy()[0], s_ref)
    assert np.array_equal(k_book.cpu().numpy()[0].view(np.uint16), kb_ref)
    assert np.array_equal(v_book.cpu().numpy()[0].view(np.uint16), vb_ref)

    shape = vq.make_shape(1, 4, 1, 2048, 0)
    cache = vq.VQCache.allocate(shape, smooth, k_book, v_book, DEV)
    cache.append(dev(case.k), dev(case.v), 0)
    out = cache.attend(dev(case.q), 2048, num_splits=8).cpu().numpy()
    kc, vc = oracle.quantize(0, case.k[0, 0], case.v[0, 0], s_ref, kb_ref, vb_ref)
    assert np.array_equal(oracle.unpack_k(0, cache.k_codes[0, 0].cpu().numpy(), 2048), kc)
    assert np.array_equal(oracle.unpack_v(0, cache.v_codes[0, 0].cpu().numpy(), 2048), vc)
    ref = oracle.attention(0, case.q, s_ref[None], kb_ref[None], vb_ref[None], kc[None, None], vc[None, None])
    assert rel_err(out, ref) <= TOL
    # The same through VQCache.step: 2047 tokens appended, then the last token's
    # step (decode_step), bit-identical to the four calls above.
    stepped = vq.VQCache.allocate(shape, smooth, k_book, v_book, DEV)
    stepped.append(dev(case.k[:, :, :2047]).contiguous(), dev(case.v[:, :, :2047]).contiguous(), 0)
    out2 = stepped.step(dev(case.q), dev(case.k[:, :, 2047:]).contiguous(), dev(case.v[:, :, 2047:]).contiguous(),
                        2047, num_splits=8).cpu().numpy()
    assert np.array_equal(out2.view(np.uint32), out.view(np.uint32))
    assert torch.equal(stepped.k_codes, cache.k_codes) and torch.equal(stepped.v_codes, cache.v_codes)
    # Quality, not parity: the 2-bit cache stays close to full-precision attention.
    fp = oracle.attention_fp(case.q, case.k, case.v)
    print(f"  VQ vs full precision: {rel_err(ref, fp):.3f}", flush=True)


# ---------------------------------------------------------- full sizes, sampled

FULL = ["llama8b_b1_t32k", "llama8b_b1_t196k", "llama8b_b32_t196k", "qwen14b_b8_t128k_1p5", "llama8b_b8_t196k_3bit",
        "qwen14b_b8_t128k_1p25", "llama8b_b8_t196k_4bit"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """The workload at its full size, in the benchmark's launch configuration
    (suggested split count, auto path), with random codes drawn on the device;
    sampled (b, KV head) slices are checked against the oracle."""
    wl = synth.WORKLOADS[name]
    say(f"full size {name}")
    fmt, B, Hq, Hkv, T = wl.fmt, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len
    E, dsub = oracle.FORMATS[fmt]
    seed = synth.seed_for(name)
    W = vq.code_bytes_per_token(fmt)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    kbytes = torch.randint(0, 256, (B, Hkv, T * W), generator=gen, dtype=torch.uint8, device=DEV)
    vbytes = torch.randint(0, 256, (B, Hkv, T * W), generator=gen, dtype=torch.uint8, device=DEV)
    kb = synth.random_fp16_book(seed, (Hkv, E, dsub), 0.6)
    vb = synth.random_fp16_book(seed + 1, (Hkv, E, dsub), 1.0)
    rng = np.random.default_rng(seed)
    q = synth.normal_numpy(rng, (B, Hq, D), "bf16")
    s = rng.uniform(0.5, 4.0, (Hkv, D)).astype(np.float32)
    shape = vq.make_shape(B, Hq, Hkv, T, fmt)
    S = vq.suggest_splits(shape, T)
    qp = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.transform_query(shape, dev(q, torch.bfloat16), dev(s), qp)
    got = run_decode(shape, qp, book_dev(kb), book_dev(vb), kbytes, vbytes, T, S)
    G = Hq // Hkv
    samples = [(b, h) for b in range(B) for h in range(Hkv)]
    pick = np.random.default_rng(seed).permutation(len(samples))[: (8 if B == 1 else 4)]
    worst = 0.0
    for i in pick:
        b, h = samples[i]
        kc = oracle.unpack_k(fmt, kbytes[b, h].cpu().numpy(), T)[None, None]
        vc = oracle.unpack_v(fmt, vbytes[b, h].cpu().numpy(), T)[None, None]
        ref = oracle.attention(fmt, q[b:b + 1, h * G:(h + 1) * G], s[h:h + 1], kb[h:h + 1], vb[h:h + 1], kc, vc)
        worst = max(worst, rel_err(got[b:b + 1, h * G:(h + 1) * G], ref))
    print(f"  S={S} max relative error over {len(pick)} slices: {worst:.3e}", flush=True)
    assert worst <= TOL


def test_full_size_append_one_token():
    """The 196k single-sequence workload's per-step append: one bf16 token at
    the last position of every KV head, bit-exact against the oracle."""
    wl = synth.WORKLOADS["llama8b_b1_t196k"]
    say("append one token at position 196607")
    T, Hkv = wl.seq_len, wl.num_kv_heads
    case, s, kb, vb = _quant_case(0, 1, Hkv, 1, "bf16", 99)
    shape = vq.make_shape(1, Hkv, Hkv, T, 0)
    kcodes = torch.zeros((1, Hkv, T * 32), dtype=torch.uint8, device=DEV)
    vcodes = torch.zeros_like(kcodes)
    vq.quantize_append(shape, dev(case.k, torch.bfloat16), dev(case.v, torch.bfloat16), T - 1, dev(s),
                       book_dev(kb), book_dev(vb), kcodes, vcodes)
    torch.cuda.synchronize()
    kc_ref, vc_ref = _oracle_codes(0, case, s, kb, vb)
    gk = kcodes[0, :, (T - 1) * 32:].cpu().numpy()
    # The value layout is blocked by 64 tokens: unpack the last block alone.
    last = vcodes[0, :, (T - 64) * 32:].cpu().numpy()
    gv = np.stack([oracle.unpack_v(0, last[h], 64)[63] for h in range(Hkv)])
    assert np.array_equal(gk, kc_ref[0, :, 0])
    assert np.array_equal(gv, vc_ref[0, :, 0])


def test_library_is_the_in_tree_build():
    path = vq.lib()._name
    assert os.path.abspath(path) == os.path.abspath(vq.LIB_PATH)
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(vq.LIB_PATH) in maps or vq.LIB_PATH in maps


@pytest.mark.parametrize("B,Hq,Hkv,T,S", [(1, 4, 1, 2048, 4), (2, 32, 8, 333, 3), (1, 40, 8, 1000, 2), (1, 8, 1, 65, 1)])
def test_bf16_baseline_matches_full_precision_oracle(B, Hq, Hkv, T, S):
    """The unquantized bf16 decode used as the speed baseline computes softmax(q.k) v."""
    say(f"bf16 baseline B{B} Hq{Hq} Hkv{Hkv} T{T} S{S}")
    rng = np.random.default_rng(T)
    cap = ((T + 63) // 64) * 64
    q = synth.normal_numpy(rng, (B, Hq, D), "bf16")
    k = synth.normal_numpy(rng, (B, Hkv, cap, D), "bf16")
    v = synth.normal_numpy(rng, (B, Hkv, cap, D), "bf16")
    shape = vq.make_shape(B, Hq, Hkv, cap, 0)
    ws = torch.empty(vq.workspace_bytes(shape, S), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    vq.baseline_bf16_decode(shape, dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), T, S, ws)
    vq.combine(shape, S, ws, out)
    torch.cuda.synchronize()
    ref = oracle.attention_fp(q, k[:, :, :T], v[:, :, :T])
    assert rel_err(out.cpu().numpy(), ref) <= TOL
