"""The transform ablation through the library (VecInfer summary card,
"Summary": key outliers leave much of the codebook unused and sit far from
the centroids; smoothing followed by a Hadamard rotation fixes both; "Key
points", ablation on transformations: either one alone gains less than both).

Each variant's codebook is trained by vqkv_train_codebook and its keys coded
by vqkv_quantize_append, on the synthetic outlier keys (N(0,1), 4 channels
x15; a 4096-token calibration draw and 1024 test tokens of one KV head):
  * smooth+rotate  the key path with the smoothing scales: x' = H (k / s);
  * rotate         the key path with unit scales: x' = H k;
  * none           the value path (raw rows, no transform) on the keys;
  * smooth         the value path on k / s (the division done here in fp32:
                   the library has no smooth-only mode).
The GPU's codebooks and codes are checked bit for bit against the oracle's
(oracle K-Means from the same initial indices, oracle nearest-centroid), and
the pages' orderings are asserted from the GPU's codes: the combined transform
gives the smallest attention-score error and key error, and the highest code
utilization (entropy of the code histogram; 8 bits is a uniform use of 256
entries)."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import vector_quantized_bit_vqkv_amd as vq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D, E, DSUB = 128, 256, 4
J = D // DSUB


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _gpu_book(rows, is_key, s, init, iters):
    n = rows.shape[0]
    ws = torch.empty(vq.train_workspace_bytes(vq.FMT_2BIT, n), dtype=torch.uint8, device=DEV)
    book = torch.empty((E, DSUB), dtype=torch.int16, device=DEV)
    vq.train_codebook(vq.FMT_2BIT, _dev(rows), is_key, _dev(s) if is_key else None, _dev(init), iters, book, ws)
    torch.cuda.synchronize()
    return book.cpu().numpy().view(np.uint16)


def _gpu_codes(rows, key_path, s, book):
    """Codes of rows [n][128] through the key path (x' = H (k / s)) or the value
    path (raw), by vqkv_quantize_append into a one-stream cache."""
    n = rows.shape[0]
    cap = ((n + 63) // 64) * 64
    shape = vq.make_shape(1, 1, 1, cap, vq.FMT_2BIT)
    x = _dev(rows.astype(np.float32)[None, None])
    zero = torch.zeros_like(x)
    b = _dev(book.view(np.int16)[None])
    kc = torch.zeros((1, 1, cap * 32), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    vq.quantize_append(shape, x if key_path else zero, zero if key_path else x, 0, _dev(s[None]), b, b, kc, vc)
    torch.cuda.synchronize()
    if key_path:
        return oracle.unpack_k(0, kc[0, 0].cpu().numpy(), n)
    return oracle.unpack_v(0, vc[0, 0].cpu().numpy(), n)


@pytest.fixture(scope="module")
def ablation():
    rng = np.random.default_rng(2024)
    ch = synth.outlier_channels(7, 1)[0]
    k_cal = rng.standard_normal((4096, D)).astype(np.float32)
    k_cal[:, ch] *= synth.OUTLIER_SCALE
    k = rng.standard_normal((1024, D)).astype(np.float32)
    k[:, ch] *= synth.OUTLIER_SCALE
    q = rng.standard_normal((32, D))
    s = oracle.smooth_scales(k_cal)                       # fp32, the oracle's (the GPU's are pinned elsewhere)
    ones = np.ones(D, dtype=np.float32)
    H = oracle.hadamard()
    init = synth.kmeans_init_indices(5, 4096 * J, E)
    iters = 10
    s64 = s.astype(np.float64)
    # (key path?, scales, calibration rows, test rows, map of a dequantized row back to key space)
    variants = {
        "smooth+rotate": (True, s, k_cal, k, lambda x: (x @ H) * s64),
        "rotate": (True, ones, k_cal, k, lambda x: x @ H),
        "none": (False, ones, k_cal, k, lambda x: x),
        "smooth": (False, ones, k_cal / s, k / s, lambda x: x * s64),
    }
    ref = q @ k.astype(np.float64).T
    out = {}
    for name, (key_path, sc, cal, test, back) in variants.items():
        print(f"\n[case] ablation variant {name}", flush=True)
        book = _gpu_book(cal, key_path, sc, init, iters)
        codes = _gpu_codes(test, key_path, sc, book)
        # The oracle from the same inputs: K-Means, then nearest centroids.
        pts = oracle.transform_keys(cal, sc) if key_path else cal.astype(np.float64)
        cent, _ = oracle.kmeans(pts.reshape(-1, DSUB), init, iters)
        book_ref = oracle.doubles_to_half(cent)
        assert np.array_equal(book, book_ref), f"{name}: codebook differs from the oracle's"
        kc_ref, vc_ref = oracle.quantize(0, test, test, sc, book_ref, book_ref)
        assert np.array_equal(codes, kc_ref if key_path else vc_ref), f"{name}: codes differ from the oracle's"
        centroids = np.array([oracle.half_to_double(int(b)) for b in book.ravel()]).reshape(E, DSUB)
        k_hat = back(centroids[codes.astype(np.int64)].reshape(test.shape))
        scores = q @ k_hat.T
        use = np.bincount(codes.ravel(), minlength=E) / codes.size
        out[name] = {
            "score_err": float(np.linalg.norm(scores - ref) / np.linalg.norm(ref)),
            "key_mse": float(((k_hat - k) ** 2).sum() / (k.astype(np.float64) ** 2).sum()),
            "entropy": float(-(use[use > 0] * np.log2(use[use > 0])).sum()),
        }
        print(f"  {name}: {out[name]}", flush=True)
    return out


def test_combined_transform_has_the_lowest_score_and_key_error(ablation):
    e = {n: r["score_err"] for n, r in ablation.items()}
    m = {n: r["key_mse"] for n, r in ablation.items()}
    for other in ("none", "smooth", "rotate"):
        assert e["smooth+rotate"] < e[other], (other, e)
        assert m["smooth+rotate"] < m[other], (other, m)


def test_combined_transform_uses_the_codebook_best(ablation):
    h = {n: r["entropy"] for n, r in ablation.items()}
    assert h["smooth+rotate"] > h["none"] and h["smooth+rotate"] > h["smooth"]
    assert h["smooth+rotate"] > 7.0
