"""Helpers shared by the GPU tests: device upload and the tolerance checks."""
import numpy as np


def dev(a, device="cuda"):
    """numpy float16 / float32 array -> torch device tensor (memory only)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_u16(t) -> np.ndarray:
    """fp16 torch tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f16_ulp(ref_bits: np.ndarray) -> np.ndarray:
    """ulp(c) = 2^(max(floor(log2|c|), -14) - 10) for finite c != 0; 2^-24 at 0.

    This is the gap from |c| to the next larger fp16 magnitude."""
    v = np.abs(ref_bits.view(np.float16).astype(np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    ulp = 2.0 ** (np.maximum(e, -14) - 10)
    return np.where(v > 0, ulp, 2.0 ** -24)


def check_f16_tolerance(got_bits, ref_bits, what=""):
    """|got - ref| <= 1 fp16 ulp(ref) + 1e-3 elementwise; +-inf must match."""
    got = got_bits.view(np.float16).astype(np.float64)
    ref = ref_bits.view(np.float16).astype(np.float64)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(got[~fin], ref[~fin]), what + ": non-finite mismatch"
    err = np.abs(got[fin] - ref[fin])
    bound = f16_ulp(ref_bits[fin]) + 1e-3
    if err.size:
        # Reported with `pytest -s`: the worst error seen, in fp16 ulps of the oracle value.
        print("[maxerr] %s: %.3g abs, %.3g ulp, %d of %d entries differ" % (
            what, err.max(), (err / f16_ulp(ref_bits[fin])).max(), np.count_nonzero(err), err.size))
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, "%s: %d entries out of tolerance, worst err %.3g (bound %.3g)" % (
        what, bad.size, err.max(), bound[np.argmax(err - bound)])


def check_f32_splitk_tolerance(got, ref, K, what=""):
    """|got - ref| <= 1e-5 * sqrt(K) * max|ref| (max over the checked entries)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = 1e-5 * np.sqrt(max(K, 1)) * max(np.abs(ref).max(), 0.0)
    err = np.abs(got - ref).max() if ref.size else 0.0
    if ref.size:
        print("[maxerr] %s: %.3g abs, %.3g of max|ref|" % (what, err, err / max(np.abs(ref).max(), 1e-300)))
    assert err <= bound, "%s: max err %.3g > bound %.3g" % (what, err, bound)


def sample_ij(M, N, count, seed, tile=256):
    """Random (i, j) pairs plus every entry of the first, last and a tile-
    boundary row/column (bounded to `count` extra entries each)."""
    rng = np.random.default_rng(seed)
    parts = [np.stack([rng.integers(0, M, count), rng.integers(0, N, count)], axis=1)]
    for i in sorted({0, M - 1, min(M - 1, tile - 1), min(M - 1, tile)}):
        js = np.unique(np.linspace(0, N - 1, min(N, 512)).astype(np.int64))
        parts.append(np.stack([np.full(js.size, i), js], axis=1))
    for j in sorted({0, N - 1, min(N - 1, tile - 1), min(N - 1, tile)}):
        is_ = np.unique(np.linspace(0, M - 1, min(M, 512)).astype(np.int64))
        parts.append(np.stack([is_, np.full(is_.size, j)], axis=1))
    return np.concatenate(parts).astype(np.int64)
