"""The distortion-rate measurement (library records written by kv_encode and
reconstructed by kv_decode on the GPU) against the same distortion computed by
the oracle: its float64 encode, dequantization and reconstruction of the same
tokens with the same bases and fixed scales."""
import numpy as np
import pytest

import workloads as W
from oracle import codec, quantizer, transform

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)
    return K


def _oracle_distortion(wl, h, t, n, r, b, static):
    x = W.tokens(wl, t, 0, h, 0, n, wl.dtype).astype(np.float64)
    _, vecs = transform.ordered_basis(W.covariance(wl, t, h))
    P = transform.folded_basis(vecs, r, W.hadamard_signs(wl, t, h, r)).astype(np.float32).astype(np.float64)
    if static:
        s = float(np.sqrt(np.trace(P.T @ W.covariance(wl, t, h) @ P) / r))
        mu, sg = quantizer.static_scale(s, b)
        c = codec.decode_records_static(codec.encode_tokens_static(x, P, b, mu, sg), r, b, mu, sg)
    else:
        c = codec.decode_records(codec.encode_tokens(x, P, b), r, b)
    return float(((x - c @ P.T) ** 2).sum() / (x ** 2).sum())


@pytest.mark.parametrize("static", [False, True])
def test_distortion_measurement_matches_oracle(K, static):
    import bench

    wl = W.LLAMA_256_HEADS
    heads, n = [3, 100, 255], 1024
    formats = [(128, 2), (64, 4), (16, 8), (128, 5)]
    got = bench.measure_distortion(K, wl, heads, n, formats, static=static)
    worst = 0.0
    for h in heads:
        for t in "KV":
            for r, b in formats:
                ref = _oracle_distortion(wl, h, t, n, r, b, static)
                rel = abs(got[(h, t, (r, b))] - ref) / ref
                worst = max(worst, rel)
                assert rel <= 1e-4, (h, t, r, b, got[(h, t, (r, b))], ref)
    print(f"distortion measurement (header-free {static}): worst relative difference {worst:.2e}", flush=True)
