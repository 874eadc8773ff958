"""Pins for the oracle's buffer fingerprint (CPU only): the XXH64 written from its
published specification against the xxhash library and the specification's
empty-input value, and the chunk-wise composition against its definition
(Megatron Core bitwise-determinism news item, news.hamidun.com, "debugging
methodology": GPU-side fingerprints, chunk-wise for order-sensitive data)."""
import numpy as np
import pytest
import xxhash

from oracle import fingerprint as fp


def test_xxh64_published_values():
    assert fp.xxh64(b"") == 0xEF46DB3751D8E999
    assert fp.xxh64(b"", seed=1) == xxhash.xxh64(b"", seed=1).intdigest()


@pytest.mark.parametrize("n", list(range(0, 70)) + [127, 128, 129, 1000, 4096, 4099])
def test_xxh64_matches_library(rng, n):
    """Every length class: short inputs, each tail (8-byte words, a 4-byte word, single
    bytes) and whole 32-byte stripes."""
    data = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
    for seed in (0, 12345):
        assert fp.xxh64(data, seed) == xxhash.xxh64(data, seed=seed).intdigest()


@pytest.mark.parametrize("n,chunk", [(0, 64), (1, 64), (64, 64), (65, 64), (1000, 32), (4096, 1024), (777, 8)])
def test_chunked_fingerprint_definition(rng, n, chunk):
    data = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
    f = fp.fingerprint(data, chunk)
    parts = [data[k:k + chunk] for k in range(0, n, chunk)] or [b""]
    assert f["chunks"] == [xxhash.xxh64(p).intdigest() for p in parts]
    assert f["hash"] == xxhash.xxh64(b"".join(c.to_bytes(8, "little") for c in f["chunks"])).intdigest()
    assert len(f["chunks"]) == fp.chunk_count(n, chunk)


def test_fingerprint_detects_one_flipped_bit(rng):
    """A single changed bit changes its chunk's hash and the whole fingerprint, and no other chunk."""
    data = bytearray(rng.integers(0, 256, size=4096, dtype=np.uint8).tobytes())
    a = fp.fingerprint(bytes(data), 512)
    data[1500] ^= 0x10
    b = fp.fingerprint(bytes(data), 512)
    diff = [k for k in range(len(a["chunks"])) if a["chunks"][k] != b["chunks"][k]]
    assert diff == [1500 // 512] and a["hash"] != b["hash"]


def test_pins_catch_wrong_rotation(rng, monkeypatch):
    orig = fp._rotl
    monkeypatch.setattr(fp, "_rotl", lambda x, r: orig(x, 30 if r == 31 else r))  # the round rotates by 30
    with pytest.raises(AssertionError):
        test_xxh64_matches_library(rng, 40)
