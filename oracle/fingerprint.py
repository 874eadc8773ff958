"""Plain-Python reference for the library's buffer fingerprints.

TEST INFRASTRUCTURE ONLY, like the rest of this package.  It shares no code
with the HIP library.

Source: the Megatron Core bitwise-determinism news item (news.hamidun.com),
"debugging methodology": tensors are fingerprinted on the GPU (with their
shape, dtype and element count recorded), chunk-wise for order-sensitive data,
and the first iteration, rank and kernel whose fingerprints differ between two
runs is narrowed down step by step.

The page does not fix a hash function.  The library uses XXH64 with seed 0,
written here from its published specification (xxHash, "XXH64 algorithm
description": five 64-bit primes; four accumulators over 32-byte stripes,
each round acc = rotl(acc + lane * P2, 31) * P1; merge, length, tail words,
tail 4-byte word and tail bytes; final avalanche).  A buffer of n bytes in
chunks of c bytes has ceil(n / c) chunks (one empty chunk when n = 0), chunk
k holding bytes [k c, min(n, (k + 1) c)); its fingerprint is XXH64 of the
chunk hashes written as little-endian 64-bit words in chunk order.
"""
from __future__ import annotations

from typing import Dict, List

M64 = (1 << 64) - 1
P1 = 0x9E3779B185EBCA87
P2 = 0xC2B2AE3D27D4EB4F
P3 = 0x165667B19E3779F9
P4 = 0x85EBCA77C2B2AE63
P5 = 0x27D4EB2F165667C5


def _rotl(x: int, r: int) -> int:
    return ((x << r) | (x >> (64 - r))) & M64


def _round(acc: int, lane: int) -> int:
    acc = (acc + lane * P2) & M64
    return (_rotl(acc, 31) * P1) & M64


def _merge(h: int, acc: int) -> int:
    h ^= _round(0, acc)
    return (h * P1 + P4) & M64


def _u64(data: bytes, i: int) -> int:
    return int.from_bytes(data[i:i + 8], "little")


def xxh64(data: bytes, seed: int = 0) -> int:
    """XXH64 of ``data`` as an unsigned 64-bit integer."""
    n = len(data)
    i = 0
    if n >= 32:
        v = [(seed + P1 + P2) & M64, (seed + P2) & M64, seed & M64, (seed - P1) & M64]
        while i + 32 <= n:
            for k in range(4):
                v[k] = _round(v[k], _u64(data, i + 8 * k))
            i += 32
        h = (_rotl(v[0], 1) + _rotl(v[1], 7) + _rotl(v[2], 12) + _rotl(v[3], 18)) & M64
        for k in range(4):
            h = _merge(h, v[k])
    else:
        h = (seed + P5) & M64
    h = (h + n) & M64
    while i + 8 <= n:
        h ^= _round(0, _u64(data, i))
        h = (_rotl(h, 27) * P1 + P4) & M64
        i += 8
    if i + 4 <= n:
        h ^= (int.from_bytes(data[i:i + 4], "little") * P1) & M64
        h = (_rotl(h, 23) * P2 + P3) & M64
        i += 4
    while i < n:
        h ^= (data[i] * P5) & M64
        h = (_rotl(h, 11) * P1) & M64
        i += 1
    h ^= h >> 33
    h = (h * P2) & M64
    h ^= h >> 29
    h = (h * P3) & M64
    h ^= h >> 32
    return h


def chunk_count(nbytes: int, chunk: int) -> int:
    return max(1, -(-nbytes // chunk))


def fingerprint(data: bytes, chunk: int) -> Dict[str, object]:
    """Chunk hashes and the whole-buffer fingerprint, as defined in the module header."""
    n = len(data)
    chunks: List[int] = [xxh64(data[k * chunk:min(n, (k + 1) * chunk)]) for k in range(chunk_count(n, chunk))]
    whole = xxh64(b"".join(c.to_bytes(8, "little") for c in chunks))
    return {"hash": whole, "chunks": chunks}
