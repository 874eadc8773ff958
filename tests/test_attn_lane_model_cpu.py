"""Lane-exact model of the attention kernels' index arithmetic (CPU only).

The attention core kernels (attention.hip) rest on three facts about gfx950:
  * v_mfma_f32_16x16x32_bf16: lane l supplies row l%16, k = 8(l/16) .. +7 of
    its first operand and column l%16 of its second, and receives
    D[4(l/16) + r][l%16], r = 0..3;
  * ds_read_b64_tr_b16: within each group of 16 lanes, result lane i takes
    element i%4 of the 8 bytes that source lane i/4 + 4e addressed (the
    mapping measured with a probe on the GPU);
  * bf16 operands, fp32 accumulation.
This test re-enacts, lane by lane, the forward kernel and the two backward
kernels (dK/dV over key blocks, dQ over query blocks) with those semantics:
the same fragment addresses, LDS tile layout, key permutation of P and dS,
masks and online softmax.  With exact arithmetic the model must reproduce
the oracle's attention and torch's attention gradients to rounding, for
every head size the kernels are built for, causal and not, with ragged
sequence lengths.  It checks the design of the kernels' indexing; it does
not run the HIP code.
"""
import math

import numpy as np
import pytest
import torch

from megatron_tensor_transformer_mlp_amd import inputs
from oracle import attn

BM, BN = 128, 64


def mfma(src0, src1, acc):
    """src0, src1: [64][8]; acc [64][4].  D = A0 @ B1 with lane l holding A0[l%16][8g+e], B1[8g+e][l%16];
    lane l gets D[4g + r][l%16]."""
    A0 = np.zeros((16, 32)); B1 = np.zeros((32, 16))
    for l in range(64):
        g, i = l // 16, l % 16
        A0[i, 8 * g:8 * g + 8] = src0[l]
        B1[8 * g:8 * g + 8, i] = src1[l]
    D = A0 @ B1
    out = acc.copy()
    for l in range(64):
        g = l // 16
        for r in range(4):
            out[l, r] += D[4 * g + r, l % 16]
    return out


class Lds:
    def __init__(self, nbytes):
        self.b = np.zeros(nbytes // 2)  # bf16 elements as float
    def write16(self, addr, vals8):
        assert addr % 16 == 0
        self.b[addr // 2:addr // 2 + 8] = vals8
    def read_b128(self, addr):
        assert addr % 16 == 0
        return self.b[addr // 2:addr // 2 + 8].copy()
    def read_tr(self, addrs):
        """ds_read_b64_tr_b16: result lane i (group G) elem e = src[16G + i//4 + 4e][i%4]."""
        src = [self.b[a // 2:a // 2 + 4] for a in addrs]
        for a in addrs:
            assert a % 8 == 0
        out = np.zeros((64, 4))
        for l in range(64):
            G, i = l // 16, l % 16
            for e in range(4):
                out[l, e] = src[16 * G + i // 4 + 4 * e][i % 4]
        return out


def chunk_off(r, c, pitch):
    """Byte offset of 16-byte chunk c of tile row r (rows padded to `pitch`)."""
    return r * pitch + 16 * c


def quad_off(r, col, pitch):
    """Byte offset of columns col..col+3 (col a multiple of 4) of tile row r."""
    return chunk_off(r, col >> 3, pitch) + 2 * (col & 7)


def tile_pitch(D):
    return 2 * D + 16


def bf16r(x):
    return inputs.bf16_bits_to_f32(inputs.round_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def model_fwd(QKV, b, s, n, d, causal, round_p=True, stats=None):
    D = ((d + 31) // 32) * 32
    KD, ND = D // 32, D // 16
    pitch = tile_pitch(D)
    ld = 3 * n * d
    T = b * s
    O = np.full((T, n * d), np.nan)
    lse = np.full((n, T), np.nan)
    scale_log2 = math.log2(math.e) / math.sqrt(d)

    def tile_load(lds, base_col, bi, row0):
        for tid in range(256):
            for u in range(D // 32):
                i = tid + 256 * u
                row, c = i // (D // 8), i % (D // 8)
                ok = row0 + row < s and c * 8 < d
                vals = QKV[bi * s + row0 + row, base_col + c * 8: base_col + c * 8 + 8] if ok else np.zeros(8)
                lds.write16(chunk_off(row, c, pitch), vals)

    for bi in range(b):
        for j in range(n):
            for qb in range((s + BM - 1) // BM):
                q0 = qb * BM
                kv_end = min(s, q0 + BM) if causal else s
                nkb = (kv_end + BN - 1) // BN
                for w in range(4):
                    qf = np.zeros((2, KD, 64, 8))
                    for rb in range(2):
                        for l in range(64):
                            row = q0 + 32 * w + 16 * rb + l % 16
                            for kk in range(KD):
                                c = kk * 4 + l // 16
                                if row < s and c * 8 < d:
                                    qf[rb, kk, l] = QKV[bi * s + row, j * d + c * 8: j * d + c * 8 + 8]
                    o = np.zeros((2, ND, 64, 4)); m = np.full((2, 64), -np.inf); nm = np.zeros((2, 64))
                    lsum = np.zeros((2, 64))  # per lane: its own keys only, merged over the row after the last step
                    for kb in range(nkb):
                        kt, vt = Lds(BN * pitch), Lds(BN * pitch)
                        tile_load(kt, n * d + j * d, bi, kb * BN)
                        tile_load(vt, 2 * n * d + j * d, bi, kb * BN)
                        kbase = kb * BN
                        for rb in range(2):
                            sacc = np.zeros((4, 64, 4))
                            for kb16 in range(4):
                                for kk in range(KD):
                                    kfrag = np.array([kt.read_b128(chunk_off(kb16 * 16 + l % 16, kk * 4 + l // 16, pitch))
                                                      for l in range(64)])
                                    sacc[kb16] = mfma(kfrag, qf[rb, kk], sacc[kb16])
                            qw = q0 + 32 * w + 16 * rb
                            masked = kbase + BN > s or (causal and kbase + BN - 1 > qw)
                            sv = sacc.copy()
                            for l in range(64):
                                q = qw + l % 16
                                key0 = kbase + 4 * (l // 16)
                                lim = (min(q, s - 1) if causal else s - 1) - key0
                                for kb16 in range(4):
                                    for r in range(4):
                                        key = key0 + kb16 * 16 + r
                                        valid = key < s and (not causal or key <= q)
                                        assert valid == (kb16 * 16 + r <= lim)
                                        # a step the kernel runs unmasked has every key valid for every row
                                        assert masked or valid
                                        if masked and not valid:
                                            sv[kb16, l, r] = -np.inf
                            lm = sv.max(axis=(0, 2)) * scale_log2  # per lane
                            if np.any(lm > m[rb] + 8.0):  # one decision for the whole wave
                                if stats is not None and kb > 0:
                                    stats["late_rescales"] = stats.get("late_rescales", 0) + 1
                                mxr = np.array([max(lm[l], lm[l ^ 16], lm[l ^ 32], lm[l ^ 48]) for l in range(64)])
                                mnew = np.maximum(m[rb], mxr)
                                corr = np.where(mnew == -np.inf, 1.0, np.exp2(m[rb] - mnew))
                                lsum[rb] *= corr
                                o[rb] *= corr[None, :, None]
                                m[rb] = mnew
                                nm[rb] = np.where(mnew == -np.inf, 0.0, -mnew)
                            p = np.exp2(sv * scale_log2 + nm[rb][None, :, None])
                            assert p.max() <= 2.0 ** 8
                            if stats is not None:
                                stats["max_p"] = max(stats.get("max_p", 0.0), float(p.max()))
                            lsum[rb] += p.sum(axis=(0, 2))
                            pr = bf16r(p) if round_p else p
                            pf = np.zeros((2, 64, 8))
                            for c in range(2):
                                pf[c, :, 0:4] = pr[2 * c]
                                pf[c, :, 4:8] = pr[2 * c + 1]
                            for nb in range(ND):
                                for c in range(2):
                                    lo = vt.read_tr([quad_off(32 * c + 4 * (l // 16) + ((l % 16) >> 2),
                                                              16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)])
                                    hi = vt.read_tr([quad_off(32 * c + 16 + 4 * (l // 16) + ((l % 16) >> 2),
                                                              16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)])
                                    vf = np.concatenate([lo, hi], axis=1)
                                    o[rb, nb] = mfma(vf, pf[c], o[rb, nb])
                    for rb in range(2):
                        lrow = np.array([lsum[rb, l] + lsum[rb, l ^ 16] + lsum[rb, l ^ 32] + lsum[rb, l ^ 48]
                                         for l in range(64)])
                        for l in range(64):
                            q = q0 + 32 * w + 16 * rb + l % 16
                            if q >= s:
                                continue
                            inv = 1.0 / lrow[l]
                            for nb in range(ND):
                                col = 16 * nb + 4 * (l // 16)
                                if col < d:
                                    O[bi * s + q, j * d + col:j * d + col + 4] = o[rb, nb, l] * inv
                            if l // 16 == 0:
                                lse[j, bi * s + q] = (m[rb, l] + math.log2(lrow[l])) * math.log(2)
    return O, lse



def tile_load(lds, src, s, d, D, pitch, row0):
    """src: [s, d] rows of one sequence/head block."""
    for tid in range(256):
        for u in range(D // 32):
            i = tid + 256 * u
            row, c = i // (D // 8), i % (D // 8)
            ok = row0 + row < s and c * 8 < d
            vals = src[row0 + row, c * 8:c * 8 + 8] if ok else np.zeros(8)
            lds.write16(chunk_off(row, c, pitch), vals)


def kfrag_rows(src, rows_fn, kk, s, d):
    """Register fragments: lane l holds src[row(l)][32kk + 8g .. +7] (zeros out of range)."""
    out = np.zeros((64, 8))
    for l in range(64):
        row, c = rows_fn(l), kk * 4 + l // 16
        if row < s and c * 8 < d:
            out[l] = src[row, c * 8:c * 8 + 8]
    return out


def dkdv(Qs, Ks, Vs, dOs, lse, delta, s, d, causal, rnd):
    """One (sequence, head): returns dK, dV [s, d]."""
    D = ((d + 31) // 32) * 32; KD, ND = D // 32, D // 16; pitch = tile_pitch(D)
    scale_log2 = math.log2(math.e) / math.sqrt(d)
    dK = np.full((s, d), np.nan); dV = np.full((s, d), np.nan)
    for kb in range((s + BN - 1) // BN):
        k0 = kb * BN
        for w in range(4):
            key_of = lambda l: k0 + 16 * w + l % 16
            kf = [kfrag_rows(Ks, key_of, kk, s, d) for kk in range(KD)]
            vf = [kfrag_rows(Vs, key_of, kk, s, d) for kk in range(KD)]
            dk = np.zeros((ND, 64, 4)); dv = np.zeros((ND, 64, 4))
            qstart = k0 if causal else 0
            nqb = (s - qstart + BN - 1) // BN if qstart < s else 0
            for qb in range(nqb):
                qbase = qstart + qb * BN
                Qt, Dt = Lds(BN * pitch), Lds(BN * pitch)
                tile_load(Qt, Qs, s, d, D, pitch, qbase); tile_load(Dt, dOs, s, d, D, pitch, qbase)
                sl = np.array([lse[qbase + i] * math.log2(math.e) if qbase + i < s else 0 for i in range(BN)])
                sd = np.array([delta[qbase + i] if qbase + i < s else 0 for i in range(BN)])
                p = np.zeros((4, 64, 4)); ds = np.zeros((4, 64, 4))
                masked = qbase + BN > s or (causal and qbase < k0 + 16 * w + 15)
                for qb16 in range(4):
                    sacc = np.zeros((64, 4)); dpacc = np.zeros((64, 4))
                    for kk in range(KD):
                        offs = [chunk_off(qb16 * 16 + l % 16, kk * 4 + l // 16, pitch) for l in range(64)]
                        sacc = mfma(np.array([Qt.read_b128(o) for o in offs]), kf[kk], sacc)
                        dpacc = mfma(np.array([Dt.read_b128(o) for o in offs]), vf[kk], dpacc)
                    for l in range(64):
                        key = key_of(l)
                        lo = key - qbase - 4 * (l // 16) if causal else 0
                        hi = s - qbase - 4 * (l // 16)
                        for r in range(4):
                            ql = qb16 * 16 + 4 * (l // 16) + r
                            q = qbase + ql
                            ok = lo <= qb16 * 16 + r < hi  # the kernel's test; keys past the end are not stored
                            if key < s:
                                assert ok == (q < s and (not causal or key <= q))
                            assert masked or ok  # a step the kernel runs unmasked has every element valid
                            pv = 2.0 ** (sacc[l, r] * scale_log2 - sl[ql])
                            p[qb16, l, r] = 0.0 if masked and not ok else pv
                            ds[qb16, l, r] = p[qb16, l, r] * (dpacc[l, r] - sd[ql])
                pr, dsr = (bf16r(p), bf16r(ds)) if rnd else (p, ds)
                pf = np.zeros((2, 64, 8)); dsf = np.zeros((2, 64, 8))
                for c in range(2):
                    pf[c, :, :4], pf[c, :, 4:] = pr[2 * c], pr[2 * c + 1]
                    dsf[c, :, :4], dsf[c, :, 4:] = dsr[2 * c], dsr[2 * c + 1]
                for nb in range(ND):
                    for c in range(2):
                        a0 = [quad_off(32 * c + 4 * (l // 16) + ((l % 16) >> 2), 16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)]
                        a1 = [quad_off(32 * c + 16 + 4 * (l // 16) + ((l % 16) >> 2), 16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)]
                        dv[nb] = mfma(np.concatenate([Dt.read_tr(a0), Dt.read_tr(a1)], axis=1), pf[c], dv[nb])
                        dk[nb] = mfma(np.concatenate([Qt.read_tr(a0), Qt.read_tr(a1)], axis=1), dsf[c], dk[nb])
            for l in range(64):
                key = key_of(l)
                if key >= s:
                    continue
                for nb in range(ND):
                    col = 16 * nb + 4 * (l // 16)
                    if col < d:
                        dK[key, col:col + 4] = dk[nb, l] / math.sqrt(d)
                        dV[key, col:col + 4] = dv[nb, l]
    return dK, dV


def dq(Qs, Ks, Vs, dOs, Os, lse, delta, s, d, causal, rnd):
    """delta is formed here as the dQ kernel forms it (per-lane partial dot products of dO and O over the
    lane's columns, merged over the row's four lanes) and checked against the one given."""
    D = ((d + 31) // 32) * 32; KD, ND = D // 32, D // 16; pitch = tile_pitch(D)
    scale_log2 = math.log2(math.e) / math.sqrt(d)
    dQ = np.full((s, d), np.nan)
    for qbk in range((s + BM - 1) // BM):
        q0 = qbk * BM
        kv_end = min(s, q0 + BM) if causal else s
        nkb = (kv_end + BN - 1) // BN
        for w in range(4):
            accs = np.zeros((2, ND, 64, 4))
            for rb in range(2):
                row_of = lambda l: q0 + 32 * w + 16 * rb + l % 16
                qf = [kfrag_rows(Qs, row_of, kk, s, d) for kk in range(KD)]
                df = [kfrag_rows(dOs, row_of, kk, s, d) for kk in range(KD)]
                lq = np.array([lse[row_of(l)] * math.log2(math.e) if row_of(l) < s else 0 for l in range(64)])
                of = [kfrag_rows(Os, row_of, kk, s, d) for kk in range(KD)]
                part = sum((df[kk] * of[kk]).sum(axis=1) for kk in range(KD))
                dl = np.array([part[l] + part[l ^ 16] + part[l ^ 32] + part[l ^ 48] for l in range(64)])
                for l in range(64):
                    if row_of(l) < s:
                        assert abs(dl[l] - delta[row_of(l)]) <= 1e-12 * (1 + abs(delta[row_of(l)]))
                    else:
                        assert dl[l] == 0.0
                for kb in range(nkb):
                    Kt, Vt = Lds(BN * pitch), Lds(BN * pitch)
                    tile_load(Kt, Ks, s, d, D, pitch, kb * BN); tile_load(Vt, Vs, s, d, D, pitch, kb * BN)
                    ds = np.zeros((4, 64, 4))
                    kbase = kb * BN
                    qw = q0 + 32 * w + 16 * rb
                    masked = kbase + BN > s or (causal and kbase + BN - 1 > qw)
                    for kb16 in range(4):
                        sacc = np.zeros((64, 4)); dpacc = np.zeros((64, 4))
                        for kk in range(KD):
                            offs = [chunk_off(kb16 * 16 + l % 16, kk * 4 + l // 16, pitch) for l in range(64)]
                            sacc = mfma(np.array([Kt.read_b128(o) for o in offs]), qf[kk], sacc)
                            dpacc = mfma(np.array([Vt.read_b128(o) for o in offs]), df[kk], dpacc)
                        for l in range(64):
                            q = row_of(l)
                            lim = (min(q, s - 1) if causal else s - 1) - kbase - 4 * (l // 16)
                            for r in range(4):
                                key = kbase + kb16 * 16 + 4 * (l // 16) + r
                                ok = kb16 * 16 + r <= lim  # the kernel's test; rows past the end are not stored
                                if q < s:
                                    assert ok == (key < s and (not causal or key <= q))
                                assert masked or ok  # a step the kernel runs unmasked has every element valid
                                pv = 2.0 ** (sacc[l, r] * scale_log2 - lq[l])
                                if masked and not ok:
                                    pv = 0.0
                                ds[kb16, l, r] = pv * (dpacc[l, r] - dl[l])
                    dsr = bf16r(ds) if rnd else ds
                    dsf = np.zeros((2, 64, 8))
                    for c in range(2):
                        dsf[c, :, :4], dsf[c, :, 4:] = dsr[2 * c], dsr[2 * c + 1]
                    for nb in range(ND):
                        for c in range(2):
                            a0 = [quad_off(32 * c + 4 * (l // 16) + ((l % 16) >> 2), 16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)]
                            a1 = [quad_off(32 * c + 16 + 4 * (l // 16) + ((l % 16) >> 2), 16 * nb + 4 * ((l % 16) & 3), pitch) for l in range(64)]
                            accs[rb, nb] = mfma(np.concatenate([Kt.read_tr(a0), Kt.read_tr(a1)], axis=1), dsf[c], accs[rb, nb])
                for l in range(64):
                    q = row_of(l)
                    if q >= s:
                        continue
                    for nb in range(ND):
                        col = 16 * nb + 4 * (l // 16)
                        if col < d:
                            dQ[q, col:col + 4] = accs[rb, nb, l] / math.sqrt(d)
    return dQ




def growing_keys(QKV, b, s, n, d, rate):
    """K rows scaled by 1 + rate * position: later key blocks score far above the first, so the running max
    must be raised (and O rescaled) after the first step, while other steps stay within the slack."""
    X = QKV.copy()
    f = np.tile(1.0 + rate * np.arange(s), b)[:, None]
    X[:, n * d:2 * n * d] = bf16r(X[:, n * d:2 * n * d] * f)
    return X


@pytest.mark.parametrize("b,s,n,d,causal,rate", [(2, 70, 2, 32, True, 0), (1, 130, 1, 64, False, 0),
                                                 (1, 64, 1, 16, True, 0), (1, 96, 1, 96, True, 0),
                                                 (1, 64, 1, 128, False, 0), (1, 200, 1, 64, True, 0.02),
                                                 (1, 200, 1, 32, False, 0.125)])
def test_forward_model_is_exact(b, s, n, d, causal, rate):
    rng = np.random.default_rng(s * d)
    QKV = growing_keys(bf16r(rng.standard_normal((b * s, 3 * n * d))), b, s, n, d, rate)
    stats = {}
    O, lse = model_fwd(QKV, b, s, n, d, causal, round_p=False, stats=stats)
    if rate:  # both branches of the lazy rescale are taken
        assert stats["late_rescales"] > 0 and stats["max_p"] > 1.0
    want = attn.attention_core(QKV[:, :n * d], QKV[:, n * d:2 * n * d], QKV[:, 2 * n * d:], n, d, b, s, causal)
    np.testing.assert_allclose(O, want["O"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, want["lse"], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("s,d,causal", [(70, 16, True), (130, 64, False), (96, 96, True), (64, 128, False)])
def test_backward_model_is_exact(s, d, causal):
    rng = np.random.default_rng(s + d)
    Q, K, V, dO = (bf16r(rng.standard_normal((s, d))) for _ in range(4))
    Qt, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    Ot = torch.nn.functional.scaled_dot_product_attention(Qt[None, None], Kt[None, None], Vt[None, None],
                                                          is_causal=causal)[0, 0]
    (Ot * torch.tensor(dO)).sum().backward()
    w = attn.attention_core(Q, K, V, 1, d, 1, s, causal)
    delta = (dO * w["O"]).sum(axis=1)
    dK, dV = dkdv(Q, K, V, dO, w["lse"][0], delta, s, d, causal, False)
    dQ = dq(Q, K, V, dO, w["O"], w["lse"][0], delta, s, d, causal, False)
    for got, want in ((dQ, Qt.grad), (dK, Kt.grad), (dV, Vt.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_tile_layout_banks(D):
    """The kernels' LDS accesses of a tile under the bank model of gfx950's LDS (128 bytes per cycle: a
    16-byte access serves 8 lanes per cycle, an 8-byte access 16).  The layout is a bijection of the
    tile's chunks; the 16-byte fragment reads touch distinct bytes modulo 128 in every cycle; the
    transposing reads touch each byte at most twice (neighbouring rows share one 16-byte slot)."""
    pitch = tile_pitch(D)
    chunks = D // 8
    offs = {chunk_off(r, c, pitch) for r in range(BN) for c in range(chunks)}
    assert len(offs) == BN * chunks and max(offs) + 16 <= BN * pitch

    def most_shared(addrs, width):
        count = np.zeros(128, int)
        for a in addrs:
            assert a % 128 + width <= 128
            count[a % 128:a % 128 + width] += 1
        return count.max()

    for base in range(0, BN, 16):  # 16-byte reads: lane l reads row base + l%16, chunk 4kk + l/16
        for kk in range(D // 32):
            addrs = [chunk_off(base + l % 16, 4 * kk + l // 16, pitch) for l in range(64)]
            for grp in range(0, 64, 8):
                assert most_shared(addrs[grp:grp + 8], 16) == 1, (base, kk, grp)
    for c in range(2):  # transposing reads: lane l reads row 32c (+16) + 4(l/16) + (l%16)/4, columns 16nb + 4(l%4)
        for half in (0, 16):
            for nb in range(D // 16):
                addrs = [quad_off(32 * c + half + 4 * (l // 16) + ((l % 16) >> 2), 16 * nb + 4 * ((l % 16) & 3), pitch)
                         for l in range(64)]
                for grp in range(0, 64, 16):
                    assert most_shared(addrs[grp:grp + 16], 8) <= 2, (c, half, nb, grp)
