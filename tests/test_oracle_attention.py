"""CPU pins of the decode-attention oracle (DCU decode page, sections 6.1
and 6.3): closed forms and invariants that a mistake in the definition,
the paging, the head mapping or the segment merge would break."""
import math

import numpy as np
import pytest

import oracle
import synth

BF = "bf16"


def _run(op, scale, **kw):
    return oracle.attention(op["Q"], op["K"], op["V"], op["block_table"], op["seq_lens"], op["B"],
                            op["Hq"], op["Hkv"], op["D"], op["block_size"], op["max_blocks"],
                            scale, **kw)


def _dec(bits):
    return oracle.decode(np.asarray(bits, np.uint16), BF)


def _row(op, cache, b, l, kvh):
    blk = op["block_table"][b, l // op["block_size"]]
    slot = l % op["block_size"]
    base = ((blk * op["block_size"] + slot) * op["Hkv"] + kvh) * op["D"]
    return cache[base:base + op["D"]]


def test_single_token_returns_its_value_row():
    op = synth.attention_operands(2, 4, 2, 16, [1, 1], 5, seed=1)
    r = _run(op, 0.3)
    for b in range(2):
        for h in range(4):
            want = _row(op, op["V"], b, 0, h // 2)
            assert np.array_equal(r.bits[(b * 4 + h) * 16:(b * 4 + h + 1) * 16], want)


def test_equal_keys_average_the_values():
    op = synth.attention_operands(1, 2, 1, 8, [37], 8, seed=2)
    # every cached key row equal: all scores equal, softmax uniform
    first = _row(op, op["K"], 0, 0, 0).copy()
    for l in range(37):
        blk = op["block_table"][0, l // 8]
        base = ((blk * 8 + l % 8) * 1) * 8
        op["K"][base:base + 8] = first
    r = _run(op, 0.7)
    vals = np.stack([_dec(_row(op, op["V"], 0, l, 0)) for l in range(37)])
    want = vals.mean(axis=0)
    for h in range(2):
        assert np.allclose(r.exact[h * 8:(h + 1) * 8], want, rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    D, L = 8, 20
    op = synth.attention_operands(1, 1, 1, D, [L], 4, seed=3)
    q = np.zeros(D); q[0] = 1.0
    op["Q"][:] = synth.to_bits(q, BF)
    for l in range(L):
        blk = op["block_table"][0, l // 4]
        base = (blk * 4 + l % 4) * D
        k = np.zeros(D); k[0] = 8.0 if l == 13 else 0.0
        op["K"][base:base + D] = synth.to_bits(k, BF)
    r = _run(op, 16.0)                 # score 128 against 0: weight 1 - O(e^-128)
    assert np.array_equal(r.bits, _row(op, op["V"], 0, 13, 0))


def test_brute_force_tiny_cases():
    for seed, (L, D, scale) in enumerate([(1, 1, 1.0), (2, 3, 0.5), (4, 2, 2.0), (3, 4, -1.0)]):
        op = synth.attention_operands(1, 1, 1, D, [L], 2, seed=10 + seed)
        r = _run(op, scale)
        q = _dec(op["Q"])
        ks = [_dec(_row(op, op["K"], 0, l, 0)) for l in range(L)]
        vs = [_dec(_row(op, op["V"], 0, l, 0)) for l in range(L)]
        s = [scale * math.fsum(q[d] * ks[l][d] for d in range(D)) for l in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        for d in range(D):
            want = math.fsum(w[l] * vs[l][d] for l in range(L)) / z
            assert abs(r.exact[d] - want) <= 1e-14 * max(1.0, abs(want))


def test_empty_sequence_gives_zero():
    op = synth.attention_operands(2, 2, 1, 8, [0, 5], 4, seed=4)
    r = _run(op, 1.0)
    assert np.all(r.bits[:16] == 0) and np.all(r.exact[:16] == 0)
    assert np.any(r.bits[16:] != 0)


def test_values_scale_exactly():
    # doubling V is exact in bfloat16 and doubles every output exactly
    op = synth.attention_operands(1, 4, 2, 16, [50], 7, seed=5)
    r1 = _run(op, 0.25)
    op2 = dict(op)
    op2["V"] = synth.to_bits(_dec(op["V"]) * 2.0, BF)
    r2 = _run(op2, 0.25)
    assert np.array_equal(r2.exact, 2.0 * r1.exact)


def test_paging_and_token_order_do_not_matter():
    # the same logical sequence stored in differently sized, scattered pages
    D, Hkv, L = 16, 2, 97
    rng = np.random.default_rng(6)
    keys = synth.to_bits(rng.normal(size=(L, Hkv, D)), BF)
    vals = synth.to_bits(rng.normal(size=(L, Hkv, D)), BF)
    Q = synth.to_bits(rng.normal(size=4 * D), BF)
    outs = []
    for bs in (1, 7, 784):
        nb = -(-L // bs)
        perm = rng.permutation(nb + 2)
        K = np.zeros((nb + 2) * bs * Hkv * D, np.uint16)
        V = np.zeros_like(K)
        for l in range(L):
            base = (perm[l // bs] * bs + l % bs) * Hkv * D
            K[base:base + Hkv * D] = keys[l].ravel()
            V[base:base + Hkv * D] = vals[l].ravel()
        bt = perm[:nb].reshape(1, nb).astype(np.int32)
        outs.append(oracle.attention(Q, K, V, bt, [L], 1, 4, Hkv, D, bs, nb, 0.25).exact)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # reversing the token order changes only the summation order
    bt = np.arange(L, dtype=np.int32)[::-1].reshape(1, L).copy()
    K = np.ascontiguousarray(keys.reshape(L, -1)).ravel()
    V = np.ascontiguousarray(vals.reshape(L, -1)).ravel()
    rev = oracle.attention(Q, K, V, bt, [L], 1, 4, Hkv, D, 1, L, 0.25).exact
    assert np.allclose(rev, outs[0], rtol=1e-12, atol=1e-14)


def test_query_heads_map_to_their_kv_head():
    # Hq = 6 over Hkv = 3: heads 2h and 2h+1 read kv head h
    op = synth.attention_operands(1, 6, 3, 8, [30], 8, seed=7)
    r = _run(op, 0.5)
    for h in range(6):
        kvh = h // 2
        K1 = np.concatenate([_row(op, op["K"], 0, l, kvh) for l in range(30)])
        V1 = np.concatenate([_row(op, op["V"], 0, l, kvh) for l in range(30)])
        q1 = op["Q"][h * 8:(h + 1) * 8]
        one = oracle.attention(q1, K1, V1, np.arange(30, dtype=np.int32).reshape(1, 30), [30],
                               1, 1, 1, 8, 1, 30, 0.5)
        assert np.array_equal(one.exact, r.exact[h * 8:(h + 1) * 8])


@pytest.mark.parametrize("nseg", [1, 2, 3, 16, 32, 150])
def test_segmented_merge_equals_the_definition(nseg):
    # the page's segmented algorithm (local max / sum / PV, global merge)
    # is the softmax, rearranged: equal up to double rounding, including
    # more segments than tokens (empty segments)
    op = synth.attention_operands(2, 4, 2, 32, [100, 37], 16, seed=8)
    r = _run(op, 0.2)
    bits, ex = oracle.attention_segmented(op["Q"], op["K"], op["V"], op["block_table"],
                                          op["seq_lens"], 2, 4, 2, 32, 16, op["max_blocks"],
                                          0.2, nseg)
    assert np.allclose(ex, r.exact, rtol=1e-12, atol=1e-14)


def _fp32_segmented(op, scale, nseg, drop=None):
    """FP32 evaluation of the segmented algorithm (positive control); drop:
    segment index left out (negative control)."""
    f32 = np.float32
    B, Hq, Hkv, D = op["B"], op["Hq"], op["Hkv"], op["D"]
    out = np.zeros(B * Hq * D, np.float64)
    for b in range(B):
        L = int(op["seq_lens"][b])
        seg = -(-L // nseg)
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            q = _dec(op["Q"][(b * Hq + h) * D:(b * Hq + h + 1) * D]).astype(f32)
            ms, ls, os_ = [], [], []
            for i in range(nseg):
                l0, l1 = i * seg, min(L, (i + 1) * seg)
                if l0 >= l1 or i == drop:
                    continue
                K = np.stack([_dec(_row(op, op["K"], b, l, kvh)) for l in range(l0, l1)]).astype(f32)
                V = np.stack([_dec(_row(op, op["V"], b, l, kvh)) for l in range(l0, l1)]).astype(f32)
                s = (K @ q) * f32(scale)
                m = s.max()
                p = np.exp(s - m).astype(f32)
                ms.append(m); ls.append(p.sum(dtype=f32)); os_.append((p[:, None] * V).sum(0, dtype=f32))
            M = max(ms)
            w = [np.exp(f32(m - M)) for m in ms]
            z = sum(f32(lv * wv) for lv, wv in zip(ls, w))
            o = sum(ov * wv for ov, wv in zip(os_, w)) / z
            out[(b * Hq + h) * D:(b * Hq + h + 1) * D] = o
    return out


def test_tolerance_controls():
    op = synth.attention_operands(2, 4, 2, 64, [300, 81], 16, seed=9)
    scale = 1 / 8.0
    ref = _run(op, scale)
    rel = oracle.attention_rel(ref, op["seq_lens"], 4, 64)
    assert np.all(rel < 1e-3)
    good = synth.to_bits(_fp32_segmented(op, scale, 16), BF)
    ok, rep = oracle.check(good, ref, BF, rel=rel)
    assert ok, rep
    # a segment left out of the merge, or outputs off by 1% of S: rejected
    bad = synth.to_bits(_fp32_segmented(op, scale, 16, drop=3), BF)
    assert not oracle.check(bad, ref, BF, rel=rel)[0]
    off = synth.to_bits(ref.exact + 1e-2 * ref.sabs, BF)
    assert not oracle.check(off, ref, BF, rel=rel)[0]


# ---- exact-class inputs at the DCU page's head shape (section 7: 16 query /
# 4 KV heads, head dim 256, pages of 784, 8K-32K cached tokens).  Every
# correct implementation with FP32 sums returns these outputs bit for bit,
# so the GPU test compares bits; the controls below show that the
# comparison sees one missing, extra or misread token.

EXACT_W = synth.WORKLOADS["attention_decode_16q4kv_d256_bf16"]


def _exact_ref(op):
    return _run(op, 1.0 / math.sqrt(EXACT_W["D"]))


@pytest.mark.parametrize("kind", ["uniform", "mask"])
@pytest.mark.parametrize("L", [8192, 32768])
def test_exact_class_matches_closed_form(kind, L):
    from helpers import attention_exact_expected
    op = synth.attention_exact_operands(L, kind)
    ref = _exact_ref(op)
    assert np.array_equal(ref.bits, attention_exact_expected(op, EXACT_W["Hq"], EXACT_W["D"]))


def test_exact_class_controls_fail_the_bit_comparison():
    """Outputs of the oracle on altered inputs differ from the true ones in
    their bits: the last 64 tokens dropped, the last token dropped, a token
    on a page boundary replaced by its neighbour, one masked token counted."""
    from helpers import exact_mismatches
    L, bs = 32768, EXACT_W["block_size"]
    op = synth.attention_exact_operands(L, "uniform")
    ref = _exact_ref(op)
    for drop in (64, 1):
        short = dict(op, seq_lens=np.array([L - drop], np.int32))
        assert exact_mismatches(_exact_ref(short).bits, ref.bits) > 0, drop
    # token 784 (first of the second page) read as token 783
    V = op["V"].reshape(-1, EXACT_W["Hkv"], EXACT_W["D"]).copy()
    bt = op["block_table"][0]
    V[bt[1] * bs + 0] = V[bt[0] * bs + bs - 1]
    assert exact_mismatches(_exact_ref(dict(op, V=V.reshape(-1))).bits, ref.bits) > 0
    # mask class: one token that should score -inf-like counted
    opm = synth.attention_exact_operands(8192, "mask")
    refm = _exact_ref(opm)
    t = int(np.flatnonzero(~opm["counted"][2])[0])
    K = opm["K"].reshape(-1, EXACT_W["Hkv"], EXACT_W["D"]).copy()
    K[opm["block_table"][0][t // bs] * bs + t % bs, 2, :] = 0
    assert exact_mismatches(_exact_ref(dict(opm, K=K.reshape(-1))).bits, refm.bits) > 0
