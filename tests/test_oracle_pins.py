"""Pins of the CPU oracle to facts outside itself (CPU only, no GPU).

Each test ties one oracle function to something the pages print, a closed form,
an invariant the pages state, a library routine, or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _bf16_from_torch(x: np.ndarray) -> np.ndarray:
    """torch's float32 -> bfloat16 conversion (round to nearest even), as bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rand_store(shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return O.round_store(x, dtype)


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------


def test_bf16_rounding_matches_torch_on_float32():
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),   # subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, np.inf, -np.inf],
                 dtype=np.float32),
    ])
    # exact ties: low half 0x8000 above an even and an odd bf16
    hi = rng.integers(0x0080, 0x7F00, 4000).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(O.bf16_round_bits(x), _bf16_from_torch(x))


def test_bf16_rounding_of_float64_is_single_rounding():
    # 1 + 2^-8 + 2^-40 lies just above the tie between 1 and 1 + 2^-7: one rounding
    # goes up; rounding to float32 first would land on the tie and go to even.
    assert O.bf16_round_bits(np.float64(1 + 2**-8 + 2**-40)) == 0x3F81
    assert O.bf16_round_bits(np.float64(1 + 2**-8)) == 0x3F80          # tie -> even
    assert O.bf16_round_bits(np.float64(1 + 3 * 2**-8)) == 0x3F82      # tie -> even (up)
    assert O.bf16_round_bits(np.float64(-(1 + 2**-8 + 2**-40))) == 0xBF81
    assert O.bf16_round_bits(np.float64(np.nan)) & 0x7FC0 == 0x7FC0
    assert O.bf16_to_f32(np.uint16(0x3F80)) == 1.0


def bf16_rne_exact(x: float) -> int:
    """Round-to-nearest-even of a float64 value to bfloat16 bits, from the
    definition in exact rational arithmetic: bfloat16 keeps 8 significant bits
    (exponent range of float32, subnormals below 2^-126), the nearer
    representable neighbour wins, a tie goes to the even significand, and a
    value at or past halfway above the largest finite one becomes infinity."""
    from fractions import Fraction
    import struct
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    if math.isinf(x):
        return sign | 0x7F80
    a = Fraction(abs(x))
    if a == 0:
        return sign
    e = math.frexp(abs(x))[1] - 1              # 2^e <= |x| < 2^(e+1)
    e = max(e, -126)                           # subnormals share the last normal binade's spacing
    ulp = Fraction(2) ** (e - 7)
    n, rem = divmod(a, ulp)
    if 2 * rem > ulp or (2 * rem == ulp and n % 2 == 1):
        n += 1
    v = n * ulp
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]   # v is a bfloat16 value: exact in float32
    return sign | (bits >> 16)


def bf16_exact_inputs(rng, n: int) -> np.ndarray:
    """float64 values across the whole range, with many exactly halfway between
    two bfloat16 values and many a hair (far below a float32 ulp) to either
    side of such a midpoint, where rounding through float32 first goes wrong."""
    mags = 10.0 ** rng.uniform(-44, 38.5, n)
    plain = mags * rng.choice([-1.0, 1.0], n)
    hi = rng.integers(0x0001, 0x7F7F, n).astype(np.uint32)
    lower = (hi << 16).view(np.float32).astype(np.float64)
    upper = ((hi + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lower + upper) / 2                                    # exact in float64
    hair = (upper - lower) * 2.0 ** -35
    sgn = rng.choice([-1.0, 1.0], n)
    return np.concatenate([plain, sgn * mid, sgn * (mid + hair), sgn * (mid - hair),
                           [2.0 ** 128 * (1 - 2.0 ** -9), 2.0 ** 128 * (1 - 2.0 ** -10), 2.0 ** -133, 2.0 ** -134,
                            3 * 2.0 ** -135, 0.0, -0.0, np.inf, -np.inf]])


def test_bf16_rounding_of_float64_matches_exact_rational_rounding():
    """One rounding from float64, checked against exact rational arithmetic on
    random values of every magnitude, on exact midpoints and just beside them,
    at the overflow threshold and in the subnormal range."""
    r = np.random.default_rng(77)
    x = bf16_exact_inputs(r, 4000)
    want = np.array([bf16_rne_exact(float(v)) for v in x], dtype=np.uint16)
    got = O.bf16_round_bits(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:5]]


# ---------------------------------------------------------------------------
# RoPE table and rotation
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("d", [16, 128])
def test_rope_table_closed_forms(d):
    c, s = O.rope_table(40, d, 10000.0)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    # pair 0 turns by exactly one radian per position
    for p in (1, 7, 39):
        assert c[p, 0] == np.float32(math.cos(p)) and s[p, 0] == np.float32(math.sin(p))
    # last pair: base^(-(d-2)/d)
    th = 10000.0 ** (-(d - 2) / d)
    assert c[3, d // 2 - 1] == np.float32(math.cos(3 * th))
    # the workload generator produces the same table, bit for bit
    wc, ws = W.rotation_table(40, d, 10000.0)
    assert np.array_equal(wc.numpy(), c) and np.array_equal(ws.numpy(), s)


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_position_zero_is_identity(style, dtype):
    c, s = O.rope_table(1, 64)
    x = _rand_store((5, 64), dtype)
    assert np.array_equal(O.rope_rotate(x, dtype, c[0], s[0], style), x)


def test_rope_quarter_turn_sign():
    # c = 0, s = 1 turns (x0, x1) into (-x1, x0) exactly: pins direction and pairing
    d = 4
    x = np.array([1.5, -2.25, 3.0, 0.5], dtype=np.float32)
    c = np.zeros(d // 2, np.float32)
    s = np.ones(d // 2, np.float32)
    r = O.rope_rotate(x, "f32", c, s, "interleaved")
    assert np.array_equal(r, np.array([2.25, 1.5, -0.5, 3.0], np.float32))
    r = O.rope_rotate(x, "f32", c, s, "half")
    assert np.array_equal(r, np.array([-3.0, -0.5, 1.5, -2.25], np.float32))


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_matches_complex_multiplication(style):
    d, P = 128, 300
    c, s = O.rope_table(P, d)
    x = rng.standard_normal((P, d)).astype(np.float32)
    half = d // 2
    if style == "interleaved":
        z = x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2]
    else:
        z = x[:, :half].astype(np.float64) + 1j * x[:, half:]
    i = np.arange(half)
    ang = np.arange(P)[:, None] * 10000.0 ** (-2.0 * i / d)[None, :]
    zr = z * np.exp(1j * ang)
    r = np.stack([O.rope_rotate(x[p], "f32", c[p], s[p], style) for p in range(P)])
    if style == "interleaved":
        re, im = r[:, 0::2], r[:, 1::2]
    else:
        re, im = r[:, :half], r[:, half:]
    # float32 table (|err| <= 2^-24 relative) and two float32 roundings per output
    np.testing.assert_allclose(re, zr.real, rtol=0, atol=4e-6 * np.abs(x).max())
    np.testing.assert_allclose(im, zr.imag, rtol=0, atol=4e-6 * np.abs(x).max())
    # each pair keeps its length
    n0 = np.abs(z)
    n1 = np.hypot(re.astype(np.float64), im)
    np.testing.assert_allclose(n1, n0, rtol=1e-6, atol=1e-6)


def _to_f32_torch(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values as float32 through torch's own conversion."""
    if dtype == "f32":
        return np.asarray(x, np.float32)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_is_the_float32_operation_sequence(style, dtype):
    """The rotation, bit for bit, against the same operation sequence in native
    IEEE single precision (numpy float32 arithmetic: every product and sum
    rounded once, nothing fused), then stored through torch's own conversion.
    A single rounding of the whole expression (a fused multiply-add) differs
    from it in the last bit of most outputs."""
    d, P = 128, 300
    c, s = O.rope_table(P, d)
    x = _rand_store((P, 3, d), dtype)
    xf = _to_f32_torch(x, dtype)
    half = d // 2
    i = np.arange(half)
    i0, i1 = (2 * i, 2 * i + 1) if style == "interleaved" else (i, i + half)
    n_diff_fused = 0
    for p in range(P):
        x0, x1 = xf[p][:, i0], xf[p][:, i1]
        cc, ss = c[p][None, :], s[p][None, :]
        r0 = x0 * cc - x1 * ss                  # float32 * float32 -> float32, then float32 - float32
        r1 = x0 * ss + x1 * cc
        want = np.empty_like(xf[p])
        want[:, i0], want[:, i1] = r0, r1
        got = O.rope_rotate_f32(x[p], dtype, c[p], s[p], style)
        assert got.dtype == np.float64 and np.array_equal(got.astype(np.float32), want)
        assert np.array_equal(got.astype(np.float32).astype(np.float64), got)    # float32 values
        stored = O.rope_rotate(x[p], dtype, c[p], s[p], style)
        ref = want if dtype == "f32" else _bf16_from_torch(want)
        assert np.array_equal(stored, ref)
        fused = (x0.astype(np.float64) * cc - x1.astype(np.float64) * ss).astype(np.float32)
        n_diff_fused += int(np.count_nonzero(fused != r0))
    assert n_diff_fused > 0     # the check can tell the two apart on these inputs


def test_rope_scores_depend_only_on_relative_position():
    d = 64
    c, s = O.rope_table(400, d)
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)

    def score(pq, pk):
        a = O.rope_rotate(q, "f32", c[pq], s[pq]).astype(np.float64)
        b = O.rope_rotate(k, "f32", c[pk], s[pk]).astype(np.float64)
        return a @ b

    base = score(20, 5)
    for shift in (1, 37, 250):
        assert abs(score(20 + shift, 5 + shift) - base) < 1e-4
    assert abs(score(21, 5) - base) > 1e-3   # a different distance does change it


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------


def _same_bits(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_exactly_one_slice(dtype):
    B, H_kv, T, d = 3, 2, 9, 8
    kc = _rand_store((B, H_kv, T, d), dtype)
    vc = _rand_store((B, H_kv, T, d), dtype)
    kn = _rand_store((B, H_kv, d), dtype)
    vn = _rand_store((B, H_kv, d), dtype)
    q = _rand_store((B, 4, d), dtype)
    cached = np.array([0, 4, 8], np.int32)
    c, s = O.rope_table(T, d)
    k2, v2, q2 = O.append_contiguous(kc, vc, cached, kn, vn, c, s, dtype, q=q)
    for b, p in enumerate(cached):
        mask = np.ones(T, bool)
        mask[p] = False
        assert _same_bits(k2[b][:, mask], kc[b][:, mask])
        assert _same_bits(v2[b][:, mask], vc[b][:, mask])
        assert _same_bits(v2[b, :, p], vn[b])
        assert _same_bits(k2[b, :, p], O.rope_rotate(kn[b], dtype, c[p], s[p]))
        assert _same_bits(q2[b], O.rope_rotate(q[b], dtype, c[p], s[p]))
    # position 0 stores the key unrotated
    assert _same_bits(k2[0, :, 0], kn[0])


def test_paged_location_matches_page_example():
    g = json.load(open(os.path.join(GOLDEN, "paged_example.json")))
    bs, n = g["block_size"], g["n_tokens"]
    assert O.paged_blocks(n, bs) == g["n_blocks"]
    assert O.paged_last_block_fill(n, bs) == g["last_block_fill"]
    for lb, (lo, hi) in enumerate(g["token_ranges"]):
        for p in (lo, hi):
            assert O.paged_location(p, bs)[0] == lb
    assert O.paged_location(41, bs) == (2, 9)
    assert O.paged_blocks(n, bs) * bs - n <= g["max_waste_tokens"]
    assert O.paged_last_block_fill(32, bs) == 16


def test_paged_append_lands_in_the_mapped_block():
    g = json.load(open(os.path.join(GOLDEN, "paged_example.json")))
    bs, table = g["block_size"], np.array([g["block_table"]], np.int32)
    H_kv, d = 2, 8
    pool = np.zeros((300, H_kv, bs, d), np.float32)
    kn = np.ones((1, H_kv, d), np.float32)
    vn = np.full((1, H_kv, d), 2.0, np.float32)
    c, s = O.rope_table(48, d)
    k2, v2, _ = O.append_paged(pool, pool, table, bs, np.array([41]), kn, vn, c, s, "f32")
    assert np.all(v2[287, :, 9] == 2.0)
    # only (block 287, slot 9) changed, in every KV head
    assert np.argwhere(np.any(v2 != pool, axis=(1, 3))).tolist() == [[287, 9]]
    assert np.argwhere(np.any(k2 != pool, axis=(1, 3))).tolist() == [[287, 9]]


def _paged_copy(kc, vc, seq_lens, bs, perm_seed=7):
    """Scatter contiguous caches [B, H, T, d] into a randomly ordered block pool."""
    B, H, T, d = kc.shape
    nblk = [-(-T // bs)] * B
    total = sum(nblk)
    perm = np.random.default_rng(perm_seed).permutation(total)
    table = np.full((B, max(nblk)), -1, np.int32)
    kp = np.zeros((total, H, bs, d), kc.dtype)
    vp = np.zeros((total, H, bs, d), vc.dtype)
    off = 0
    for b in range(B):
        for lb in range(nblk[b]):
            phys = perm[off]
            off += 1
            table[b, lb] = phys
            lo, hi = lb * bs, min(T, (lb + 1) * bs)
            kp[phys, :, : hi - lo] = kc[b, :, lo:hi]
            vp[phys, :, : hi - lo] = vc[b, :, lo:hi]
    return kp, vp, table


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_append_equals_contiguous_append(dtype):
    B, H_kv, T, d, bs = 3, 2, 40, 8, 16
    kc = _rand_store((B, H_kv, T, d), dtype)
    vc = _rand_store((B, H_kv, T, d), dtype)
    kn = _rand_store((B, H_kv, d), dtype)
    vn = _rand_store((B, H_kv, d), dtype)
    cached = np.array([0, 17, 39], np.int32)
    c, s = O.rope_table(T, d)
    kp, vp, table = _paged_copy(kc, vc, cached + 1, bs)
    k2, v2, _ = O.append_contiguous(kc, vc, cached, kn, vn, c, s, dtype)
    kp2, vp2, _ = O.append_paged(kp, vp, table, bs, cached, kn, vn, c, s, dtype)
    for b in range(B):
        assert _same_bits(O.gather_paged(kp2, table, bs, b, T)[:, :T], k2[b])
        assert _same_bits(O.gather_paged(vp2, table, bs, b, T)[:, :T], v2[b])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def _brute_force_mha(q, K, V, L):
    """Pure-Python MHA decode: one KV head per query head, math.exp and loops."""
    B, H, d = q.shape
    out = np.zeros((B, H, d))
    for b in range(B):
        for h in range(H):
            sc = [sum(float(q[b, h, i]) * float(K[b, h, t, i]) for i in range(d)) / math.sqrt(d)
                  for t in range(L[b])]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            z = sum(e)
            for i in range(d):
                out[b, h, i] = sum(e[t] * float(V[b, h, t, i]) for t in range(L[b])) / z
    return out


def test_mha_case_equals_brute_force():
    B, H, T, d = 2, 3, 7, 5
    q = _rand_store((B, H, d), "f32")
    K = _rand_store((B, H, T, d), "f32")
    V = _rand_store((B, H, T, d), "f32")
    L = [7, 3]
    got = O.decode_attention(q, K, V, L, "f32")
    np.testing.assert_allclose(got, _brute_force_mha(q, K, V, L), rtol=0, atol=1e-12)


@pytest.mark.parametrize("H_q,H_kv", [(8, 2), (6, 3), (8, 1), (4, 4)])
def test_gqa_equals_mha_on_repeated_kv(H_q, H_kv):
    B, T, d, G = 2, 11, 16, H_q // H_kv
    q = _rand_store((B, H_q, d), "bf16")
    K = _rand_store((B, H_kv, T, d), "bf16")
    V = _rand_store((B, H_kv, T, d), "bf16")
    L = [11, 6]
    gqa = O.decode_attention(q, K, V, L, "bf16")
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)   # repeat_interleave
    mha = O.decode_attention(q, Kr, Vr, L, "bf16")
    assert np.array_equal(gqa, mha)
    if 1 < H_kv < H_q:
        # a wrong (modular) head map would read np.tile'd KV instead
        tiled = O.decode_attention(q, np.tile(K, (1, G, 1, 1)), np.tile(V, (1, G, 1, 1)), L, "bf16")
        assert not np.allclose(gqa, tiled)


def test_mqa_is_gqa_with_one_kv_head_and_heads_stay_distinct():
    B, H_q, T, d = 1, 4, 9, 8
    q = _rand_store((B, H_q, d), "f32")
    K = _rand_store((B, 1, T, d), "f32")
    V = _rand_store((B, 1, T, d), "f32")
    out = O.decode_attention(q, K, V, [T], "f32")
    for h in range(H_q):
        one = O.decode_attention(q[:, h:h + 1], K, V, [T], "f32")
        assert np.array_equal(out[:, h], one[:, 0])
    # different queries on shared K/V give different outputs
    assert not np.allclose(out[0, 0], out[0, 1])
    # swapping two query heads of a group swaps their outputs
    q2 = q.copy()
    q2[:, [0, 1]] = q2[:, [1, 0]]
    out2 = O.decode_attention(q2, K, V, [T], "f32")
    assert np.array_equal(out2[:, [1, 0]], out[:, [0, 1]])


def test_softmax_rows_sum_to_one():
    q = _rand_store((2, 4, 16), "bf16")
    K = _rand_store((2, 2, 50, 16), "bf16")
    ws = O.decode_attention_weights(q, K, [50, 13], "bf16")
    for row in ws:
        for w in row:
            assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)


def test_closed_forms():
    d = 16
    K = _rand_store((1, 1, 20, d), "f32")
    V = _rand_store((1, 1, 20, d), "f32")
    q = _rand_store((1, 2, d), "f32")
    # one token: the output is that token's value
    out = O.decode_attention(q, K, V, [1], "f32")
    assert np.array_equal(out[0, 0], V[0, 0, 0].astype(np.float64))
    # zero query: uniform weights, the output is the mean value
    out = O.decode_attention(np.zeros_like(q), K, V, [20], "f32")
    np.testing.assert_allclose(out[0, 1], V[0, 0].astype(np.float64).mean(0), atol=1e-14)
    # all keys equal: uniform weights again
    Ke = np.repeat(K[:, :, :1], 20, axis=2)
    out = O.decode_attention(q, Ke, V, [20], "f32")
    np.testing.assert_allclose(out[0, 0], V[0, 0].astype(np.float64).mean(0), atol=1e-14)
    # permuting tokens (K and V rows together) leaves the output unchanged
    perm = rng.permutation(20)
    out1 = O.decode_attention(q, K, V, [20], "f32")
    out2 = O.decode_attention(q, K[:, :, perm], V[:, :, perm], [20], "f32")
    np.testing.assert_allclose(out1, out2, atol=1e-13)
    # empty sequence: zeros by definition
    assert np.all(O.decode_attention(q, K, V, [0], "f32") == 0)


@pytest.mark.parametrize("H_q,H_kv,dtype", [(8, 2, "bf16"), (4, 4, "f32"), (32, 1, "bf16")])
def test_matches_torch_sdpa_float64(H_q, H_kv, dtype):
    B, T, d = 2, 37, 32
    q = _rand_store((B, H_q, d), dtype)
    K = _rand_store((B, H_kv, T, d), dtype)
    V = _rand_store((B, H_kv, T, d), dtype)
    L = [37, 20]
    got = O.decode_attention(q, K, V, L, dtype)
    G = H_q // H_kv
    for b in range(B):
        qt = torch.from_numpy(O.to_f64(q[b], dtype))[:, None, :]           # [H, 1, d]
        Kt = torch.from_numpy(O.to_f64(K[b, :, :L[b]], dtype)).repeat_interleave(G, 0)
        Vt = torch.from_numpy(O.to_f64(V[b, :, :L[b]], dtype)).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous())
        np.testing.assert_allclose(got[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_nan_past_length_is_never_read():
    K = _rand_store((1, 2, 10, 8), "bf16")
    V = _rand_store((1, 2, 10, 8), "bf16")
    K[:, :, 6:] = 0x7FC0
    V[:, :, 6:] = 0x7FC0
    out = O.decode_attention(_rand_store((1, 4, 8), "bf16"), K, V, [6], "bf16")
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_attention_equals_contiguous(dtype):
    B, H_q, H_kv, T, d, bs = 3, 8, 2, 50, 16, 16
    q = _rand_store((B, H_q, d), dtype)
    kc = _rand_store((B, H_kv, T, d), dtype)
    vc = _rand_store((B, H_kv, T, d), dtype)
    L = np.array([50, 17, 1])
    kp, vp, table = _paged_copy(kc, vc, L, bs)
    a = O.decode_attention(q, kc, vc, L, dtype)
    p = O.decode_attention_paged(q, kp, vp, table, bs, L, dtype)
    assert np.array_equal(a, p)


# ---------------------------------------------------------------------------
# cached decode == full causal recomputation
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_incremental_decode_equals_full_recompute(dtype, style):
    H_q, H_kv, n, d = 4, 2, 9, 16
    c, s = O.rope_table(n, d)
    q_raw = _rand_store((H_q, n, d), dtype)
    k_raw = _rand_store((H_kv, n, d), dtype)
    v = _rand_store((H_kv, n, d), dtype)
    full = O.causal_attention_full(q_raw, k_raw, v, c, s, dtype, style)
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    kc = np.full((1, H_kv, n, d), nan, dtype=k_raw.dtype)
    vc = np.full((1, H_kv, n, d), nan, dtype=v.dtype)
    for p in range(n):
        kc, vc, qr = O.append_contiguous(kc, vc, np.array([p]), k_raw[None, :, p], v[None, :, p],
                                         c, s, dtype, style, q=q_raw[None, :, p])
        step = O.decode_attention(qr, kc, vc, [p + 1], dtype)
        np.testing.assert_allclose(step[0], full[:, p], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# accounting
# ---------------------------------------------------------------------------


def test_cache_sizes_match_page_numbers():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_sizes.json")))
    for e in g["per_token"]:
        assert O.kv_bytes_per_token(e["n_layers"], e["n_kv_heads"], e["d_head"], e["elem_bytes"]) == e["bytes"], e["cite"]
    for e in g["totals_decimal_gb"]:
        b = O.kv_cache_bytes(e["n_layers"], e["n_kv_heads"], e["d_head"], e["elem_bytes"], e["tokens"], e["batch"])
        assert round(b / 1e9, e["digits"]) == e["gb"], e["cite"]
    for e in g["totals_binary"]:
        b = O.kv_cache_bytes(e["n_layers"], e["n_kv_heads"], e["d_head"], e["elem_bytes"], e["tokens"], e["batch"])
        assert b / 2**20 == e["mib"], e["cite"]
    for e in g["bounds"]:
        b = O.kv_cache_bytes(e["n_layers"], e["n_kv_heads"], e["d_head"], e["elem_bytes"], e["tokens"], e["batch"])
        if "more_than_bytes" in e:
            assert b > e["more_than_bytes"], e["cite"]
        else:
            assert abs(b / e["about_bytes"] - 1) < e["rel_tol"], e["cite"]


def test_per_layer_scalars_and_step_bytes():
    # 2 * T * H_kv * d scalars per layer ("Ukuran KV cache mengikuti jumlah KV head")
    assert O.kv_elements_per_layer(8193, 8, 128) * 2 == O.kv_cache_bytes(1, 8, 128, 2, 8193, 1)
    w = W.WORKLOADS["gqa_8b"]
    lens = [w.cached_lo + 1] * w.B
    assert O.decode_kv_read_bytes(lens, w.H_kv, w.d, 2) == O.kv_cache_bytes(1, w.H_kv, w.d, 2, 8193, w.B)
    assert O.decode_kv_read_bytes(lens, w.H_kv, w.d, 2) == 536_936_448
    # MQA: halving KV heads halves the bytes, query heads do not matter
    assert O.decode_kv_read_bytes([10], 1, 128, 2) * 8 == O.decode_kv_read_bytes([10], 8, 128, 2)
    assert O.decode_flops([10], 32, 128) == 2 * 2 * 10 * 32 * 128
