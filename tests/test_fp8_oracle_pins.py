"""Pins of the FP8-cache oracle (oracle/kvc_fp8_oracle.py) to what fixes it
other than itself.

* The 256 codes of each format decode as torch's own float8 types read them
  (torch.float8_e4m3fn, torch.float8_e5m2: a library implementation of the
  OCP formats), and a few codes as the format definition gives them by hand
  (largest finite value, smallest subnormal, 1.0, infinity, NaN).
* Encoding: equal, code for code, to torch's float32 -> float8 cast (round to
  nearest, ties to even) over random values of every magnitude and over every
  midpoint between neighbouring values (the ties); and to a brute-force
  search over the finite values (plain Python, ties to the even mantissa);
  values past the largest finite one saturate to it.
* Quantizer (E4M3): equal, bit for bit, to the same expressions evaluated with
  torch float32 tensors (amax / 448, x / scale, the float8 cast) over 20000
  vectors; the vector's largest element lands on +-448 exactly; a zero vector
  gets scale 1 and zero codes; every element reads back within half a unit in
  the last place.  E5M2: scale 1 and the direct cast.
* Dequantize: torch's float8 reading times the scale.
* Append: only the new token's slot changes; the stored key is the quantized
  float32 rotation (before any storage rounding), the value the quantized raw
  value; contiguous and paged agree.
* Decode: one attended token gives its dequantized value exactly; attention
  over the dequantized cache equals torch's scaled_dot_product_attention in
  float64 on the same values.

Planted mistakes in a copy of the oracle (a wrong bias, truncation, ties away
from zero, no saturation, the scale over 127, the key pairs for the values, the
key quantized before rotation) each fail a pin.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle.kvc_fp8_oracle as F
import oracle.kvc_oracle as O

SRC = open(F.__file__).read()
TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _values(fmt, n, seed):
    """float32 values of every magnitude inside the format's range, plus every
    midpoint between neighbouring finite values (both signs)."""
    rng = np.random.default_rng(seed)
    vmax = F.FORMATS[fmt][3]
    x = rng.standard_normal(n) * rng.choice([1e-6, 1e-4, 1e-2, 1.0, 30.0, 300.0, 5000.0], n)
    x = np.clip(x, -vmax, vmax).astype(np.float32)
    tab = torch.arange(256, dtype=torch.uint8).view(TORCH[fmt]).double().numpy()
    fin = np.sort(np.unique(tab[np.isfinite(tab)]))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    return np.concatenate([x, mids, -mids, fin.astype(np.float32)]).astype(np.float32)


# --- checks (each returns True when the module passes) ----------------------


def check_table_torch(M) -> bool:
    ok = True
    for fmt in ("e4m3", "e5m2"):
        got = M.fp8_table(fmt)
        ref = torch.arange(256, dtype=torch.uint8).view(TORCH[fmt]).double().numpy()
        ok &= bool(np.array_equal(np.isnan(got), np.isnan(ref)))
        ok &= bool(np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)]))
    return ok


def check_table_by_hand(M) -> bool:
    e4 = {0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0xB8: -1.0, 0x3C: 1.5, 0x00: 0.0}
    e5 = {0x7B: 57344.0, 0x01: 2.0 ** -16, 0x04: 2.0 ** -14, 0x3C: 1.0, 0x3E: 1.5, 0x7C: math.inf, 0xFC: -math.inf}
    ok = all(M.fp8_value(c, "e4m3") == v for c, v in e4.items())
    ok &= all(M.fp8_value(c, "e5m2") == v for c, v in e5.items())
    ok &= math.isnan(M.fp8_value(0x7F, "e4m3")) and math.isnan(M.fp8_value(0xFF, "e4m3"))
    ok &= math.isnan(M.fp8_value(0x7D, "e5m2"))
    return bool(ok)


def check_encode_torch(M) -> bool:
    ok = True
    for fmt in ("e4m3", "e5m2"):
        x = _values(fmt, 40000, 1)
        ref = torch.from_numpy(x).to(TORCH[fmt]).view(torch.uint8).numpy()
        ok &= bool(np.array_equal(M.fp8_encode(x, fmt), ref))
    return ok


def check_encode_brute_force(M) -> bool:
    ok = True
    for fmt in ("e4m3", "e5m2"):
        finite = [(c, F.fp8_value(c, fmt)) for c in range(256) if math.isfinite(F.fp8_value(c, fmt))]
        x = _values(fmt, 600, 2)[::7]
        got = M.fp8_encode(x, fmt)
        for xi, gi in zip(x.tolist(), got.tolist()):
            best = None
            for c, v in finite:
                if (v == 0.0) and (c & 0x80) != (0x80 if math.copysign(1.0, xi) < 0 else 0):
                    continue                       # zero keeps the input's sign
                dist = abs(v - xi)
                key = (dist, c & 1)                # ties: the even mantissa
                if best is None or key < best[0]:
                    best = (key, c)
            ok &= gi == best[1]
        vmax = F.FORMATS[fmt][3]
        sat = M.fp8_encode(np.array([vmax * 1.2, -vmax * 4, vmax], np.float32), fmt)
        ok &= bool(F.fp8_value(int(sat[0]), fmt) == vmax and F.fp8_value(int(sat[1]), fmt) == -vmax)
        ok &= bool(F.fp8_value(int(sat[2]), fmt) == vmax)
    return bool(ok)


def check_quantize_torch(M) -> bool:
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20000, 128)) * rng.choice([1e-3, 1.0, 50.0], (20000, 1))).astype(np.float32)
    codes, sz = M.quantize_fp8(x, "e4m3")
    xt = torch.from_numpy(x)
    scale = xt.abs().amax(dim=-1, keepdim=True) / 448.0
    ref = (xt / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = bool(np.array_equal(codes, ref)) and bool(np.array_equal(sz[:, 0:1], scale.numpy()))
    ok &= bool(np.all(sz[:, 1] == 0.0))
    # the largest element lands on +-448
    i = np.argmax(np.abs(x), axis=-1)
    ok &= bool(np.all(np.abs(F.fp8_table("e4m3")[codes[np.arange(x.shape[0]), i]]) == 448.0))
    # within half a unit in the last place (relative 2^-4 for normals; 2^-10 absolute on the subnormal grid)
    back = F.fp8_table("e4m3")[codes] * sz[:, 0:1].astype(np.float64)
    err = np.abs(back - x.astype(np.float64))
    bound = np.maximum(np.abs(x.astype(np.float64)) * 2.0 ** -4, 2.0 ** -10 * sz[:, 0:1]) * (1 + 1e-6)
    ok &= bool(np.all(err <= bound))
    # vectors whose elements divide exactly onto ties: scale s (no exact
    # reciprocal in float32), the largest element 448 s, the others s times each
    # midpoint between neighbouring E4M3 values
    tab = F.fp8_table("e4m3")
    fin = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
    mids = (fin[1:] + fin[:-1]) / 2
    for s in (3.0, 5.0, 7.0, 0.3):
        sf = np.float32(s)
        row = np.concatenate([[448.0 * sf], (mids * sf).astype(np.float32), -(mids * sf).astype(np.float32)])
        row = row.astype(np.float32)[None, :]
        rt = torch.from_numpy(row)
        sc = rt.abs().amax(dim=-1, keepdim=True) / 448.0
        c_ref = (rt / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ok &= bool(np.array_equal(M.quantize_fp8(row, "e4m3")[0], c_ref))
    z_codes, z_sz = M.quantize_fp8(np.zeros((2, 16), np.float32), "e4m3")
    ok &= bool(np.all(z_codes == 0) and np.all(z_sz[:, 0] == 1.0))
    # E5M2: the direct cast
    c5, s5 = M.quantize_fp8(x[:2000], "e5m2")
    ok &= bool(np.array_equal(c5, xt[:2000].to(torch.float8_e5m2).view(torch.uint8).numpy()))
    ok &= bool(np.all(s5[:, 0] == 1.0) and np.all(s5[:, 1] == 0.0))
    return ok


def check_dequantize(M) -> bool:
    rng = np.random.default_rng(4)
    ok = True
    for fmt in ("e4m3", "e5m2"):
        codes = rng.integers(0, 256, (50, 32), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes (E5M2: also no inf / NaN)
        if fmt == "e5m2":
            codes[(codes & 0x7C) == 0x7C] = 0x11
        sz = np.stack([rng.uniform(0.001, 0.02, 50).astype(np.float32), np.zeros(50, np.float32)], -1)
        ref = torch.from_numpy(codes).view(TORCH[fmt]).double().numpy() * sz[:, 0:1].astype(np.float64)
        ok &= bool(np.array_equal(M.dequantize_fp8(codes, sz, fmt), ref))
    return ok


def _append_case(M, fmt, paged):
    rng = np.random.default_rng(5)
    B, H_q, H_kv, d, T = 3, 4, 2, 16, 12
    cos, sin = O.rope_table(T, d)
    kc = rng.integers(0, 120, (B, H_kv, T, d), dtype=np.uint8)
    vc = rng.integers(0, 120, (B, H_kv, T, d), dtype=np.uint8)
    ks = np.abs(rng.standard_normal((B, H_kv, T, 2))).astype(np.float32)
    vs = np.abs(rng.standard_normal((B, H_kv, T, 2))).astype(np.float32)
    kn = O.round_store(rng.standard_normal((B, H_kv, d)).astype(np.float32), "bf16")
    vn = O.round_store(rng.standard_normal((B, H_kv, d)).astype(np.float32), "bf16")
    q = O.round_store(rng.standard_normal((B, H_q, d)).astype(np.float32), "bf16")
    cached = np.array([0, 5, 11])
    if not paged:
        return M.append_contiguous_fp8(kc, ks, vc, vs, cached, kn, vn, cos, sin, "bf16", fmt, q=q), \
            (kc, ks, vc, vs, cached, kn, vn, cos, sin, q)
    bs = 4
    tbl = np.array([[2, 0, 7], [5, 1, 3], [4, 6, 8]], np.int32)
    nblk = 9
    pk = rng.integers(0, 120, (nblk, H_kv, bs, d), dtype=np.uint8)
    pv = rng.integers(0, 120, (nblk, H_kv, bs, d), dtype=np.uint8)
    pks = np.abs(rng.standard_normal((nblk, H_kv, bs, 2))).astype(np.float32)
    pvs = np.abs(rng.standard_normal((nblk, H_kv, bs, 2))).astype(np.float32)
    return M.append_paged_fp8(pk, pks, pv, pvs, tbl, bs, cached, kn, vn, cos, sin, "bf16", fmt, q=q), \
        (pk, pks, pv, pvs, cached, kn, vn, cos, sin, q, tbl, bs)


def check_append(M) -> bool:
    ok = True
    for fmt in ("e4m3", "e5m2"):
        (kc2, ks2, vc2, vs2, q2), (kc, ks, vc, vs, cached, kn, vn, cos, sin, q) = _append_case(M, fmt, False)
        for b, p in enumerate(cached.tolist()):
            kr = O.rope_rotate_f32(kn[b], "bf16", cos[p], sin[p]).astype(np.float32)
            # the stored key reads back within the format's half unit of the float32 rotation
            back = F.dequantize_fp8(kc2[b, :, p], ks2[b, :, p], fmt)
            rel = 2.0 ** -4 if fmt == "e4m3" else 2.0 ** -3
            ok &= bool(np.all(np.abs(back - kr) <= np.abs(kr) * rel + 1e-6))
            vback = F.dequantize_fp8(vc2[b, :, p], vs2[b, :, p], fmt)
            vf = O.to_f32(vn[b], "bf16").astype(np.float64)
            ok &= bool(np.all(np.abs(vback - vf) <= np.abs(vf) * rel + 1e-6))
            # the key's largest rotated element (E4M3) lands on 448 * scale exactly
            if fmt == "e4m3":
                j = np.argmax(np.abs(kr), axis=-1)
                ok &= bool(np.all(np.abs(F.fp8_table(fmt)[kc2[b, np.arange(2), p, j]]) == 448.0))
            # the query is rotated as in the unquantized oracle
            ok &= bool(np.array_equal(q2[b], O.rope_rotate(q[b], "bf16", cos[p], sin[p])))
        # nothing else changed
        mask = np.ones(kc.shape[:3], bool)
        for b, p in enumerate(cached.tolist()):
            mask[b, :, p] = False
        ok &= bool(np.array_equal(kc2[mask], kc[mask]) and np.array_equal(vc2[mask], vc[mask]))
        ok &= bool(np.array_equal(ks2[mask], ks[mask]) and np.array_equal(vs2[mask], vs[mask]))
        # the paged append writes the same codes and pairs into the table's slot
        (pk2, pks2, pv2, pvs2, _), (pk, pks, pv, pvs, cached, *_rest, tbl, bs) = _append_case(M, fmt, True)
        for b, p in enumerate(cached.tolist()):
            blk, off = int(tbl[b][p // bs]), p % bs
            ok &= bool(np.array_equal(pk2[blk, :, off], kc2[b, :, p]) and np.array_equal(pv2[blk, :, off], vc2[b, :, p]))
            ok &= bool(np.array_equal(pks2[blk, :, off], ks2[b, :, p]) and np.array_equal(pvs2[blk, :, off], vs2[b, :, p]))
    return ok


def check_decode(M) -> bool:
    rng = np.random.default_rng(6)
    ok = True
    for fmt in ("e4m3", "e5m2"):
        B, H_q, H_kv, d, T = 2, 8, 2, 16, 20
        x = rng.standard_normal((B, H_kv, T, d)).astype(np.float32)
        kc, ks = M.quantize_fp8(x, fmt)
        vc, vs = M.quantize_fp8(rng.standard_normal((B, H_kv, T, d)).astype(np.float32), fmt)
        q = O.round_store(rng.standard_normal((B, H_q, d)).astype(np.float32), "bf16")
        lens = [20, 1]
        out = M.decode_attention_fp8(q, kc, ks, vc, vs, lens, "bf16", fmt)
        G = H_q // H_kv
        # one token: its dequantized value, exactly
        v0 = torch.from_numpy(vc[1, :, 0]).view(TORCH[fmt]).double().numpy() * vs[1, :, 0, 0:1].astype(np.float64)
        ok &= bool(np.array_equal(out[1], np.repeat(v0, G, axis=0)))
        # the plain definition in torch on the same dequantized values
        K = torch.from_numpy(kc[0]).view(TORCH[fmt]).double() * torch.from_numpy(ks[0, ..., 0:1]).double()
        V = torch.from_numpy(vc[0]).view(TORCH[fmt]).double() * torch.from_numpy(vs[0, ..., 0:1]).double()
        qt = torch.from_numpy(O.to_f64(q[0], "bf16"))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, K.repeat_interleave(G, 0).contiguous(), V.repeat_interleave(G, 0).contiguous())[:, 0].numpy()
        ok &= bool(np.allclose(out[0], ref, rtol=0, atol=1e-12))
        # paged equals contiguous on the same data
        bs = 4
        nb = B * T // bs
        perm = rng.permutation(nb)
        tbl = perm.reshape(B, T // bs).astype(np.int32)
        pk = np.zeros((nb, H_kv, bs, d), np.uint8)
        pv = np.zeros_like(pk)
        pks = np.zeros((nb, H_kv, bs, 2), np.float32)
        pvs = np.zeros_like(pks)
        for b in range(B):
            for t in range(T):
                blk = tbl[b, t // bs]
                pk[blk, :, t % bs], pv[blk, :, t % bs] = kc[b, :, t], vc[b, :, t]
                pks[blk, :, t % bs], pvs[blk, :, t % bs] = ks[b, :, t], vs[b, :, t]
        outp = M.decode_attention_paged_fp8(q, pk, pks, pv, pvs, tbl, bs, lens, "bf16", fmt)
        ok &= bool(np.array_equal(outp, out))
    return ok


CHECKS = [check_table_torch, check_table_by_hand, check_encode_torch, check_encode_brute_force,
          check_quantize_torch, check_dequantize, check_append, check_decode]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_pin(chk):
    assert chk(F)


MUTATIONS = {
    "e4m3 bias 8": ('"e4m3": (4, 3, 7, 448.0, False)', '"e4m3": (4, 3, 8, 448.0, False)'),
    "truncation": ("if r > 0.5 or (r == 0.5 and n % 2 == 1):", "if False:"),
    "ties away from zero": ("if r > 0.5 or (r == 0.5 and n % 2 == 1):", "if r >= 0.5:"),
    "no saturation": ("            if value > vmax:\n                value = vmax", "            if False:\n                value = vmax"),
    "scale over 127": ("scale = (amax / np.float32(FORMATS[fmt][3])).astype(np.float32)",
                       "scale = (amax / np.float32(127.0)).astype(np.float32)"),
    "scale by reciprocal": ("codes = fp8_encode((v / scale).astype(np.float32), fmt)",
                            "codes = fp8_encode((v * (np.float32(1.0) / scale)).astype(np.float32), fmt)"),
    "values read with the key pairs": ("v[b, :, :L] = dequantize_fp8(v_codes[b, :, :L], v_sz[b, :, :L], fmt)",
                                       "v[b, :, :L] = dequantize_fp8(v_codes[b, :, :L], k_sz[b, :, :L], fmt)"),
    "key quantized before rotation": ("kr = O.rope_rotate_f32(k_new, dtype, cos[p], sin[p], style).astype(np.float32)",
                                      "kr = O.to_f32(k_new, dtype)"),
    "subnormal exponent": ("    emin = 1 - bias", "    emin = -bias"),
    "e5m2 mantissa bits": ('"e5m2": (5, 2, 15, 57344.0, True)', '"e5m2": (5, 3, 15, 57344.0, True)'),
}


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("fp8_oracle_mutant")
    src = src.replace("from . import kvc_oracle as O", "import oracle.kvc_oracle as O")
    src = src.replace("from . import kvc_quant_oracle as Q", "import oracle.kvc_quant_oracle as Q")
    exec(compile(src, "fp8_oracle_mutant", "exec"), m.__dict__)
    return m


def _passes(chk, M) -> bool:
    try:
        return bool(chk(M))
    except Exception:
        return False


def test_checks_pass_on_an_unedited_copy():
    M = _load(SRC)
    assert all(_passes(c, M) for c in CHECKS)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found once: {old}"
    M = _load(SRC.replace(old, new))
    assert not all(_passes(c, M) for c in CHECKS), f"no pin catches: {name}"
