"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case edits one line of the oracle's source, loads the edited copy as a new
module, and runs the pin checks against it: at least one check must fail.  The
same checks must all pass on the unedited oracle.  This shows that a dropped
term, a wrong sign or index, or a swapped operand cannot hide behind the pins.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.kvc_oracle as ORIG

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = open(ORIG.__file__).read()


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), m.__dict__)
    return m


def _rs(M, rng, shape, dtype):
    return M.round_store(rng.standard_normal(shape).astype(np.float32), dtype)


# --- checks (each returns True when the module passes) ----------------------


def check_sdpa(M) -> bool:
    rng = np.random.default_rng(5)
    ok = True
    for H_q, H_kv in ((8, 2), (4, 4), (6, 1)):
        B, T, d = 2, 19, 16
        q, K, V = _rs(M, rng, (B, H_q, d), "bf16"), _rs(M, rng, (B, H_kv, T, d), "bf16"), _rs(M, rng, (B, H_kv, T, d), "bf16")
        L = [19, 7]
        got = M.decode_attention(q, K, V, L, "bf16")
        G = H_q // H_kv
        for b in range(B):
            qt = torch.from_numpy(ORIG.to_f64(q[b], "bf16"))[:, None, :]
            Kt = torch.from_numpy(ORIG.to_f64(K[b, :, :L[b]], "bf16")).repeat_interleave(G, 0).contiguous()
            Vt = torch.from_numpy(ORIG.to_f64(V[b, :, :L[b]], "bf16")).repeat_interleave(G, 0).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, 0].numpy()
            ok &= bool(np.allclose(got[b], ref, rtol=0, atol=1e-12))
    return ok


def check_rope_complex(M) -> bool:
    d, P = 32, 50
    c, s = M.rope_table(P, d)
    x = np.random.default_rng(6).standard_normal((P, d)).astype(np.float32)
    i = np.arange(d // 2)
    ang = np.arange(P)[:, None] * 10000.0 ** (-2.0 * i / d)[None, :]
    ok = True
    for style in ("interleaved", "half"):
        if style == "interleaved":
            z = x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2]
        else:
            z = x[:, : d // 2].astype(np.float64) + 1j * x[:, d // 2:]
        zr = z * np.exp(1j * ang)
        r = np.stack([M.rope_rotate(x[p], "f32", c[p], s[p], style) for p in range(P)])
        re, im = (r[:, 0::2], r[:, 1::2]) if style == "interleaved" else (r[:, : d // 2], r[:, d // 2:])
        ok &= bool(np.allclose(re, zr.real, atol=3e-5) and np.allclose(im, zr.imag, atol=3e-5))
    return ok


def check_incremental(M) -> bool:
    rng = np.random.default_rng(7)
    H_q, H_kv, n, d = 4, 2, 7, 8
    c, s = M.rope_table(n, d)
    q_raw, k_raw, v = _rs(M, rng, (H_q, n, d), "f32"), _rs(M, rng, (H_kv, n, d), "f32"), _rs(M, rng, (H_kv, n, d), "f32")
    full = M.causal_attention_full(q_raw, k_raw, v, c, s, "f32")
    kc = np.full((1, H_kv, n, d), np.nan, np.float32)
    vc = np.full((1, H_kv, n, d), np.nan, np.float32)
    ok = True
    for p in range(n):
        kc, vc, qr = M.append_contiguous(kc, vc, np.array([p]), k_raw[None, :, p], v[None, :, p], c, s, "f32", q=q_raw[None, :, p])
        step = M.decode_attention(qr, kc, vc, [p + 1], "f32")
        ok &= bool(np.allclose(step[0], full[:, p], atol=1e-12))
    return ok


def check_sizes(M) -> bool:
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_sizes.json")))
    return all(M.kv_bytes_per_token(e["n_layers"], e["n_kv_heads"], e["d_head"], e["elem_bytes"]) == e["bytes"]
               for e in g["per_token"])


def check_paged(M) -> bool:
    g = json.load(open(os.path.join(GOLDEN, "paged_example.json")))
    bs = g["block_size"]
    return (M.paged_blocks(g["n_tokens"], bs) == g["n_blocks"]
            and M.paged_last_block_fill(g["n_tokens"], bs) == g["last_block_fill"]
            and M.paged_location(41, bs) == (2, 9) and M.paged_location(16, bs) == (1, 0))


def check_bf16(M) -> bool:
    rng = np.random.default_rng(8)
    hi = rng.integers(0x0080, 0x7F00, 2000).astype(np.uint32)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32), ((hi << 16) | 0x8000).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bool(np.array_equal(M.bf16_round_bits(x), ref))


def check_table(M) -> bool:
    c, s = M.rope_table(8, 16)
    th = 10000.0 ** (-14 / 16)
    return bool(c[3, 0] == np.float32(math.cos(3)) and c[3, 7] == np.float32(math.cos(3 * th))
                and s[5, 7] == np.float32(math.sin(5 * th)))


def check_rope_f32(M) -> bool:
    """The rotation against native float32 arithmetic (numpy: every operation
    rounded once, nothing fused), bit for bit."""
    d, P = 64, 40
    c, s = M.rope_table(P, d)
    x = np.random.default_rng(9).standard_normal((P, 4, d)).astype(np.float32)
    ok = True
    for style in ("interleaved", "half"):
        i = np.arange(d // 2)
        i0, i1 = (2 * i, 2 * i + 1) if style == "interleaved" else (i, i + d // 2)
        for p in range(P):
            x0, x1 = x[p][:, i0], x[p][:, i1]
            want = np.empty_like(x[p])
            want[:, i0] = x0 * c[p] - x1 * s[p]
            want[:, i1] = x0 * s[p] + x1 * c[p]
            ok &= bool(np.array_equal(M.rope_rotate(x[p], "f32", c[p], s[p], style), want))
    return ok


def check_bf16_exact(M) -> bool:
    """One rounding from float64 to bfloat16 against exact rational rounding,
    on midpoints and values a hair beside them."""
    from test_oracle_pins import bf16_exact_inputs, bf16_rne_exact
    x = bf16_exact_inputs(np.random.default_rng(10), 300)
    want = np.array([bf16_rne_exact(float(v)) for v in x], dtype=np.uint16)
    return bool(np.array_equal(M.bf16_round_bits(x), want))


def _passes(chk, M) -> bool:
    """A check that raises (e.g. an index out of range) counts as failed."""
    try:
        return bool(chk(M))
    except Exception:
        return False


CHECKS = [check_sdpa, check_rope_complex, check_incremental, check_sizes, check_paged, check_bf16, check_table,
          check_rope_f32, check_bf16_exact]

MUTATIONS = {
    "modular_head_map": ("for h in range(j * G, (j + 1) * G):\n                out[b, h], _ = _head_attention(qf[b, h], K, V, sc)\n    return out\n\n\ndef decode_attention_weights",
                         "for h in range(j, H_q, H_kv):\n                out[b, h], _ = _head_attention(qf[b, h], K, V, sc)\n    return out\n\n\ndef decode_attention_weights"),
    "scale_dropped": ("s = (K @ qv) * scale", "s = (K @ qv)"),
    "normalisation_dropped": ("return (w @ V) / z, w / z", "return (w @ V), w / z"),
    "rope_sign": ("r0 = _fl(_fl(x0 * c) - _fl(x1 * s))", "r0 = _fl(_fl(x0 * c) + _fl(x1 * s))"),
    "rope_pairing": ("return 2 * i, 2 * i + 1", "return i, i + half"),
    "rope_swapped_table": ("r1 = _fl(_fl(x0 * s) + _fl(x1 * c))", "r1 = _fl(_fl(x0 * c) + _fl(x1 * s))"),
    "length_off_by_one": ("K = to_f64(k_cache[b, j, :L], dtype)\n            V = to_f64(v_cache[b, j, :L], dtype)",
                          "K = to_f64(k_cache[b, j, :L - 1], dtype)\n            V = to_f64(v_cache[b, j, :L - 1], dtype)"),
    "append_slot_shift": ("k2[b, :, p, :] = rope_rotate(k_new[b], dtype, cos[p], sin[p], style)",
                          "k2[b, :, p, :] = rope_rotate(k_new[b], dtype, cos[p + 1], sin[p + 1], style)"),
    "causal_mask_inverted": ("mask = np.triu(np.ones((n, n), dtype=bool), k=1)", "mask = np.tril(np.ones((n, n), dtype=bool), k=-1)"),
    "kv_factor_two_dropped": ("return 2 * n_layers * n_kv_heads * d_head * elem_bytes", "return n_layers * n_kv_heads * d_head * elem_bytes"),
    "paged_offset": ("return pos // block_size, pos % block_size", "return pos // block_size, (pos + 1) % block_size"),
    "bf16_ties_to_odd": ("even = (cand & 1) == 0", "even = (cand & 1) == 1"),
    # the rotation with one rounding per output (what a fused multiply-add gives)
    "rope_single_rounding": ("r0 = _fl(_fl(x0 * c) - _fl(x1 * s))\n    r1 = _fl(_fl(x0 * s) + _fl(x1 * c))",
                             "r0 = _fl(x0 * c - x1 * s)\n    r1 = _fl(x0 * s + x1 * c)"),
    # float64 rounded to float32 first, then to bfloat16 (two roundings)
    "bf16_double_rounding": ("        _nearest_bf16(flat, mag, sign, best, best_d)",
                             "        _nearest_bf16(f32.astype(np.float64), mag, sign, best, best_d)"),
    "rope_frequency": ("theta = base ** (-(2.0 * i) / d)", "theta = base ** (-(1.0 * i) / d)"),
}


def test_checks_pass_on_the_oracle():
    M = _load(SRC)
    for chk in CHECKS:
        assert chk(M), chk.__name__


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique/present"
    M = _load(SRC.replace(old, new))
    failed = [chk.__name__ for chk in CHECKS if not _passes(chk, M)]
    assert failed, f"planted mistake {name} passed every pin"
