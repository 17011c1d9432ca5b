"""Pins of the quantized-cache oracle (oracle/kvc_quant_oracle.py), on the CPU.

The quantizer follows the QuantizedKVCache listing of "KV Cache 최적화 심층
분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략" (youngju.dev).  The pins
check it against what the listing's arithmetic fixes independently of its own
code: vectors on an exact grid come back exactly, any vector comes back within
half a step, the extremes take the end codes, a worked example of the zero
point clamp, and decoding over a grid cache equals the unquantized oracle's
decoding of the same values.  Planted mistakes in a copy of the module must
each fail one of them.
"""
import json
import os
import types

import numpy as np
import pytest
import torch

import oracle.kvc_oracle as O
import oracle.kvc_quant_oracle as QO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = open(QO.__file__).read()


def _grid(rng, rows, d, k=7):
    """Vectors (c - z) * 2^-k with codes c covering 0 and 255 and a zero point z."""
    s = np.float32(2.0 ** -k)
    c = rng.integers(0, 256, size=(rows, d))
    c[:, 0], c[:, 1] = 0, 255
    z = rng.integers(0, 256, size=(rows, 1))
    x = ((c - z).astype(np.float32) * s).astype(np.float32)
    return x, c.astype(np.uint8), np.float32(s), z[:, 0].astype(np.float32)


# --- checks (True when the module passes) ------------------------------------


def check_grid_exact(M) -> bool:
    rng = np.random.default_rng(11)
    ok = True
    for k in (3, 7, 12):
        x, c, s, z = _grid(rng, 9, 64, k)
        codes, sz = M.quantize_u8(x)
        ok &= bool(np.array_equal(codes, c) and np.all(sz[:, 0] == s) and np.array_equal(sz[:, 1], z))
        ok &= bool(np.array_equal(M.dequantize_u8(codes, sz), x))
    return ok


def check_half_step(M) -> bool:
    rng = np.random.default_rng(12)
    ok = True
    for d in (16, 128, 256):
        x = rng.standard_normal((200, d)).astype(np.float32)
        codes, sz = M.quantize_u8(x)
        err = np.abs(M.dequantize_u8(codes, sz).astype(np.float64) - x)
        ok &= bool(np.all(err <= 0.5 * sz[:, :1] * (1 + 2 ** -20) + 1e-7 * np.abs(x)))
        ok &= bool(np.all(codes[np.arange(200), x.argmin(-1)] == 0))
        ok &= bool(np.all(codes[np.arange(200), x.argmax(-1)] >= 254))
        order = np.argsort(x, axis=-1)
        ok &= bool(np.all(np.diff(np.take_along_axis(codes.astype(int), order, -1), axis=-1) >= 0))
    return ok


def check_clamp_example(M) -> bool:
    """Worked by hand from the listing: x = [1, 2] gives step 1/255, -min/step =
    -255 clamped to zero point 0, and x/step = [255, 510] clipped to [255, 255]."""
    codes, sz = M.quantize_u8(np.array([[1.0, 2.0]], np.float32))
    return bool(np.array_equal(codes, [[255, 255]]) and sz[0, 1] == 0 and sz[0, 0] == np.float32(1.0) / np.float32(255.0))


def check_decode_grid(M) -> bool:
    """Over a cache whose values lie on the grid, the quantized decode equals the
    unquantized oracle's decode of the same float32 values."""
    rng = np.random.default_rng(13)
    B, H_q, H_kv, T, d = 2, 6, 2, 21, 32
    kx, _, _, _ = _grid(rng, B * H_kv * T, d, 6)
    vx, _, _, _ = _grid(rng, B * H_kv * T, d, 5)
    kx, vx = kx.reshape(B, H_kv, T, d), vx.reshape(B, H_kv, T, d)
    kc, ks = M.quantize_u8(kx)
    vc, vs = M.quantize_u8(vx)
    q = rng.standard_normal((B, H_q, d)).astype(np.float32)
    L = [21, 8]
    got = M.decode_attention_u8(q, kc, ks, vc, vs, L, "f32")
    ref = O.decode_attention(q, kx, vx, L, "f32")
    return bool(np.allclose(got, ref, rtol=0, atol=1e-12))


def check_append_half_step(M) -> bool:
    """The appended key and value read back within half a step of the rotated
    key and raw value written by the unquantized oracle (plus its bf16
    rounding); nothing else in the cache changes."""
    rng = np.random.default_rng(14)
    B, H_q, H_kv, T, d = 3, 4, 2, 10, 16
    c, s = O.rope_table(T, d)
    cached = np.array([4, 0, 9])
    kn = O.round_store(rng.standard_normal((B, H_kv, d)).astype(np.float32), "bf16")
    vn = O.round_store(rng.standard_normal((B, H_kv, d)).astype(np.float32), "bf16")
    kc = rng.integers(0, 256, (B, H_kv, T, d)).astype(np.uint8)
    ks = rng.random((B, H_kv, T, 2)).astype(np.float32)
    vc, vs = kc.copy(), ks.copy()
    kc2, ks2, vc2, vs2, _ = M.append_contiguous_u8(kc, ks, vc, vs, cached, kn, vn, c, s, "bf16")
    kb, vb, _ = O.append_contiguous(np.zeros((B, H_kv, T, d), np.uint16), np.zeros((B, H_kv, T, d), np.uint16),
                                    cached, kn, vn, c, s, "bf16")
    ok = True
    for b, p in enumerate(cached):
        for new, sz, ref, bf_slack in ((kc2, ks2, kb, 2 ** -8), (vc2, vs2, vb, 0.0)):
            r = O.to_f64(ref[b, :, p], "bf16")
            got = M.dequantize_u8(new[b, :, p], sz[b, :, p]).astype(np.float64)
            ok &= bool(np.all(np.abs(got - r) <= 0.5 * sz[b, :, p, :1] * (1 + 1e-6) + bf_slack * np.abs(r) + 1e-7))
        mask = np.ones(T, bool)
        mask[p] = False
        for new, old in ((kc2, kc), (ks2, ks), (vc2, vc), (vs2, vs)):
            ok &= bool(np.array_equal(new[b][:, mask], old[b][:, mask]))
    return ok


def check_paged(M) -> bool:
    rng = np.random.default_rng(15)
    B, H_q, H_kv, bs, d = 2, 4, 2, 4, 16
    L = [10, 5]
    T = 12
    kx = rng.standard_normal((B, H_kv, T, d)).astype(np.float32)
    vx = rng.standard_normal((B, H_kv, T, d)).astype(np.float32)
    kc, ks = M.quantize_u8(kx)
    vc, vs = M.quantize_u8(vx)
    nb = T // bs
    perm = rng.permutation(B * nb)
    table = perm.reshape(B, nb)
    pk, pv = np.zeros((B * nb, H_kv, bs, d), np.uint8), np.zeros((B * nb, H_kv, bs, d), np.uint8)
    pks, pvs = np.zeros((B * nb, H_kv, bs, 2), np.float32), np.zeros((B * nb, H_kv, bs, 2), np.float32)
    for b in range(B):
        for lb in range(nb):
            sl = slice(lb * bs, (lb + 1) * bs)
            pk[table[b, lb]], pv[table[b, lb]] = kc[b, :, sl], vc[b, :, sl]
            pks[table[b, lb]], pvs[table[b, lb]] = ks[b, :, sl], vs[b, :, sl]
    q = rng.standard_normal((B, H_q, d)).astype(np.float32)
    a = M.decode_attention_u8(q, kc, ks, vc, vs, L, "f32")
    p = M.decode_attention_paged_u8(q, pk, pks, pv, pvs, table, bs, L, "f32")
    return bool(np.array_equal(a, p))


def _torch_affine_u8(x: np.ndarray):
    """The affine 8-bit grid of each vector evaluated with torch float32 CPU
    tensors (IEEE single precision, every operation rounded once; torch.round
    takes ties to even): step = span / 255, zero code = -min / step rounded and
    clamped to [0, 255], codes = x / step + zero code rounded and clamped."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    lo, hi = torch.aminmax(t, dim=-1, keepdim=True)
    step = torch.div(hi - lo, 255.0)
    step = torch.where(step == 0, torch.ones_like(step), step)
    zero = torch.clamp(torch.round(torch.div(-lo, step)), 0.0, 255.0)
    codes = torch.clamp(torch.round(torch.div(t, step) + zero), 0.0, 255.0).to(torch.uint8)
    return codes.numpy(), step[..., 0].numpy(), zero[..., 0].numpy()


def _tie_vectors() -> np.ndarray:
    """Vectors whose codes (and zero points) fall exactly halfway between two
    codes: step 1 with values k + 1/2, and zero points of exactly 127.5."""
    k = np.arange(0, 255, dtype=np.float32)
    a = np.concatenate([[0.0, 255.0], k[:62] + 0.5]).astype(np.float32)          # step 1, zero 0
    b = np.concatenate([[-127.5, 127.5], k[:62] - 127.0]).astype(np.float32)     # step 1, zero rint(127.5)
    c = np.concatenate([[-1.5, 253.5], k[:62] * 3 + 0.5]).astype(np.float32)     # step 1, zero rint(1.5)
    return np.stack([a, b, c])


def check_float32_torch(M) -> bool:
    """Bit-exact agreement with the grid evaluated in torch float32 (the precision
    the page's float tensors carry) on 65536 N(0, 1) vectors of 128 and on
    vectors built to land on rounding ties."""
    rng = np.random.default_rng(16)
    ok = True
    for x in (rng.standard_normal((1 << 16, 128)).astype(np.float32),
              (rng.standard_normal((512, 64)) * 1e3 + 7).astype(np.float32), _tie_vectors()):
        codes, sz = M.quantize_u8(x)
        tc, ts, tz = _torch_affine_u8(x)
        ok &= bool(np.array_equal(codes, tc) and np.array_equal(sz[..., 0], ts) and np.array_equal(sz[..., 1], tz))
    return ok


CHECKS = [check_grid_exact, check_half_step, check_clamp_example, check_decode_grid, check_append_half_step,
          check_paged, check_float32_torch]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_pin_holds(chk):
    assert chk(QO)


def test_constant_vector_reading():
    """The listing divides by a zero step for a constant vector; the reading
    takes the step as 1 there, which reads such a vector back within 1/2."""
    for v in (0.0, -3.25, 7.0, 200.4):
        x = np.full((1, 32), v, np.float32)
        codes, sz = QO.quantize_u8(x)
        assert sz[0, 0] == 1.0
        assert np.all(np.abs(QO.dequantize_u8(codes, sz) - x) <= 0.5)


def test_code_bytes_per_token_match_the_page():
    """One byte per cached element: the code arrays of an 80-layer, 8-KV-head,
    d=128 cache hold the FP8/INT8 per-token figure printed in section 2 of
    "Arsitektur Inferensi LLM" (tveniu.com); the (step, zero point) pairs add 16
    bytes per token and KV head on top."""
    case = [c for c in json.load(open(os.path.join(GOLDEN, "kv_cache_sizes.json")))["per_token"]
            if c["elem_bytes"] == 1][0]
    H_kv, d = case["n_kv_heads"], case["d_head"]
    codes, sz = QO.quantize_u8(np.random.default_rng(0).standard_normal((H_kv, 1, d)).astype(np.float32))
    per_layer = 2 * codes.nbytes          # K and V codes of one token
    assert per_layer * case["n_layers"] == case["bytes"]
    assert 2 * sz.nbytes == 16 * H_kv
    assert QO.decode_kv_read_bytes_u8([1], H_kv, d) == per_layer + 2 * sz.nbytes


# --- planted mistakes -------------------------------------------------------

MUTATIONS = {
    "step over 256": ("_STEPS = np.float32(255.0)", "_STEPS = np.float32(256.0)"),
    "zero point truncated": ("np.rint(np.negative(lo) / step)", "np.floor(np.negative(lo) / step)"),
    "codes truncated": ("np.rint(x / step + zero)", "np.floor(x / step + zero)"),
    "zero point not clamped": ("np.clip(np.rint(np.negative(lo) / step), 0, _TOP_CODE)", "np.rint(np.negative(lo) / step)"),
    "range over the whole tensor": ("np.min(v, axis=-1, keepdims=True), np.max(v, axis=-1, keepdims=True)",
                                    "np.full(v.shape[:-1] + (1,), v.min(), np.float32), np.max(v, axis=-1, keepdims=True)"),
    # the same steps evaluated in float64 (rounded to float32 only when stored)
    "quantizer in float64": ("v = np.asarray(x, dtype=np.float32)", "v = np.asarray(x, dtype=np.float64)"),
    # the division by the step replaced by a product with its reciprocal
    "codes via reciprocal": ("np.rint(x / step + zero)", "np.rint(x * (np.float32(1.0) / step) + zero)"),
    "dequantize without zero point": ("(np.asarray(codes).astype(np.float32) - zp) * step",
                                      "np.asarray(codes).astype(np.float32) * step"),
    "values read with the key pairs": ("v[b, :, :L] = dequantize_u8(v_codes[b, :, :L], v_sz[b, :, :L])",
                                       "v[b, :, :L] = dequantize_u8(v_codes[b, :, :L], k_sz[b, :, :L])"),
    "key quantized before rotation": ("kr = O.rope_rotate_f32(k_new, dtype, cos[p], sin[p], style).astype(np.float32)",
                                      "kr = O.to_f32(k_new, dtype)"),
    "paged pairs of the wrong cache": ("ks[b, :, :L] = O.gather_paged(k_sz, block_table, block_size, b, L)",
                                       "ks[b, :, :L] = O.gather_paged(v_sz, block_table, block_size, b, L)"),
}


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("quant_oracle_mutant")
    src = src.replace("from . import kvc_oracle as O", "import oracle.kvc_oracle as O")
    exec(compile(src, "quant_oracle_mutant", "exec"), m.__dict__)
    return m


def _passes(chk, M) -> bool:
    try:
        return bool(chk(M))
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found once: {old}"
    M = _load(SRC.replace(old, new))
    assert not all(_passes(c, M) for c in CHECKS), f"no pin catches: {name}"


def test_checks_pass_on_an_unedited_copy():
    M = _load(SRC)
    assert all(_passes(c, M) for c in CHECKS)
