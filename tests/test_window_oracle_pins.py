"""Pins of the sliding-window oracle (oracle/kvc_window_oracle.py), on the CPU.

The window follows the SlidingWindowAttention listing of "KV Cache 최적화 심층
분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략" (youngju.dev).  The pins
hold the oracle to things other than itself:

* the listing's own procedure, replayed token by token with a list cache that
  is concatenated and cut to its last W tokens, and an explicit softmax loop in
  plain Python floats;
* full recomputation of a whole sequence with a band mask (key t visible to
  query p iff p - W < t <= p) through torch's scaled_dot_product_attention in
  float64;
* closed forms: W >= L is the unwindowed decode, W = 1 returns the new value;
* the ring holds exactly the last T tokens, each in slot t mod T;
* paged == contiguous.

Planted mistakes in a copy of the module must each fail one of them.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle.kvc_oracle as O
import oracle.kvc_window_oracle as WO

SRC = open(WO.__file__).read()


def _seq(rng, n, H_q, H_kv, d, dtype="f32"):
    """Raw q, k, v of one sequence at positions 0..n-1: [n, H, d] in storage dtype."""
    mk = lambda *s: O.round_store(rng.standard_normal(s).astype(np.float32), dtype)
    return mk(n, H_q, d), mk(n, H_kv, d), mk(n, H_kv, d)


def _listing_replay(q_raw, k_raw, v_raw, W, cos, sin, dtype):
    """The listing's procedure for one sequence, one token per step: rotate the
    new query and key at their position, append key and value to a list cache,
    keep its last W entries, attend.  Returns [n, H_q, d] float outputs."""
    n, H_q, d = q_raw.shape
    H_kv = k_raw.shape[1]
    G = H_q // H_kv
    cache = []
    outs = np.zeros((n, H_q, d))
    for p in range(n):
        qr = O.to_f64(O.rope_rotate(q_raw[p], dtype, cos[p], sin[p]), dtype)
        kr = O.to_f64(O.rope_rotate(k_raw[p], dtype, cos[p], sin[p]), dtype)
        cache.append((kr, O.to_f64(v_raw[p], dtype)))
        if len(cache) > W:
            cache = cache[-W:]
        for h in range(H_q):
            j = h // G
            s = [sum(float(qr[h, i]) * float(k[j, i]) for i in range(d)) / math.sqrt(d) for k, _ in cache]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for i in range(d):
                outs[p, h, i] = sum(wt * float(v[j, i]) for wt, (_, v) in zip(w, cache)) / z
    return outs


def _grow(M, q_raw, k_raw, v_raw, T_full, T_ring, cos, sin, dtype):
    """Append positions 0..n-1 of one sequence to a full cache (unwindowed
    oracle's append) and to a ring of T_ring slots; yield after every step."""
    n, H_q, d = q_raw.shape
    H_kv = k_raw.shape[1]
    zeros = lambda T: np.zeros((1, H_kv, T, d), np.float32)
    kf, vf = zeros(T_full), zeros(T_full)
    kr, vr = zeros(T_ring), zeros(T_ring)
    for p in range(n):
        pos = np.array([p])
        kf, vf, qf = O.append_contiguous(kf, vf, pos, k_raw[p:p + 1], v_raw[p:p + 1], cos, sin, dtype,
                                         q=q_raw[p:p + 1])
        kr, vr, qr = M.append_ring(kr, vr, pos, k_raw[p:p + 1], v_raw[p:p + 1], cos, sin, dtype, q=q_raw[p:p + 1])
        yield p, (kf, vf, qf), (kr, vr, qr)


# --- checks (True when the module passes) ------------------------------------


def check_listing_replay(M) -> bool:
    rng = np.random.default_rng(21)
    n, H_q, H_kv, d, W = 13, 4, 2, 8, 5
    cos, sin = O.rope_table(n, d)
    q_raw, k_raw, v_raw = _seq(rng, n, H_q, H_kv, d)
    ref = _listing_replay(q_raw, k_raw, v_raw, W, cos, sin, "f32")
    ok = True
    for p, (kf, vf, qf), (kr, vr, qr) in _grow(M, q_raw, k_raw, v_raw, n, W, cos, sin, "f32"):
        L = [p + 1]
        a = M.decode_attention_window(qf, kf, vf, L, W, "f32")[0]
        r = M.decode_attention_ring(qr, kr, vr, L, "f32")[0]
        ok &= bool(np.allclose(a, ref[p], rtol=0, atol=1e-12) and np.allclose(r, ref[p], rtol=0, atol=1e-12))
    return ok


def check_band_mask(M) -> bool:
    """Row p of a band-masked full recomputation == the windowed decode step p."""
    rng = np.random.default_rng(22)
    n, H_q, H_kv, d = 11, 6, 2, 16
    G = H_q // H_kv
    cos, sin = O.rope_table(n, d)
    q_raw, k_raw, v_raw = _seq(rng, n, H_q, H_kv, d, "bf16")
    qs = np.stack([O.to_f64(O.rope_rotate(q_raw[p], "bf16", cos[p], sin[p]), "bf16") for p in range(n)], 1)
    ks = np.stack([O.to_f64(O.rope_rotate(k_raw[p], "bf16", cos[p], sin[p]), "bf16") for p in range(n)], 1)
    vs = O.to_f64(v_raw, "bf16").transpose(1, 0, 2)
    ok = True
    for W in (1, 3, 7, 20):
        pp = np.arange(n)[:, None]
        tt = np.arange(n)[None, :]
        mask = torch.from_numpy((tt <= pp) & (tt > pp - W))
        full = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qs), torch.from_numpy(np.repeat(ks, G, axis=0)),
            torch.from_numpy(np.repeat(vs, G, axis=0)), attn_mask=mask).numpy()     # [H_q, n, d]
        for p, (kf, vf, qf), _ in _grow(M, q_raw, k_raw, v_raw, n, max(W, 1), cos, sin, "bf16"):
            a = M.decode_attention_window(qf, kf, vf, [p + 1], W, "bf16")[0]
            ok &= bool(np.allclose(a, full[:, p], rtol=0, atol=1e-12))
    return ok


def check_closed_forms(M) -> bool:
    rng = np.random.default_rng(23)
    B, H_q, H_kv, T, d = 3, 4, 2, 12, 16
    k = O.round_store(rng.standard_normal((B, H_kv, T, d)).astype(np.float32), "bf16")
    v = O.round_store(rng.standard_normal((B, H_kv, T, d)).astype(np.float32), "bf16")
    q = O.round_store(rng.standard_normal((B, H_q, d)).astype(np.float32), "bf16")
    L = [12, 5, 1]
    ok = True
    for W in (12, 13, 100):            # the window covers every token
        ok &= bool(np.array_equal(M.decode_attention_window(q, k, v, L, W, "bf16"),
                                  O.decode_attention(q, k, v, L, "bf16")))
    ok &= bool(np.array_equal(M.decode_attention_window(q, k, v, L, 0, "bf16"),
                              O.decode_attention(q, k, v, L, "bf16")))
    one = M.decode_attention_window(q, k, v, L, 1, "bf16")
    for b in range(B):
        for h in range(H_q):
            ok &= bool(np.array_equal(one[b, h], O.to_f64(v[b, h // 2, L[b] - 1], "bf16")))
    return ok


def check_ring_contents(M) -> bool:
    """After n > T steps, slot s holds the token t in [n - T, n) with t = s mod T."""
    rng = np.random.default_rng(24)
    n, H_q, H_kv, d, T = 17, 2, 1, 8, 5
    cos, sin = O.rope_table(n, d)
    q_raw, k_raw, v_raw = _seq(rng, n, H_q, H_kv, d)
    ok = True
    for p, (kf, vf, _), (kr, vr, _) in _grow(M, q_raw, k_raw, v_raw, n, T, cos, sin, "f32"):
        for t in range(max(0, p + 1 - T), p + 1):
            ok &= bool(np.array_equal(kr[0, :, t % T], kf[0, :, t]) and np.array_equal(vr[0, :, t % T], vf[0, :, t]))
    return ok


def check_paged(M) -> bool:
    rng = np.random.default_rng(25)
    B, H_q, H_kv, bs, d = 3, 4, 2, 4, 16
    T = 20
    nb = T // bs
    k = O.round_store(rng.standard_normal((B, H_kv, T, d)).astype(np.float32), "bf16")
    v = O.round_store(rng.standard_normal((B, H_kv, T, d)).astype(np.float32), "bf16")
    q = O.round_store(rng.standard_normal((B, H_q, d)).astype(np.float32), "bf16")
    table = rng.permutation(B * nb).reshape(B, nb)
    pk = np.zeros((B * nb, H_kv, bs, d), np.uint16)
    pv = np.zeros_like(pk)
    for b in range(B):
        for lb in range(nb):
            pk[table[b, lb]] = k[b, :, lb * bs:(lb + 1) * bs]
            pv[table[b, lb]] = v[b, :, lb * bs:(lb + 1) * bs]
    L = [20, 9, 3]
    ok = True
    for W in (1, 6, 7, 30):
        ok &= bool(np.array_equal(M.decode_attention_window_paged(q, pk, pv, table, bs, L, W, "bf16"),
                                  M.decode_attention_window(q, k, v, L, W, "bf16")))
    return ok


CHECKS = [check_listing_replay, check_band_mask, check_closed_forms, check_ring_contents, check_paged]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_pin_holds(chk):
    assert chk(WO)


def test_window_start_examples():
    """Mistral's 4096-token window ([KVC] step 6): a sequence of 5000 tokens
    attends tokens 904..4999; one of 4096 or fewer attends all of them."""
    assert WO.window_start(5000, 4096) == 904
    assert WO.window_start(4096, 4096) == 0
    assert WO.window_start(10, 4096) == 0
    assert WO.window_start(10, 0) == 0


# --- planted mistakes -------------------------------------------------------

MUTATIONS = {
    "window starts one late": ("max(0, L - window) if", "max(0, L - window + 1) if"),
    "window starts one early": ("max(0, L - window) if", "max(0, L - window - 1) if"),
    "start not clamped at zero": ("max(0, L - window) if", "(L - window) if"),
    "ring slot shifted": ("return pos % T", "return (pos + 1) % T"),
    "ring attends one slot less": ("min(int(L), T) for L", "min(int(L), T - 1) for L"),
    "ring append stops at the last slot": ("s = ring_slot(p, T)", "s = min(p, T - 1)"),
    "ring key rotated at its slot": ("O.rope_rotate(k_new[b], dtype, cos[p], sin[p], style)",
                                     "O.rope_rotate(k_new[b], dtype, cos[s], sin[s], style)"),
    "paged window cut from the front": ("K = O.gather_paged(k_pool, block_table, block_size, b, L)[None, :, lo:L]",
                                        "K = O.gather_paged(k_pool, block_table, block_size, b, L)[None, :, :L - lo]"),
}


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("window_oracle_mutant")
    src = src.replace("from . import kvc_oracle as O", "import oracle.kvc_oracle as O")
    exec(compile(src, "window_oracle_mutant", "exec"), m.__dict__)
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
