"""The compacted schedule of the bf16 matrix-core decode kernel (contiguous
cache, split plans of several rounds), modelled on the host (no GPU).

The host plans the shortest split length the kernel may use (T_min, which
sizes the workspace: n_splits partial slots per output row) and launches
B * H_kv * n_splits workgroups.  Every workgroup reads all lengths and picks
the split length T itself: a first estimate from the tokens the splits cover
over the slots (less half a split per unit), then longer until the units'
splits fit in one round of `slots` workgroups (twice in proportion to the
count's excess, then in proportion to the splits beyond each unit's first;
five times at most); never shorter than T_min nor longer than one split per
sequence.  The splits that exist, counted in unit order (unit u = b * H_kv + j holds
nsp_b splits), take workgroup indices 0, 1, ...; the others exit.  The first
split of each unit records nsp_b for the merge kernel.

This model restates that integer arithmetic and checks, over many ragged
shapes and windows, what the kernel relies on: every split of every unit is
taken by exactly one workgroup; the workgroups that exist cover them (the
count never exceeds the launched grid); every split index stays below
n_splits, so its partial slot lies inside the workspace; T is a multiple of
the loop step between T_min and one split per sequence; the splits of one
unit tile its attended range.  The library's own plan (split length, whether
the schedule applies) is read back through the C ABI, which needs no GPU.
"""
import random

import pytest
import torch

import mqa_decode_attention_amd as kvc

CU = 256             # compute units the library assumes without a device (MI355X)
CMP_CHUNKS = 4       # kvc_internal.h: kCmpChunks (64 lengths each)


def token_range(L, window=0, ring=0, T_max=0):
    """[lo, hi) attended and the splits' origin org (contiguous cache: align 1)."""
    if ring:
        return 0, min(L, T_max), 0
    lo = L - window if (window > 0 and L > window) else 0
    return lo, L, lo


def splits(L, T, tail, **kw):
    lo, hi, org = token_range(L, **kw)
    return max(1, (hi - org - tail + T - 1) // T)


def pick_T(lens, H_kv, t_min, tmax, step, slots, tail, **kw):
    """The kernel's choice of split length (cmp_locate)."""
    span = sum(token_range(L, **kw)[1] - token_range(L, **kw)[2] for L in lens)
    units = len(lens) * H_kv
    room = max(1, slots - units // 2)
    # (float32 on the device; only the starting point of the search)
    steps = -(-(span * H_kv) // (room * step))
    T = tmax if steps >= tmax // step else steps * step
    T = max(T, t_min)
    for n_pass in range(6):
        cnt = sum(splits(L, T, tail, **kw) for L in lens) * H_kv
        if cnt <= slots or T >= tmax or n_pass == 5:
            break
        free = max(1, slots - units)
        grown = T * cnt // slots if n_pass < 2 else (T * (cnt - units) + free - 1) // free
        T = min(max(T + step, (grown + step - 1) // step * step), tmax)
    return T


def locate(wid, lens, H_kv, T, tail, **kw):
    """(unit, split, nsp) of workgroup wid, or None: the prefix sum of H_kv * nsp_b."""
    before = 0
    for b, L in enumerate(lens):
        n = splits(L, T, tail, **kw) * H_kv
        if wid < before + n:
            r = wid - before
            nsp = n // H_kv
            return b * H_kv + r // nsp, r % nsp, nsp
        before += n
    return None


def host_plan(B, H_q, H_kv, d, max_len, window=0):
    """The library's plan through the C ABI, plus the model's host constants."""
    G = H_q // H_kv
    step = 64 if d <= 128 else 128
    per_cu = 2 if (d <= 64 and G > 16) else (1 if G > 16 else (2 if d <= 64 else 1))
    slots = CU * per_cu
    span = kvc.window_span(max_len, window) if window else max_len
    is_compact = kvc.compact(torch.bfloat16, B, H_q, H_kv, d, span)
    t_min = kvc.split_tokens(torch.bfloat16, B, H_q, H_kv, d, span)
    tail = 0          # (no remainder joins a last split under this schedule)
    n_splits = max(1, (max(span, 1) - tail + t_min - 1) // t_min)
    tmax = (max(span, 1) + step - 1) // step * step
    return is_compact, t_min, n_splits, tmax, step, slots, tail


def check(lens, H_q, H_kv, d, window=0):
    B = len(lens)
    max_len = max(lens)
    is_compact, t_min, n_splits, tmax, step, slots, tail = host_plan(B, H_q, H_kv, d, max_len, window)
    assert is_compact, f"expected the compacted schedule for B={B} H_q={H_q} H_kv={H_kv} d={d} max_len={max_len}"
    kw = dict(window=window)
    T = pick_T(lens, H_kv, t_min, tmax, step, slots, tail, **kw)
    assert T % step == 0 and t_min <= T <= max(tmax, t_min), (T, t_min, tmax)
    grid = B * H_kv * n_splits
    seen = {}
    for wid in range(grid):
        got = locate(wid, lens, H_kv, T, tail, **kw)
        if got is None:
            continue
        u, s, nsp = got
        assert s < nsp <= n_splits, "split index past the workspace's partial slots"
        assert (u, s) not in seen, f"split {(u, s)} taken twice"
        seen[(u, s)] = wid
    want = {(b * H_kv + j, s) for b, L in enumerate(lens) for j in range(H_kv)
            for s in range(splits(L, T, tail, **kw))}
    assert set(seen) == want, "some split has no workgroup"
    # the workgroups taking a split are exactly 0 .. total - 1
    assert sorted(seen.values()) == list(range(len(want)))
    # the splits of a unit tile [org, hi): split s covers [org + s T, ...), the last to hi
    for b, L in enumerate(lens):
        lo, hi, org = token_range(L, **kw)
        nsp = splits(L, T, tail, **kw)
        cover = []
        for s in range(nsp):
            e = org + (s + 1) * T
            cover.append((org + s * T, hi if (s == nsp - 1 or e > hi) else e))
        assert cover[0][0] == org and cover[-1][1] == hi
        assert all(cover[i][1] == cover[i + 1][0] for i in range(nsp - 1))
        assert all(a < z or (hi == org) for a, z in cover), "empty split of a nonempty range"
    total = len(want)
    return T, total, slots


def test_ragged_mqa_workload_fits_one_round():
    g = torch.Generator().manual_seed(2)
    lens = (torch.randint(512, 4097, (64,), generator=g) + 1).tolist()
    T, total, slots = check(lens, 32, 1, 128)
    assert total <= slots, (T, total)
    # the shortest step multiple that fits: one step less would not
    assert T == 640, T
    assert sum(splits(L, T - 64, 0) for L in lens) > slots


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(seed):
    rnd = random.Random(seed)
    d = rnd.choice([64, 128, 256])
    H_kv = rnd.choice([1, 1, 2, 4])
    G = rnd.choice([20, 24, 32])
    if d == 256:
        G = min(G, 32)
    slots = CU * (2 if d <= 64 else 1)
    B = rnd.randint(1, min(256, max(1, slots // (2 * H_kv))))
    max_len = rnd.choice([20000, 40000, 70000])
    lens = [rnd.choice([0, 1, 2, 63, 64, 65, rnd.randint(1, max_len)]) for _ in range(B)]
    lens[rnd.randrange(B)] = max_len
    window = rnd.choice([0, 0, 0, rnd.randint(1, max_len)])
    H_q = G * H_kv
    is_compact = host_plan(B, H_q, H_kv, d, max_len, window)[0]
    if not is_compact:
        pytest.skip("a one-round plan for these sizes")
    T, total, slots = check(lens, H_q, H_kv, d, window)
    tmax = host_plan(B, H_q, H_kv, d, max_len, window)[3]
    assert total <= slots or T >= tmax, (T, total, slots)
    # close to the shortest step multiple that fits
    step = 64 if d <= 128 else 128
    t = host_plan(B, H_q, H_kv, d, max_len, window)[1]
    while t < tmax and sum(splits(L, t, 0, window=window) for L in lens) * H_kv > slots:
        t += step
    assert T <= t * 1.1 + 128, (T, t)


def test_uniform_long_lengths():
    lens = [16385] * 8
    T, total, slots = check(lens, 32, 1, 128)
    assert total <= slots


def test_not_used_where_the_split_plan_is_one_round():
    # gqa_8b and long_gqa: one round of the split plan
    assert not kvc.compact(torch.bfloat16, 16, 32, 8, 128, 8193)
    assert not kvc.compact(torch.bfloat16, 1, 64, 8, 128, 131073)
    # paged pools, explicit split lengths, float32 and the quantized cache keep their plans
    assert not kvc.compact(torch.bfloat16, 64, 32, 1, 128, 4097, pool_tokens=64 * 4112)
    assert not kvc.compact(torch.bfloat16, 64, 32, 1, 128, 4097, split_tokens=384)
    assert not kvc.compact(torch.float32, 64, 32, 1, 128, 4097)
    assert kvc.compact(torch.bfloat16, 64, 32, 1, 128, 4097)
    assert kvc.merge_launch(torch.bfloat16, 64, 32, 1, 128, 4097) is True
