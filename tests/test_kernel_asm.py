"""Checks on the gfx950 assembly of the streaming decode kernels (CPU only:
hipcc cross-compiles; nothing runs on a GPU).

* Every transposed read of a staged V tile (ds_read_b64_tr_b16) must come after
  an s_waitcnt that leaves at most one tile's loads outstanding, counted from
  the last direct-to-LDS load before it.  The V rows reach LDS by direct
  loads; a build whose compiler-placed waits missed this read stale tiles
  from the second loop iteration on, so the kernels place the wait
  themselves, and this guards it.
* No direct-to-LDS load may be issued while an LDS read may still be
  outstanding (an s_waitcnt lgkmcnt(0) must come between them).  A direct
  load writes LDS when its data returns, outside the order of the wave's DS
  instructions; a build that let the compiler move a stage's refill in among
  the previous tile's reads of that stage gave wrong results where the refill
  lay past the split (such loads return almost at once).
* The kernels used at head_dim 64 / 128 must not spill to scratch.

Both waits are checked on every path through each kernel's control-flow
graph (basic blocks from the labels and branches of the assembly).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mqa_decode_attention_amd", "csrc", "kvc_decode_mfma.hip")
SRC_U8 = os.path.join(ROOT, "mqa_decode_attention_amd", "csrc", "kvc_decode_u8.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _compile(tmp_path_factory, src, name):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / name
    subprocess.run([cc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    src, "-o", str(out)], check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, SRC, "decode_mfma.s")


@pytest.fixture(scope="module")
def asm_u8(tmp_path_factory):
    return _compile(tmp_path_factory, SRC_U8, "decode_u8.s")


def kernels_u8(text):
    """(mangled name, head_dim, mode, lines) of each quantized-cache decode kernel."""
    lines = text.split("\n")
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3kvc\S*decode_u8_kernelILi(\d+)ELi\d+ELi(\d+)E\S*):", l)
        if m:
            end = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
            yield m.group(1), int(m.group(2)), int(m.group(3)), [x.split(";")[0].strip() for x in lines[i + 1:end]]


def kernels(text, with_hb=False):
    """(mangled name, head_dim, cache mode, lines) of each streaming decode kernel
    (template arguments: head_dim, head blocks, waves, mode, fused), from its
    label to the end of the function (blocks may follow an s_endpgm); with
    with_hb, (name, head_dim, mode, (head blocks, several new tokens), lines)."""
    lines = text.split("\n")
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3kvc\S*decode_mfma_kernelILi(\d+)ELi(\d+)ELi\d+ELi(\d+)ELb\dELb(\d)E\S*):", l)
        if m:
            end = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
            body = [x.split(";")[0].strip() for x in lines[i + 1:end]]
            if with_hb:
                yield m.group(1), int(m.group(2)), int(m.group(4)), (int(m.group(3)), m.group(5) == "1"), body
            else:
                yield m.group(1), int(m.group(2)), int(m.group(4)), body


def tile_loads(d, mode, hb=1, mq=False):
    """Vector memory operations one wave may have outstanding at a transposed
    read: a contiguous cache up to d = 128 stages 16-row tiles, K and V both by
    direct loads, one tile ahead (two head blocks of several new tokens' rows:
    two tiles ahead); otherwise 32-row tiles, K into registers (two 16-row
    blocks of d / 32 chunks)."""
    lanes_per_row = d // 8
    if mode == 0 and d <= 128:
        return 2 * (16 * lanes_per_row // 64) * (2 if hb == 2 and mq else 1)
    return 2 * (d // 32) + 32 * lanes_per_row // 64


def is_lds_dma(ins):
    return ("buffer_load" in ins and ins.endswith(" lds")) or "global_load_lds" in ins


def basic_blocks(body):
    """[(label, instructions, successor labels)] in layout order.  A block ends
    at a label or after a branch or s_endpgm (blocks reached only by falling
    through a conditional branch have no label in the assembly)."""
    raw, label, ins = [], "entry", []
    for line in body:
        if re.match(r"^\.LBB\S*:$", line):
            raw.append((label, ins))
            label, ins = line[:-1], []
        elif line and not line.startswith(".") and not line.startswith("%"):
            ins.append(line)
            if re.match(r"s_(c?branch|endpgm)", line):
                raw.append((label, ins))
                label, ins = f"fallthrough{len(raw)}", []
    raw.append((label, ins))
    out = []
    for k, (lab, ins) in enumerate(raw):
        succ = []
        last = ins[-1] if ins else ""
        m = re.match(r"s_(c?)branch\S*\s+(\.LBB\S+)", last)
        if m:
            succ.append(m.group(2))
        if not (last.startswith("s_branch") or last.startswith("s_endpgm")) and k + 1 < len(raw):
            succ.append(raw[k + 1][0])
        out.append((lab, ins, succ))
    return out


def flagged(body, sets, clears, check):
    """Instructions satisfying `check` that some path reaches with a `sets`
    instruction after the last `clears` one (forward dataflow, OR at joins)."""
    bl = basic_blocks(body)
    idx = {lab: k for k, (lab, _, _) in enumerate(bl)}
    state_in = [False] * len(bl)

    def run(k, report=None):
        st = state_in[k]
        for i in bl[k][1]:
            if report is not None and check(i) and st:
                report.append(i)
            if sets(i):
                st = True
            elif clears(i):
                st = False
        return st

    changed = True
    while changed:
        changed = False
        for k in range(len(bl)):
            if run(k):
                for s in bl[k][2]:
                    j = idx.get(s)
                    if j is not None and not state_in[j]:
                        state_in[j] = changed = True
    bad = []
    for k in range(len(bl)):
        run(k, bad)
    return bad


def waitcnt_field(ins, field):
    m = re.search(field + r"\((\d+)\)", ins) if ins.startswith("s_waitcnt") else None
    return int(m.group(1)) if m else None


def unguarded_transposed_reads(body, limit):
    def clears(i):
        v = waitcnt_field(i, "vmcnt")
        return v is not None and v <= limit
    return flagged(body, is_lds_dma, clears, lambda i: i.startswith("ds_read_b64_tr_b16"))


def refills_over_pending_reads(body):
    return flagged(body, lambda i: i.startswith("ds_read"), lambda i: waitcnt_field(i, "lgkmcnt") == 0, is_lds_dma)


def test_dataflow_sees_waits_on_back_edges():
    """The checker itself: a wait placed on the loop's back edge, laid out after
    the read it guards, counts; a path that skips it does not."""
    loop = [".LBB0_1:", "ds_read_b64_tr_b16 v[0:1], v2", "buffer_load_dwordx4 v3, s[0:3], 0 offen lds",
            "s_waitcnt vmcnt(4)", "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    pre = ["buffer_load_dwordx4 v3, s[0:3], 0 offen lds", "s_waitcnt vmcnt(0)"]
    assert unguarded_transposed_reads(pre + loop, 4) == []
    skip = ["buffer_load_dwordx4 v3, s[0:3], 0 offen lds", "s_cbranch_vccz .LBB0_2", "s_waitcnt vmcnt(0)",
            ".LBB0_2:", "ds_read_b64_tr_b16 v[0:1], v2", "s_endpgm"]
    assert unguarded_transposed_reads(skip, 4) == ["ds_read_b64_tr_b16 v[0:1], v2"]
    refill = ["ds_read_b128 v[0:3], v4", "s_cbranch_vccz .LBB0_3", "s_waitcnt lgkmcnt(0)", ".LBB0_3:",
              "buffer_load_dwordx4 v3, s[0:3], 0 offen lds", "s_endpgm"]
    assert refills_over_pending_reads(refill) == ["buffer_load_dwordx4 v3, s[0:3], 0 offen lds"]


def test_transposed_reads_wait_for_their_tile(asm):
    seen = 0
    for name, d, mode, (hb, mq), body in kernels(asm, with_hb=True):
        seen += 1
        bad = unguarded_transposed_reads(body, tile_loads(d, mode, hb, mq))
        assert not bad, f"{name}: transposed V reads with no wait for their tile's loads: {bad[:2]}"
    assert seen >= 12, "expected the decode kernel instantiations in the assembly"


def test_no_refill_while_lds_reads_pending(asm):
    seen = 0
    for name, d, mode, body in kernels(asm):
        seen += 1
        bad = refills_over_pending_reads(body)
        assert not bad, f"{name}: direct-to-LDS loads issued while LDS reads may be outstanding: {bad[:2]}"
    assert seen >= 12


def test_no_scratch_at_common_head_dims(asm):
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        name, body = m.group(1), m.group(2)
        if "decode_mfma_kernelILi64E" in name or "decode_mfma_kernelILi128E" in name:
            scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", body).group(1))
            assert scratch == 0, f"{name} spills {scratch} bytes per lane"


def test_u8_no_refill_while_lds_reads_pending(asm_u8):
    seen = 0
    for name, d, mode, body in kernels_u8(asm_u8):
        seen += 1
        bad = refills_over_pending_reads(body)
        assert not bad, f"{name}: direct-to-LDS loads issued while LDS reads may be outstanding: {bad[:2]}"
    assert seen >= 8


def test_u8_staged_reads_wait_for_their_loads(asm_u8):
    """Reads of staged codes and pairs (64/128-bit LDS reads) come after a wait
    that leaves at most one tensor's tile loads outstanding (codes d / 32 loads
    plus 1 or 2 pair loads), the transposed reads of the V codes included.
    Excluded: 32-bit reads (table entries and the merge's scalars)."""
    def staged_read(i):
        return (i.startswith("ds_read") and not re.match(r"ds_read2?(st64)?_b32", i)
                and not i.startswith("ds_read_u") and not i.startswith("ds_read_i"))
    seen = 0
    for name, d, mode, body in kernels_u8(asm_u8):
        seen += 1
        limit = d // 32 + (2 if mode == 3 else 1)
        def clears(i, limit=limit):
            v = waitcnt_field(i, "vmcnt")
            return v is not None and v <= limit
        bad = flagged(body, is_lds_dma, clears, staged_read)
        assert not bad, f"{name}: staged reads with no wait for their loads: {bad[:2]}"
    assert seen >= 8


def test_u8_no_scratch(asm_u8):
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm_u8, re.S):
        name, body = m.group(1), m.group(2)
        if "decode_u8_kernel" in name:
            scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", body).group(1))
            assert scratch == 0, f"{name} spills {scratch} bytes per lane"
