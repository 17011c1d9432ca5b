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

(Straight-line scans in layout order.)
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mqa_decode_attention_amd", "csrc", "kvc_decode_mfma.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "decode_mfma.s"
    subprocess.run([cc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    SRC, "-o", str(out)], check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


def kernels(text):
    """(mangled name, head_dim, cache mode, instruction lines) of each streaming
    decode kernel (template arguments: head_dim, head blocks, waves, mode, fused)."""
    lines = text.split("\n")
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3kvc\S*decode_mfma_kernelILi(\d+)ELi\d+ELi\d+ELi(\d+)E\S*):", l)
        if m:
            end = next(k for k in range(i, len(lines)) if "s_endpgm" in lines[k])
            yield m.group(1), int(m.group(2)), int(m.group(3)), [x.split(";")[0].strip() for x in lines[i:end]]


def tile_loads(d, mode):
    """Vector memory operations of one wave's tile: a contiguous cache up to
    d = 128 stages 16-row tiles, K and V both by direct loads; otherwise
    32-row tiles, K into registers (two 16-row blocks of d / 32 chunks)."""
    lanes_per_row = d // 8
    if mode == 0 and d <= 128:
        return 2 * (16 * lanes_per_row // 64)
    return 2 * (d // 32) + 32 * lanes_per_row // 64


def is_lds_dma(ins):
    return ("buffer_load" in ins and ins.endswith(" lds")) or "global_load_lds" in ins


def unguarded_transposed_reads(body, limit):
    pending, bad = False, []
    for ins in body:
        if is_lds_dma(ins):
            pending = True
        elif ins.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", ins)
            if m and int(m.group(1)) <= limit:
                pending = False
        elif ins.startswith("ds_read_b64_tr_b16") and pending:
            bad.append(ins)
    return bad


def refills_over_pending_reads(body):
    pending, bad = False, []
    for ins in body:
        if ins.startswith("ds_read"):
            pending = True
        elif ins.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", ins)
            if m and int(m.group(1)) == 0:
                pending = False
        elif is_lds_dma(ins) and pending:
            bad.append(ins)
    return bad


def test_transposed_reads_wait_for_their_tile(asm):
    seen = 0
    for name, d, mode, body in kernels(asm):
        seen += 1
        bad = unguarded_transposed_reads(body, tile_loads(d, mode))
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
