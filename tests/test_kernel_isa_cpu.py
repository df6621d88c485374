"""Code-generation guards for the GEMM kernel (no GPU needed).

The GEMM's K loop overlaps LDS DMA (buffer_load ... lds, counted by vmcnt)
with LDS fragment reads.  If the compiler cannot tell the two apart it
inserts a full `s_waitcnt vmcnt(0)` before the reads, which serialises the
loads with the MFMAs and roughly halves throughput without changing any
result, so no parity test would notice.  These tests compile the kernel
source for gfx950 with the library's own flags and read the AMD assembly.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sequence_transformer_gemms_amd", "csrc", "gemm_mfma.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from sequence_transformer_gemms_amd import build
    if not os.path.exists(build.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm_mfma.s"
    cmd = [build.HIPCC, *build.COMMON, "--cuda-device-only", "-S", "-x", "hip", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def kernels(text):
    """{mangled gemm_kernel / gemm_pair_kernel name: (body lines, metadata dict)}"""
    lines = text.split("\n")
    bodies, cur = {}, None
    for ln in lines:
        m = re.match(r"^(_ZN\S*gemm_(?:pair_)?kernel\S*):", ln)
        if m:
            cur = m.group(1)
            bodies[cur] = []
            continue
        if cur is not None:
            if ln.strip().startswith("s_endpgm"):
                cur = None
            else:
                bodies[cur].append(ln.strip())
    meta = {}
    for block in re.split(r"\n\s*- \.", text):
        nm = re.search(r"\.name:\s+(\S*gemm_(?:pair_)?kernel\S*)", block)
        if not nm:
            continue
        vals = {k: int(v) for k, v in re.findall(r"\.(vgpr_spill_count|sgpr_spill_count|group_segment_fixed_size"
                                                 r"|private_segment_fixed_size):\s+(\d+)", block)}
        meta[nm.group(1)] = vals
    return bodies, meta


def test_every_gemm_variant_is_compiled(asm):
    bodies, meta = kernels(asm)
    # 4 bf16 operand layouts + gated + fp8 (3 format pairs) + MXFP8, and the
    # paired linear-backward launch (either GEMM first)
    assert len(bodies) == 11
    assert set(meta) == set(bodies)


def k_loops(body):
    """Instruction lists of the K loops of a kernel body: loop bodies (a label
    and the backward branch to it) holding at least 16 MFMAs."""
    code = [ln for ln in body if ln and not ln.startswith(";")]
    labels = {}
    for i, ln in enumerate(code):
        m = re.match(r"^(\.LBB\d+_\d+):", ln)
        if m:
            labels[m.group(1)] = i
    loops, seen = [], set()
    for i, ln in enumerate(code):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i and m.group(1) not in seen:
            seg = code[labels[m.group(1)]:i + 1]
            if sum(x.startswith("v_mfma") for x in seg) >= 16 and len(seg) < 1000:
                seen.add(m.group(1))
                loops.append(seg)
    return loops


def test_no_full_vmcnt_wait_before_lds_reads(asm):
    # in the K loop (the epilogue may wait for its own global loads)
    bodies, _ = kernels(asm)
    for name, body in bodies.items():
        loops = k_loops(body)
        assert loops, f"{name}: no K loop found"
        for code in loops:
            bad = [i for i in range(len(code) - 1)
                   if re.match(r"s_waitcnt\s+vmcnt\(0\)", code[i]) and code[i + 1].startswith("ds_read")]
            assert not bad, f"{name}: {len(bad)} x 's_waitcnt vmcnt(0)' right before an LDS read in the K loop"


def test_k_loop_forms_lds_dma_addresses_in_32_bits(asm):
    # Casting a generic pointer to an LDS address per DMA load costs a 64-bit
    # add, a compare against the null pointer and a select, all scalar
    # instructions in front of every load (272 of them in the K loops when
    # the loads took generic pointers).  The loops form the LDS addresses as
    # 32-bit offsets; the null compare is the cast's signature.
    bodies, _ = kernels(asm)
    for name, body in bodies.items():
        for code in k_loops(body):
            casts = [ln for ln in code if re.match(r"s_cmp_lg_u64\s", ln)]
            assert not casts, f"{name}: {len(casts)} x 's_cmp_lg_u64' (generic-to-LDS casts) in the K loop"


def test_no_register_spills_and_lds_fits(asm):
    # (scalar registers that overflow go to VGPR lanes, not memory: allowed)
    _, meta = kernels(asm)
    for name, m in meta.items():
        assert m.get("vgpr_spill_count", 0) == 0, name
        assert m.get("private_segment_fixed_size", 0) == 0, name
        assert m["group_segment_fixed_size"] <= 160 * 1024, name
