"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

- Every buffer-to-LDS DMA takes a zero scalar offset; the k-step offset is carried by the
  descriptor base, the form AMD's own libraries use for these loads on gfx950.  (An earlier
  kernel with a nonzero scalar offset faulted, but it also carried the sign-extension bug
  below, which its compiled code shows and which is the cause; the zero offset is kept as
  the documented form, not as the fix.)
- No kernel spills to scratch, and none needs a waterfall loop around a DMA (a descriptor
  or offset the compiler believes divergent).
- No scalar sign-extension of a 32-bit word into 64 bits (s_bfe_i64 with width 32).  A
  buffer-descriptor helper once rebuilt a pointer from two readfirstlane results, whose
  signed int type sign-extended the low word into the high word whenever bit 31 of the
  address was set: the descriptor base became 0xffff'xxxx'xxxx and the first access faulted.
- No __builtin_bit_cast of a subscripted vector element in the kernel sources: this hipcc
  reads element 0 whatever the subscript (an fp32 epilogue built that way stored column 0
  of every 4-column run four times).  The compiler behaviour itself is pinned too.
- Every 16-byte output store takes four distinct registers (no broadcast of one value).
- The one-role kernel writes its MFMAs as inline asm, whose results the compiler's hazard
  tracking does not see: no accumulator is read, moved or stored within 20 wait states of an
  MFMA, and none is written by a vector instruction within 3 wait states before one.  Its
  k-loop holds only the matrix instructions, the fragment reads, the copies and the per-step
  scalar work: no address arithmetic between the MFMAs.
"""
import os
import re
import shutil
import subprocess

import pytest

from pipelined_tiled_gemm_amd import build

hipcc_missing = shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    # every device source, each with the flags the library is built with
    d = tmp_path_factory.mktemp("isa")
    text = []
    for src in build.DEVICE_SOURCES:
        out = d / (src + ".s")
        cmd = [build.hipcc(), *build.compile_flags(source=src), "-S", "--cuda-device-only",
               os.path.join(build.CSRC, src), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True)
        text.append(out.read_text())
    return "\n".join(text)


def kernels(asm_text):
    # the pipelined GEMM kernels, the one-role dense kernel and the attention kernel
    for m in re.finditer(r"\n(_ZN3ptg(?:10ptg_kernel|4attn16attention_kernel|12_GLOBAL__N_114onerole_kernel)\S+):",
                         asm_text):
        start = m.start()
        end = asm_text.index(".Lfunc_end", start)
        yield m.group(1), asm_text[start:end].split("\n")


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_lds_dma_scalar_offset_is_zero(asm):
    n = 0
    for name, body in kernels(asm):
        for line in body:
            if "buffer_load_dword" in line and " lds" in line:
                ops = line.split(None, 1)[1].split(",")
                assert ops[2].strip().split()[0] == "0", f"{name}: {line.strip()}"
                n += 1
    assert n > 0


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_no_scratch_and_no_waterfall(asm):
    for name, body in kernels(asm):
        assert not any("scratch_" in l for l in body), f"{name} spills to scratch"
        for k, line in enumerate(body):
            if "buffer_load_dword" in line and " lds" in line:
                assert "saveexec" not in body[k - 1], f"{name}: waterfall loop around a DMA"


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_no_sign_extended_address_words(asm):
    for name, body in kernels(asm):
        for line in body:
            if line.strip().startswith("s_bfe_i64") and line.strip().endswith("0x200000"):
                raise AssertionError(f"{name}: sign-extends a 32-bit word: {line.strip()}")


def test_promotion_rule_behind_the_guard():
    """The C rule the guard is about: an int OR-ed into a uint64_t is sign-extended, so a
    low address word with bit 31 set turns the high word into 0xffffffff."""
    lo_bits, hi = 0x9ABC0000, 0x00007F12
    as_int = lo_bits - (1 << 32) if lo_bits & (1 << 31) else lo_bits   # readfirstlane's int
    sign_extended = as_int & ((1 << 64) - 1)                              # int -> uint64_t
    wrong = (hi << 32) | sign_extended
    right = (hi << 32) | (as_int & 0xFFFFFFFF)                           # via uint32_t
    assert wrong >> 32 == 0xFFFFFFFF
    assert right == 0x00007F12_9ABC0000


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_no_bit_cast_of_vector_elements():
    pat = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+\s*\[")
    for name in os.listdir(build.CSRC):
        if name.endswith((".hip", ".hpp", ".h", ".cpp")):
            text = open(os.path.join(build.CSRC, name)).read()
            assert not pat.search(text), f"{name}: __builtin_bit_cast of a vector element"


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_compiler_bit_cast_of_element_reads_element_zero(tmp_path):
    """Why the rule above exists: bit_cast(float, x[2]) compiles to element 0."""
    src = tmp_path / "bc.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "typedef __attribute__((ext_vector_type(4))) unsigned u32x4;\n"
        "__global__ void k(const u32x4* in, float* out) {\n"
        "  u32x4 x = in[threadIdx.x];\n"
        "  out[threadIdx.x] = __builtin_bit_cast(float, x[2]);\n"
        "}\n")
    out = tmp_path / "bc.ll"
    subprocess.run([build.hipcc(), "--offload-arch=gfx950", "-O3", "--cuda-device-only", "-S",
                    "-emit-llvm", str(src), "-o", str(out)], check=True, capture_output=True)
    ir = out.read_text()
    # if a fixed compiler extracts element 2, this test fails and the rule can be relaxed
    assert "extractelement <4 x float> %6, i64 0" in ir or re.search(r"extractelement <4 x \w+> %\d+, i64 0", ir)


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_wide_output_stores_take_distinct_registers(asm):
    n = 0
    for name, body in kernels(asm):
        for k, line in enumerate(body):
            if "buffer_store_dwordx4" not in line:
                continue
            n += 1
            reg = line.split()[1].rstrip(",")          # v[a:b]
            a = int(reg[2:reg.index(":")])
            movs = [l for l in body[max(0, k - 8):k] if "v_mov_b32" in l]
            srcs = {}
            for l in movs:
                dst, src = [x.strip() for x in l.split(None, 1)[1].split(",")[:2]]
                if dst.startswith("v") and dst[1:].isdigit() and a <= int(dst[1:]) <= a + 3:
                    srcs[dst] = src
            assert len(srcs) < 4 or len(set(srcs.values())) > 1, f"{name}: broadcast store {line.strip()}"
    assert n > 0


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_stress_pauses_only_in_the_test_build(asm, tmp_path):
    """The product kernels read no cycle counter (the ring-stress pauses are compiled out);
    the stress build's GEMM kernels do, at their handoffs."""
    def memtimes(text):
        return sum(1 for _, body in kernels(text) for l in body if l.strip().startswith("s_memtime"))
    assert memtimes(asm) == 0
    out = tmp_path / "delay.s"
    src = "ptg_kernels.hip"
    cmd = [build.hipcc(), *build.compile_flags(build.VARIANTS["delay"], source=src), "-S",
           "--cuda-device-only", os.path.join(build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    assert memtimes(out.read_text()) > 0


def onerole_bodies(asm_text):
    """{form: kernel body} of the one-role kernel's four instantiations: B N x K or K x N
    ("nk", "kn"), bf16 or fp32 output (suffix "_f32")."""
    found = {}
    for name, body in kernels(asm_text):
        if "onerole_kernel" in name:
            # the Cfg's B_KN flag is its eighth template argument; the output flag follows the Cfg
            args = re.search(r"CfgILi256ELi256ELi32ELi5ELi2ELi2ELi4ELb(\d)\S*?EEELb(\d)E", name)
            found[("kn" if args.group(1) == "1" else "nk") + ("_f32" if args.group(2) == "1" else "")] = body
    assert sorted(found) == ["kn", "kn_f32", "nk", "nk_f32"], sorted(found)
    return found


def wait_states(line):
    m = re.match(r"s_nop (\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def instructions(body):
    for line in body:
        s = line.strip()
        if s and not s.startswith((";", ".")) and not s.endswith(":"):
            yield s


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
@pytest.mark.parametrize("variant", [None, "delay"])
def test_onerole_waits_for_its_asm_mfmas(asm, tmp_path, variant):
    """In code order (every block boundary after an MFMA run is preceded by the padding, so
    order is enough): reads of accumulators wait out the MFMA's passes, and writes to them
    come at least 3 wait states before the next MFMA.  Checked in the product and the stress
    build, whose pauses add block boundaries."""
    if variant is None:
        text = asm
    else:
        out = tmp_path / "onerole_delay.s"
        src = "ptg_onerole.hip"
        subprocess.run([build.hipcc(), *build.compile_flags(build.VARIANTS[variant], source=src), "-S",
                        "--cuda-device-only", os.path.join(build.CSRC, src), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    for layout, body in onerole_bodies(text).items():
        check_acc_waits(layout, body)
    # everything inlined: no calls, no accumulators passed through memory
    for body in onerole_bodies(text).values():
        assert not any(re.match(r"\s+(s_swappc|s_setpc|flat_load|flat_store|scratch_)", l) for l in body)
    assert not re.search(r"\n_ZZN3ptg12_GLOBAL__N_114onerole_kernel\S*:", text), "a lambda left out of line"


def check_acc_waits(layout, body):
    since_mfma, since_acc_write = None, 99
    n_mfma = 0
    for s in instructions(body):
        if s.startswith("v_mfma"):
            n_mfma += 1
            assert since_acc_write >= 3, f"{layout}: accumulator written {since_acc_write} wait states before {s}"
            since_mfma = 0
            since_acc_write += 1
            continue
        reads_acc = re.match(r"(v_accvgpr_(read|mov)|buffer_store|v_cvt|v_permlane)", s)
        if since_mfma is not None and reads_acc:
            assert since_mfma >= 20, f"{layout}: {s}: {since_mfma} wait states after an MFMA"
        if re.match(r"v_accvgpr_(write|mov)", s):
            since_acc_write = 0
        else:
            since_acc_write += wait_states(s)
        if since_mfma is not None:
            since_mfma += wait_states(s)
    assert n_mfma >= 640, layout


def vgprs(op):
    m = re.match(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
@pytest.mark.parametrize("variant", [None, "delay"])
def test_onerole_mfma_sources_settle(asm, tmp_path, variant):
    """No vector instruction writes a register that an asm MFMA reads as its A or B operand
    within 8 wait states before it (the compiler inserts no wait states for the asm): the
    fragment registers are written by LDS reads (counted waits) and by the one move of the
    x/y fragments before the last step, which is padded."""
    if variant is None:
        text = asm
    else:
        out = tmp_path / "onerole_delay.s"
        src = "ptg_onerole.hip"
        subprocess.run([build.hipcc(), *build.compile_flags(build.VARIANTS[variant], source=src), "-S",
                        "--cuda-device-only", os.path.join(build.CSRC, src), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    for layout, body in onerole_bodies(text).items():
        recent = []  # (wait states since, registers written, instruction)
        for s in instructions(body):
            if s.startswith("v_mfma"):
                ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
                src = vgprs(ops[1]) | vgprs(ops[2])
                for ago, w, txt in recent:
                    assert not (ago < 8 and w & src), f"{layout}: {txt} then {s} after {ago} wait states"
            elif s.startswith("v_") and not s.startswith("v_accvgpr_read") and " " in s:
                recent.append((0, vgprs(s.split(None, 1)[1].split(",")[0].strip()), s))
            recent = [(a + wait_states(s), w, x) for a, w, x in recent if a + wait_states(s) < 16]


def sgprs(op):
    m = re.match(r"s\[(\d+):(\d+)\]", op)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {op} if re.match(r"s\d+$", op) else set()


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
@pytest.mark.parametrize("variant", [None, "delay"])
def test_onerole_copies_wait_for_their_scalar_operands(asm, tmp_path, variant):
    """Every copy to LDS (a buffer load with the LDS flag) comes at least 5 wait states after a
    vector instruction (v_readfirstlane, v_readlane) wrote a scalar register of its descriptor,
    and at least 1 after a write of M0 (its LDS address); sooner, the load may read the old
    value.  The compiler pads its own loads (B stored N x K), not the asm copies (K x N), which
    carry the padding inside the asm.  Checked in code order, in the product and the stress
    build."""
    if variant is None:
        text = asm
    else:
        out = tmp_path / "onerole_delay.s"
        src = "ptg_onerole.hip"
        subprocess.run([build.hipcc(), *build.compile_flags(build.VARIANTS[variant], source=src), "-S",
                        "--cuda-device-only", os.path.join(build.CSRC, src), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    for layout, body in onerole_bodies(text).items():
        copies, bad = copy_operand_violations(instructions(body))
        assert not bad, f"{layout}: {bad[:3]}"
        assert copies >= 80, layout


def copy_operand_violations(lines):
    """(number of copies to LDS, list of violations) in an instruction sequence, in code order:
    a copy less than 5 wait states after a v_readfirstlane/v_readlane wrote a scalar register of
    its descriptor (a scalar write of that register in between clears it), or right after a
    write of M0."""
    since = {}  # scalar register (or m0) -> wait states since its last write of concern
    copies, bad = 0, []
    for s in lines:
        if re.match(r"buffer_load\S* .* lds$", s):
            copies += 1
            ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
            for r in sgprs(ops[1]):
                if since.get(r, 99) < 5:
                    bad.append(f"{s} reads {r} {since[r]} wait states after a vector write")
            if since.get("m0", 99) < 1:
                bad.append(f"{s} right after a write of m0")
        m = re.match(r"v_read(firstlane|lane)_b32 (s\d+),", s)
        w = re.match(r"s_\w+ m0,", s)
        for r in since:
            since[r] += wait_states(s)
        if m:
            since[m.group(2)] = 0
        elif re.match(r"s_\w+ (s\d+|s\[\d+:\d+\]),", s):
            # a scalar write replaces the vector one
            for r in sgprs(s.split(None, 1)[1].split(",")[0].strip()):
                since.pop(r, None)
        if w:
            since["m0"] = 0
    return copies, bad


def test_copy_operand_check_flags_hazards():
    """The check above on hand-written sequences: it flags a descriptor word or M0 written too
    shortly before a copy, and passes the padded and the unrelated cases."""
    load = "buffer_load_dwordx4 v139, s[16:19], 0 offen lds"
    cases = {
        ("v_readfirstlane_b32 s18, v128", load): 1,                     # size word, no wait
        ("v_readfirstlane_b32 s16, v1", "s_nop 2", load): 1,            # 3 wait states
        ("v_readfirstlane_b32 s18, v128", "s_nop 4", load): 0,          # 5 wait states
        ("v_readfirstlane_b32 s30, v128", load): 0,                     # not a descriptor word
        ("v_readfirstlane_b32 s18, v128", "s_mov_b32 s18, s5", load): 0,  # rewritten by a scalar op
        ("s_mov_b32 m0, s67", load): 1,                                 # M0, no wait
        ("s_add_i32 m0, s4, 0x1000", "s_nop 0", load): 0,               # M0, one wait state
        ("s_mov_b32 m0, s67", "v_readfirstlane_b32 s17, v2", load): 1,  # M0 waited, s17 not
    }
    for seq, n in cases.items():
        copies, bad = copy_operand_violations(list(seq))
        assert copies == 1 and len(bad) == n, (seq, bad)


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
@pytest.mark.parametrize("layout", ["nk", "kn", "nk_f32", "kn_f32"])
def test_onerole_k_loop_is_lean(asm, layout):
    """The k-loop (the block of ten unrolled steps): 640 MFMAs; the fragment reads (160 of 16
    bytes for B stored N x K; for K x N, 80 of 16 bytes for A and 160 transposing 8-byte reads
    for B); 80 copies to LDS; 10 barriers; no vector-memory wait for all copies; and no more
    than 40 other vector instructions (the copies' descriptor work), none of them writing LDS
    or touching scratch."""
    body = onerole_bodies(asm)[layout]
    blocks, cur = [], None
    for line in body:
        if re.match(r"^(\.LBB\S+|; %bb\.\d+):", line):
            cur = []
            blocks.append(cur)
        elif cur is not None:
            cur.append(line.strip())
    loops = [b for b in blocks if sum(l.startswith("v_mfma") for l in b) == 640]
    assert len(loops) == 1
    loop = loops[0]
    count = lambda p: sum(1 for l in loop if l.startswith(p))
    if layout.startswith("nk"):
        assert count("ds_read_b128") == 160
    else:
        assert count("ds_read_b128") == 80 and count("ds_read_b64_tr_b16") == 160
    assert count("buffer_load_dwordx4") == 80 and all(" lds" in l for l in loop if l.startswith("buffer_load"))
    assert count("s_barrier") == 10
    assert count("ds_write") == 0 and count("scratch_") == 0
    # the only vector-memory waits are the kernel's own per-step ones: a compiler wait for
    # every copy in flight (before an LDS read it cannot tell from the copies) serialises
    # copies and matrix work
    assert count("s_waitcnt vmcnt(0)") == 0
    other_valu = [l for l in loop if l.startswith("v_") and not l.startswith(("v_mfma", "v_accvgpr"))]
    assert len(other_valu) <= 40, other_valu
