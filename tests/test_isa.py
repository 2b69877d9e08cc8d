"""CPU checks on the generated gfx950 code (hipcc cross-compiles here).

* The direct-to-LDS kernel sets M0 in its own inline-asm DMA sequence; the
  compiler is told M0 is clobbered but treats it as reserved, so the code is
  only safe while nothing the compiler generates in these kernels reads or
  writes M0.  This test pins that.
* The library is built with packed fp32 disabled: no v_pk_*_f32 may appear.
* No kernel spills to scratch.
* The fused ReLU is a compare and select, never v_max_f32 (NaN must pass).
* The debug build (-DSGEMM_LDS_POISON) writes NaN over LDS stages between
  their retirement and their refill in every kernel that reuses a stage;
  the release build has none of it.
* The large wave-tile kernels issue their MFMAs as inline assembly, which the
  compiler's hazard checks do not see: the pauses the kernel writes itself
  must be in place (after the accumulators are zeroed, and at least 11 wait
  states between the last MFMA and the first instruction that reads an
  accumulator register), and no VALU instruction may write an MFMA operand
  just before it.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "register_lds_tiled_amd", "csrc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "--cuda-device-only", "-S"]


POISON = "-DSGEMM_LDS_POISON"   # the debug build's define (csrc/lds_poison.h)


def asm_of(src, tmp_path, *extra):
    out = tmp_path / (os.path.basename(src) + "".join(extra) + ".s")
    subprocess.run(["/opt/rocm/bin/hipcc", *FLAGS, *extra, src, "-o", str(out)], check=True,
                   capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def big_asm(tmp_path_factory):
    """The two large sources, release and LDS-poison builds, compiled side by
    side (each takes minutes).  Keys: file name, and file name + POISON."""
    d = tmp_path_factory.mktemp("isa")
    jobs = {}
    for name in ("sgemm_mfma.hip", "sgemm_lowp.hip"):
        for extra in ((), (POISON,)):
            key = name + "".join(extra)
            out = d / (key + ".s")
            jobs[key] = (out, subprocess.Popen(["/opt/rocm/bin/hipcc", *FLAGS, *extra,
                                                os.path.join(CSRC, name), "-o", str(out)],
                                               stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    texts = {}
    for name, (out, proc) in jobs.items():
        log = proc.communicate()[0]
        assert proc.returncode == 0, log.decode(errors="replace")[-2000:]
        texts[name] = out.read_text()
    return texts


@pytest.fixture(scope="module")
def mfma_asm(big_asm):
    return big_asm["sgemm_mfma.hip"]


@pytest.fixture(scope="module")
def lowp_asm(big_asm):
    return big_asm["sgemm_lowp.hip"]


@pytest.mark.parametrize("which", ["mfma", "lowp"])
def test_m0_only_in_dma_asm(which, mfma_asm, lowp_asm):
    lines = (mfma_asm if which == "mfma" else lowp_asm).splitlines()
    uses = [i for i, l in enumerate(lines) if re.search(r"\bm0\b", l) and not l.lstrip().startswith(";")]
    assert uses, "expected the DMA sequences to set M0"
    for i in uses:
        assert re.match(r"\s*s_mov_b32 m0, s\d+\s*$", lines[i]), lines[i]
        # the asm may first set EXEC to a lane mask (save, set, s_nop)
        j = i - 1
        if re.match(r"\s*s_nop 0\s*$", lines[j]):
            assert re.match(r"\s*s_mov_b64 exec, s\[\d+:\d+\]\s*$", lines[j - 1]), lines[j - 1]
            assert re.match(r"\s*s_mov_b64 s\[\d+:\d+\], exec\s*$", lines[j - 2]), lines[j - 2]
            assert re.match(r"\s*s_mov_b64 exec, s\[\d+:\d+\]\s*$", lines[i + 2]), lines[i + 2]
            j -= 3
        assert "ASMSTART" in lines[j], f"M0 write outside the DMA asm: {lines[i]}"
        assert re.match(r"\s*global_load_lds_dword(x4)?\s", lines[i + 1]), lines[i + 1]


@pytest.mark.parametrize("name", ["sgemm_mfma.hip", "sgemm_valu.hip", "sgemm_micro.hip",
                                  "sgemm_lowp.hip", "sgemm_skinny.hip"])
def test_no_packed_fp32_and_no_spills(name, tmp_path, request):
    # the two large sources are compiled once per module (their fixtures)
    fixture = {"sgemm_mfma.hip": "mfma_asm", "sgemm_lowp.hip": "lowp_asm"}.get(name)
    text = request.getfixturevalue(fixture) if fixture else asm_of(os.path.join(CSRC, name), tmp_path)
    assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", text)
    scratch = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", text)]
    assert scratch and max(scratch) == 0, f"scratch use {scratch}"


def test_streaming_kernels_relu_is_compare_and_select(tmp_path):
    """The few-row and few-column kernels apply the same epilogue in their
    store: no v_max_f32 there either."""
    text = asm_of(os.path.join(CSRC, "sgemm_skinny.hip"), tmp_path)
    assert not re.search(r"\bv_max_f32\b", text)


def test_fused_relu_is_compare_and_select(mfma_asm):
    """ReLU must let NaN through, so it may not be compiled to v_max_f32
    (which returns the other operand for NaN).  The kernels without the
    fused epilogue have no reason to use it either."""
    assert re.search(r"sgemm_mfma\w*kernel\w*Lb1EEEvNS_8GemmArgsEii:", mfma_asm), \
        "expected fused-epilogue kernel instances"
    assert not re.search(r"\bv_max_f32\b", mfma_asm)


def functions(asm, pattern):
    for name in re.findall(r"^(" + pattern + r"):", asm, re.M):
        start = asm.index(name + ":")
        end = asm.index(".Lfunc_end", start)
        lines = [l.split(";")[0].strip() for l in asm[start:end].splitlines()]
        yield name, [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]


def wait_states(lines):
    return sum(int(l.split()[1]) + 1 for l in lines if l.startswith("s_nop"))


@pytest.mark.parametrize("which", ["mfma", "lowp"])
def test_big_kernel_mfma_pauses(which, mfma_asm, lowp_asm):
    asm, pattern = ((mfma_asm, r"_Z\w*sgemm_mfma_big_kernel\w*") if which == "mfma"
                    else (lowp_asm, r"_Z\w*gemm_lowp_big_kernel\w*"))
    # result latency the pause must cover: 8-pass MFMAs need 11 wait states;
    # the 16-bit kernel keeps to the 16-pass figure (19)
    need = 11 if which == "mfma" else 19
    found = 0
    for name, lines in functions(asm, pattern):
        found += 1
        mfma = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        assert mfma, name
        first, last = mfma[0], mfma[-1]
        agpr = re.compile(r"\ba(\d+|\[\d+:\d+\])")
        # zeroing: the last AGPR write before the first MFMA
        zero = [i for i, l in enumerate(lines[:first])
                if l.startswith(("v_accvgpr_write", "v_accvgpr_mov"))]
        assert zero and wait_states(lines[zero[-1] + 1:first]) >= 2, name
        # between the first and the last MFMA nothing else touches an
        # accumulator: the compiler's own copies would not keep the wait
        # states an inline-assembly MFMA's result needs
        for l in lines[first:last]:
            assert l.startswith("v_mfma") or not agpr.search(l), (name, l)
        # and no vector ALU instruction runs there: each one costs the
        # matrix pipe about 14 cycles at one wave per SIMD, so the loop
        # addresses memory from scalar bases
        valu = [l for l in lines[first:last]
                if l.startswith("v_") and not l.startswith(("v_mfma", "v_accvgpr"))]
        assert not valu, (name, valu[:3])
        # the first instruction after the last MFMA that touches an AGPR
        # (v_accvgpr_read, or a store straight from the accumulators)
        uses = [i for i, l in enumerate(lines) if i > last and agpr.search(l)]
        assert uses and wait_states(lines[last + 1:uses[0]]) >= need, (name, lines[uses[0]])
        for i in mfma:
            ops = re.findall(r"\bv(\d+)\b", lines[i].split(",", 1)[1])
            for prev in lines[max(0, i - 3):i]:
                m = re.match(r"v_\w+\s+v(\d+)\b", prev)
                if prev.startswith("v_") and not prev.startswith(("v_mfma", "v_accvgpr")) and m:
                    assert m.group(1) not in ops, (name, prev, lines[i])
    assert found >= 2, "expected the large wave-tile kernel instances"


# kernels that reuse an LDS stage, by source: each instance of each must
# carry the poison in the debug build
STAGED = {"sgemm_mfma.hip": ["sgemm_mfma_kernel", "sgemm_mfma_dma_kernel", "sgemm_mfma_big_kernel"],
          "sgemm_lowp.hip": ["gemm_lowp_kernel", "gemm_lowp_big_kernel"],
          "sgemm_valu.hip": ["sgemm_valu_kernel"],
          "sgemm_skinny.hip": ["skinny_n_lds_kernel", "skinny_n_vec_kernel", "skinny_m16_kernel",
                               "skinny_m_split_kernel"],
          "sgemm_micro.hip": ["micro4x4_kernel"]}


@pytest.mark.parametrize("name", list(STAGED))
def test_ldspoison_build_poisons_every_staged_kernel(name, tmp_path, request):
    if name in ("sgemm_mfma.hip", "sgemm_lowp.hip"):
        asm = request.getfixturevalue("big_asm")
        release, poison = asm[name], asm[name + POISON]
    else:
        src = os.path.join(CSRC, name)
        release, poison = asm_of(src, tmp_path), asm_of(src, tmp_path, POISON)
    nan = "0x7fc00000"   # the quiet NaN the poison writes
    assert nan not in release
    for family in STAGED[name]:
        found = list(functions(poison, r"_Z\w*\d" + family + r"\w*"))
        assert found, family
        for fn, lines in found:
            assert any(nan in l for l in lines), fn
            assert any(l.startswith("ds_write_b32") for l in lines), fn
