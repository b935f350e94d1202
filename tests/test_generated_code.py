"""The gfx950 code of the built library, read back on the CPU from its own code objects.

- Scratch: no kernel spills inside its K-loop (the innermost loop holding MFMAs), and no kernel
  that the configuration choice can pick uses private memory at all. The 4-wave 256x256 forms (one
  128x128 wave tile per wave: 256 accumulators plus double-buffered fragments, reachable only through
  the configuration override) spill outside their K-loop, and the one with 32-deep K-tiles inside it;
  both are listed here so that any other kernel starting to spill fails.
- M0: in the two-group kernels M0 is written only by the direct global->LDS load sequence written in
  inline assembly (M0 write, one wait state, the load). The compiler does not know that sequence
  leaves a value in M0, so the sequence is only safe while nothing else in the kernel reads or writes
  M0; this checks that the compiler's own code does not, and that every such load has its own M0
  write in front of it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "software_pipelined_tiled_amd", "libsptgemm.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# instructions that read or write M0 without naming it
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_ttracedata|ds_gws_|ds_append|ds_consume|ds_ordered_count|v_movrel|s_movrel|"
                         r"v_interp|ds_read_addtid|ds_write_addtid|global_load_lds|s_set_gpr_idx)")


def check_m0(instructions):
    """Violations of the M0 rule in one function's instructions (mnemonic + operands, in order)."""
    bad = []
    for i, ins in enumerate(instructions):
        op = ins.split()[0]
        if IMPLICIT_M0.match(op):
            bad.append(f"{i}: {ins} uses M0 implicitly")
        elif re.search(r"\bm0\b", ins):
            if not ins.startswith("s_mov_b32 m0,"):
                bad.append(f"{i}: {ins} names M0 outside the load sequence")
            elif i + 2 >= len(instructions) or instructions[i + 1] != "s_nop 0" or not (
                    instructions[i + 2].startswith("buffer_load_dwordx4") and instructions[i + 2].endswith(" lds")):
                bad.append(f"{i}: {ins} is not followed by one wait state and a load to LDS")
        elif op.startswith("buffer_load") and ins.endswith(" lds"):
            if i < 2 or instructions[i - 1] != "s_nop 0" or not instructions[i - 2].startswith("s_mov_b32 m0,"):
                bad.append(f"{i}: {ins} has no M0 write of its own in front of it")
    return bad


def test_m0_checker_flags_each_kind_of_mistake():
    good = ["s_mov_b32 m0, s2", "s_nop 0", "buffer_load_dwordx4 v1, s[8:11], s3 offen lds", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"]
    assert check_m0(good) == []
    assert len(check_m0(good[:1] + good[2:])) == 2                            # wait state missing
    assert len(check_m0(good[2:])) == 1                                       # load without its own M0 write
    assert len(check_m0(good + ["s_add_u32 s5, m0, 4"])) == 1                 # the compiler reading M0
    assert len(check_m0(good + ["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"])) == 1  # implicit use


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not installed")
    return path


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    """The gfx950 ELF of every translation unit in the library's offload section."""
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built")
    objcopy = shutil.which("objcopy")
    if objcopy is None:
        pytest.skip("objcopy not installed")
    bundler = _tool("clang-offload-bundler")
    d = tmp_path_factory.mktemp("code")
    fat = d / "fatbin"
    subprocess.run([objcopy, "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fat)], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in the library"
    elfs = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part = d / f"bundle{n}"
        part.write_bytes(data[a:b])
        out = d / f"bundle{n}.elf"
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}", f"--targets={TARGET}", f"--output={out}"],
                       check=True)
        if out.stat().st_size:
            elfs.append(str(out))
    return elfs


def _kernels(elf):
    """(name, private segment bytes, VGPR spills) of each kernel, from the code object's metadata."""
    text = subprocess.run([_tool("llvm-readelf"), "--notes", elf], check=True, capture_output=True, text=True).stdout
    out, cur = [], {}
    for line in text.splitlines():
        m = re.match(r"\s+\.(name|private_segment_fixed_size|vgpr_spill_count):\s+(\S+)", line)
        if not m:
            continue
        key, val = m.groups()
        if key == "name" and not val.endswith(".kd"):
            cur = {"name": val}
            out.append(cur)
        elif cur:
            cur[key] = val
    return out


def _functions(elf):
    """Each function's instructions as (address, mnemonic and operands, backward-or-forward branch
    target address or None)."""
    text = subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", "--no-show-raw-insn", elf],
                          check=True, capture_output=True, text=True).stdout
    funcs, starts, cur = {}, {}, None
    for line in text.splitlines():
        m = re.match(r"^([0-9a-f]+) <(.+)>:$", line)
        if m:
            starts[m.group(2)] = int(m.group(1), 16)
            cur = funcs.setdefault(m.group(2), [])
            continue
        if cur is None or not line.startswith("\t") or "//" not in line:
            continue
        code, comment = line.split("//", 1)
        ins = " ".join(code.split())
        a = re.match(r"\s*([0-9A-Fa-f]+):", comment)
        if not ins or not a:
            continue
        target = None
        t = re.search(r"<(.+)\+0x([0-9a-f]+)>", comment)
        if ins.startswith(("s_branch", "s_cbranch")) and t and t.group(1) in starts:
            target = starts[t.group(1)] + int(t.group(2), 16)
        cur.append((int(a.group(1), 16), ins, target))
    return funcs


def k_loops(instructions):
    """Address ranges of the innermost loops that hold MFMAs (a backward branch and its target)."""
    loops = [(t, a) for a, _, t in instructions if t is not None and t <= a]
    mfma = [a for a, ins, _ in instructions if ins.startswith("v_mfma")]
    hot = [(s, e) for s, e in loops if any(s <= q <= e for q in mfma)]
    return [(s, e) for s, e in hot if not any((s2, e2) != (s, e) and s <= s2 and e2 <= e for s2, e2 in hot)]


# 4-wave kernels with 256x256 tiles (128x128 wave tiles); they are never chosen, only forced
FOUR_WAVE_256 = "15gemm_dma_kernelILi256ELi256E"
SPILLS_IN_K_LOOP = "15gemm_dma_kernelILi256ELi256ELi32E"  # 32-deep K-tiles


def test_k_loops_found_and_loop_finder_sane():
    ins = [(0, "s_mov_b32 s0, 0", None), (4, "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]", None),
           (8, "s_cbranch_scc1 -3", 0), (12, "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]", None),
           (16, "scratch_load_dword v1, off, off", None), (20, "s_cbranch_scc0 -6", 0)]
    assert k_loops(ins) == [(0, 8)]  # the outer loop holds the inner one: only the inner counts


def test_no_kernel_spills_in_its_k_loop(code_objects):
    checked = 0
    for elf in code_objects:
        for name, ins in _functions(elf).items():
            loops = k_loops(ins)
            if not loops:
                continue
            checked += 1
            inside = [i for a, i, _ in ins if i.startswith("scratch_") and any(s <= a <= e for s, e in loops)]
            if SPILLS_IN_K_LOOP in name:
                assert inside, name  # known: listed above; remove from the list once fixed
            else:
                assert not inside, (name, inside[:4])
    assert checked >= 150, checked


def test_kernels_the_choice_can_pick_use_no_scratch(code_objects):
    kernels = [k for elf in code_objects for k in _kernels(elf)]
    names = [k["name"] for k in kernels]
    assert any("gemm_pp_kernel" in n for n in names) and any("gemm_dma_kernel" in n for n in names), names[:5]
    for k in kernels:
        if FOUR_WAVE_256 in k["name"]:
            continue
        assert k.get("private_segment_fixed_size") == "0", k
        assert k.get("vgpr_spill_count", "0") == "0", k


def test_two_group_kernels_use_m0_only_for_their_loads(code_objects):
    checked = 0
    for elf in code_objects:
        for name, ins in _functions(elf).items():
            if "gemm_pp_kernel" not in name:
                continue
            text = [i for _, i, _ in ins]
            assert any(i.endswith(" lds") for i in text), name
            assert check_m0(text) == [], (name, check_m0(text)[:5])
            checked += 1
    assert checked == 9 * 2, checked  # three kernel forms x three output types x two input types
