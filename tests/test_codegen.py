"""Checks on the gfx950 code the build produced (CPU only: no kernel runs).

A buffer access whose resource the compiler cannot prove uniform over the wave
is wrapped in a loop over the distinct resources (readfirstlane, compare,
exec mask, the access, exec restore, branch back).  Such loops cost
instructions around every load and stop the compiler from counting the loads
in flight, so a wave waits for all of them: the kernels keep every buffer
resource in scalar registers, and this test reads the disassembly of the built
library to keep it so.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gqa_decode_attention_amd", "libasr_attn.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _disassembly(tmp_path):
    fat = tmp_path / "fatbin"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fat}", LIB], check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    text = []
    for k in range(len(starts) - 1):
        part, obj = tmp_path / f"b{k}", tmp_path / f"co{k}.o"
        part.write_bytes(data[starts[k]:starts[k + 1]])
        subprocess.run([TOOLS[1], "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--input={part}", f"--output={obj}"], check=True, capture_output=True)
        if obj.stat().st_size == 0:
            continue
        text.append(subprocess.run([TOOLS[2], "-d", "--mcpu=gfx950", str(obj)], check=True, capture_output=True,
                                   text=True).stdout)
    return "\n".join(text)


def waterfall_sites(disassembly):
    """(function, instruction) of every buffer access inside a loop over resources."""
    func, sites, ops = "?", [], []
    for line in disassembly.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line.strip())
        if m:
            func, ops = m.group(1), []
            continue
        ins = line.strip().split("//")[0].strip()
        if not ins or ins.endswith(":"):
            continue
        ops.append(ins)
        if (len(ops) >= 3 and ops[-1].startswith("s_cbranch_execnz") and ops[-2].startswith("s_xor_b64 exec, exec")
                and ops[-3].startswith("buffer_")):
            sites.append((func, ops[-3]))
    return sites


def test_waterfall_detector_finds_the_pattern():
    # the shape the compiler emits for a buffer load with a resource in vector registers
    text = """0000000000001000 <k>:
	v_readfirstlane_b32 s16, v34
	v_cmp_eq_u64_e32 vcc, s[16:17], v[34:35]
	s_and_saveexec_b64 s[0:1], vcc
	buffer_load_dwordx4 v[36:39], v61, s[16:19], 0 offen
	s_xor_b64 exec, exec, s[0:1]
	s_cbranch_execnz 65530
	buffer_load_dwordx4 v[40:43], v61, s[20:23], 0 offen
	s_waitcnt vmcnt(0)
"""
    assert waterfall_sites(text) == [("k", "buffer_load_dwordx4 v[36:39], v61, s[16:19], 0 offen")]


@pytest.mark.skipif(not os.path.exists(LIB), reason="the HIP library is not built")
@pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools not found")
def test_no_buffer_access_loops_over_resources(tmp_path):
    text = _disassembly(tmp_path)
    assert "k_attn_vmfma" in text and "k_attn_waves" in text, "kernels missing from the disassembly"
    sites = waterfall_sites(text)
    funcs = sorted({f for f, _ in sites})
    assert not sites, f"{len(sites)} buffer accesses in loops over resources, in: {funcs[:8]}"
