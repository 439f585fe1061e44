"""The built gfx950 code objects (no GPU): read the kernel metadata of libgdn.so
and check that no kernel spills registers to scratch memory and that the prep
kernel of the headline shape and the bf16 attention kernel keep the register
budgets their launch sizes assume.  Uses ROCm's LLVM tools on this library's own build."""
import os
import re
import subprocess
import textwrap

import pytest
import yaml

LLVM = "/opt/rocm/llvm/bin"
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "linear_attention_recurrence_03_amd", "libgdn.so")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.access(path, os.X_OK):
        pytest.skip("%s not installed" % path)
    return path


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    """{kernel symbol: {metadata key: int}} over every gfx950 code object."""
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built")
    tmp = tmp_path_factory.mktemp("codeobj")
    fat = tmp / "fat.bin"
    subprocess.run([_tool("llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin", LIB,
                    str(fat)], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundles in .hip_fatbin"
    out = {}
    for i, a in enumerate(starts):
        b = starts[i + 1] if i + 1 < len(starts) else len(data)
        bundle, co = tmp / ("b%d.bin" % i), tmp / ("co%d.o" % i)
        bundle.write_bytes(data[a:b])
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                        "--input=" + str(bundle), "--targets=" + TARGET, "--output=" + str(co)],
                       check=True)
        notes = subprocess.run([_tool("llvm-readelf"), "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        # the AMDGPU metadata note is a YAML document ("---" ... "...")
        y0 = notes.rindex("\n", 0, notes.index("---")) + 1
        y1 = notes.index("\n...", y0)
        body = textwrap.dedent(notes[y0:y1]).replace("---", "", 1)
        doc = yaml.safe_load(body)
        for k in doc["amdhsa.kernels"]:
            out[k[".name"]] = {key[1:]: v for key, v in k.items() if isinstance(v, int)}
    return out


def test_every_kernel_is_found(kernels):
    names = " ".join(kernels)
    for k in ("chunk_prep_kernel", "chunk_scan_kernel", "chunk_lag_kernel", "recurrent_kernel",
              "attn_split_mma_kernel", "attn_combine_kernel"):
        assert k in names, k


def test_no_register_spills(kernels):
    bad = {n: (m.get("private_segment_fixed_size"), m.get("vgpr_spill_count"),
               m.get("sgpr_spill_count"))
           for n, m in kernels.items()
           if m.get("private_segment_fixed_size", 0) or m.get("vgpr_spill_count", 0)
           or m.get("sgpr_spill_count", 0)}
    assert not bad, bad


def _waves_per_simd(m):
    # unified register file: 512 registers per lane and SIMD, allocated in
    # granules of 8; accumulation registers follow the vector registers
    total = (m["vgpr_count"] + 3) // 4 * 4 + m.get("agpr_count", 0)
    total = (total + 7) // 8 * 8
    return min(8, 512 // total)


def test_attention_register_budget(kernels):
    """The bf16 decode attention kernel at d=128 keeps four workgroups per CU (the
    cache ranges are sized for one round of them)."""
    att = [m for n, m in kernels.items() if "attn_split_mma_kernelILi128E" in n]
    assert len(att) == 1, sorted(kernels)
    assert _waves_per_simd(att[0]) >= 4, att[0]


def test_prep_register_budget(kernels):
    """bf16 rows of 128 (the headline prefill): five prep workgroups per CU, one wave
    per SIMD each (also the variant that leaves P to the whole-head pass); the lag
    form's prep, which also forms the cross-chunk matrices, three (two when the op
    normalises q and k)."""
    prep = {n: m for n, m in kernels.items() if "chunk_prep_kernelILi128ELb1E" in n}
    assert len(prep) == 5, sorted(kernels)
    for n, m in prep.items():
        # template arguments after <128, true>: NORM, LAG, PQ
        norm, lag = (n.split("chunk_prep_kernelILi128ELb1E")[1][i] == "1" for i in (2, 6))
        want = (2 if norm else 3) if lag else 5
        assert _waves_per_simd(m) >= want, (n, m, want)


def test_lag_scan_register_budget(kernels):
    """The lag scan keeps two register sets of operands and runs two waves per SIMD
    (one workgroup of five waves per CU), for every width."""
    lag = {n: m for n, m in kernels.items() if "chunk_lag_kernel" in n}
    assert len(lag) == 4, sorted(kernels)
    for n, m in lag.items():
        assert _waves_per_simd(m) >= 2, (n, m)


def test_head_scan_register_budget(kernels):
    """The whole-head pass keeps every value in vector registers (no copies to and
    from accumulation registers) at two or more waves per SIMD, for every width."""
    head = {n: m for n, m in kernels.items() if "chunk_head_kernel" in n}
    assert len(head) == 8, sorted(kernels)
    for n, m in head.items():
        assert m.get("agpr_count", 0) == 0 and _waves_per_simd(m) >= 2, (n, m)
