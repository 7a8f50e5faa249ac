"""Register, scratch and LDS budgets of the built kernels, read from the code
objects inside libmoe4.so (no GPU needed).

A kernel that spills keeps some values in scratch memory; in the main loops
of the expert GEMMs every reload of such a value must wait for all vector
loads in flight, the buffer-to-LDS prefetches of later k-tiles included, so a
spill silently turns the three-stage LDS ring into a shallower one. These
tests hold every kernel of the library to zero scratch bytes, and the tiled
GEMMs to the budget of two waves per SIMD (256 registers) and one workgroup's
LDS (160 KiB)."""
import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "bit_mixture_experts_amd", "libmoe4.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _kernels(tmp_path):
    """Metadata of every kernel: {name: {field: int}} over all device objects."""
    for tool in ("objcopy", f"{LLVM}/clang-offload-bundler", f"{LLVM}/llvm-readelf"):
        if shutil.which(tool) is None:
            pytest.skip(f"{tool} not found")
    if not os.path.exists(LIB):
        pytest.fail("libmoe4.so is not built (run __graft_entry__.build())")
    fat = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fat}", LIB, str(tmp_path / "x.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    out = {}
    for i, s in enumerate(starts):
        e = starts[i + 1] if i + 1 < len(starts) else len(data)
        b, co = tmp_path / f"b{i}.bin", tmp_path / f"c{i}.elf"
        b.write_bytes(data[s:e])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={b}",
                        f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        # one metadata map per kernel: split at each ".name:" entry's block
        for blk in re.split(r"\n\s+- \.agpr_count:", notes)[1:]:
            name = re.search(r"^\s+\.name:\s+(\S+)", blk, re.M)
            if not name:
                continue
            fields = {"agpr_count": int(blk.split("\n", 1)[0].strip() or 0)}
            for key in ("private_segment_fixed_size", "group_segment_fixed_size", "vgpr_count",
                        "vgpr_spill_count", "sgpr_spill_count"):
                m = re.search(rf"^\s+\.{key}:\s+(\d+)", blk, re.M)
                if m:
                    fields[key] = int(m.group(1))
            out[name.group(1)] = fields
    return out


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    return _kernels(tmp_path_factory.mktemp("co"))


def test_every_kernel_is_read(kernels):
    # the expert GEMMs of both families in every format, routing and the codecs
    names = " ".join(kernels)
    for part in ("k_tiled", "k_skinny", "k_dgrad", "k_route", "k_combine", "k_quantize_nf4"):
        assert part in names, f"no {part} kernel found in the code objects"
    assert len(kernels) >= 50


def test_no_kernel_uses_scratch(kernels):
    # (scalar spills go to lanes of vector registers, not to memory)
    spilled = {n: f for n, f in kernels.items()
               if f.get("private_segment_fixed_size", 0) or f.get("vgpr_spill_count", 0)}
    assert not spilled, "kernels with scratch or spills: " + ", ".join(
        f"{n} {f}" for n, f in spilled.items())


WATERFALL = re.compile(r"v_cmp_eq_u64_e(?:32|64) \S+, s\[\d+:\d+\], v\[\d+:\d+\]")


def test_no_buffer_resource_in_vector_registers(tmp_path):
    # A buffer resource the compiler cannot prove wave-uniform lives in vector
    # registers, and every access through it becomes a loop over its distinct
    # values (read one lane's resource, compare it with every lane's, run the
    # access for the matching lanes, repeat): correct, and many times slower.
    # Its mark is a 64-bit compare of a scalar pair with a vector pair.
    objdump = f"{LLVM}/llvm-objdump"
    if shutil.which(objdump) is None:
        pytest.skip("llvm-objdump not found")
    _kernels(tmp_path)   # unbundles the code objects into tmp_path
    hits = {}
    for co in sorted(tmp_path.glob("c*.elf")):
        text = subprocess.run([objdump, "-d", "--no-show-raw-insn", str(co)], check=True,
                              capture_output=True, text=True).stdout
        name = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
            if m:
                name = m.group(1)
            elif WATERFALL.search(line):
                hits[name] = hits.get(name, 0) + 1
    assert not hits, f"per-lane resource loops in: {hits}"


def test_tiled_gemms_fit_two_waves_per_simd_and_the_lds(kernels):
    tiled = {n: f for n, f in kernels.items() if "k_tiled" in n}
    assert len(tiled) >= 9   # three formats x (gate_up, gate_up gathered, down)
    for n, f in tiled.items():
        assert f["vgpr_count"] + f["agpr_count"] <= 256, (n, f)
        # static LDS (tables); the stage ring is dynamic and checked at launch
        assert f["group_segment_fixed_size"] <= 160 * 1024, (n, f)
