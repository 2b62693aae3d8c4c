"""Resource use of the compiled kernels (CPU: hipcc -S for gfx950).

The HIP sources are compiled to gfx950 assembly here, with the library's own
flags, and every kernel's descriptor and code are read back:

* LDS: the static group segment fits the 160 KB of a compute unit.
* Registers: no kernel touches scratch memory inside a loop.  Spilled values
  reloaded on every tile step would put memory round trips on the hot path;
  a kernel at the register limit of its launch bounds may spill a few set-up
  values outside its loops.
* The private segment (spills and stack) stays below a small bound.
* Every kernel the launchers name is present: keys, rows and combine
  kernels at head_dim 64, 96 and 128 and the append kernel.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "self_speculative_verify_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or (
    "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc"))
LDS_BYTES = 160 * 1024
PRIVATE_MAX = 128            # bytes per lane

pytestmark = pytest.mark.skipif(not HIPCC, reason="hipcc not available")

LABEL = re.compile(r"^(\.LBB\d+_\d+|; %bb\.\d+):(.*)$")


def _flags():
    from self_speculative_verify_amd import _build
    skip = {"-shared", "-fPIC", "-Wall", "-Wno-unused-function"}
    return [f for f in _build.HIPCC_FLAGS if f not in skip]


def _compile(src: str, out: str) -> str:
    cmd = [HIPCC, *_flags(), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


def parse(asm: str) -> dict:
    """kernel name -> lds, vgpr, private bytes, scratch instructions (all,
    and those in blocks the compiler marks as inside a loop)."""
    lines = asm.split("\n")
    kernels = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):\s*;\s*@", line)
        if not m:
            continue
        name = m.group(1)
        in_loop = False
        scratch = scratch_loop = 0
        j = i + 1
        while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
            ln = lines[j]
            lab = LABEL.match(ln)
            if lab:
                in_loop = "Loop Header" in lab.group(2) or "in Loop:" in lab.group(2)
            else:
                op = ln.strip().split(" ")[0]
                if op.startswith("scratch_") or (op.startswith("buffer_") and "lds" not in ln):
                    scratch += 1
                    scratch_loop += in_loop
            j += 1
        kernels[name] = {"scratch": scratch, "scratch_in_loops": scratch_loop}
    for name, k in kernels.items():
        def meta(pattern, default=None):
            m = re.search(pattern, asm)
            return int(m.group(1)) if m else default
        esc = re.escape(name)
        k["private"] = meta(r"\.set " + esc + r"\.private_seg_size, (\d+)", 0)
        k["vgpr"] = meta(r"\.set " + esc + r"\.num_vgpr, (\d+)")
        block = re.search(r"\.amdhsa_kernel " + esc + r"\n(.*?)\.end_amdhsa_kernel", asm, re.S)
        assert block, f"no kernel descriptor for {name}"
        k["lds"] = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", block.group(1)).group(1))
    return kernels


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    out = {}
    for src in ("verify_mfma.hip", "append.hip"):
        out.update(parse(_compile(src, str(d / (src + ".s")))))
    return out


def test_parser_on_a_small_listing():
    """The parser finds a spill inside a loop and one outside it."""
    asm = "\n".join([
        "_ZN1k1fEv:  ; @_ZN1k1fEv",
        "  scratch_store_dword off, v1, off",
        ".LBB0_1:                                ; =>This Loop Header: Depth=1",
        "  v_add_f32 v0, v0, v1",
        "; %bb.2:                                ;   in Loop: Header=BB0_1 Depth=1",
        "  scratch_load_dword v2, off, off offset:4",
        ".LBB0_3:",
        "  s_endpgm",
        ".Lfunc_end0:",
        "\t.set _ZN1k1fEv.num_vgpr, 3",
        "\t.set _ZN1k1fEv.private_seg_size, 8",
        "\t.amdhsa_kernel _ZN1k1fEv",
        "\t\t.amdhsa_group_segment_fixed_size 1024",
        "\t.end_amdhsa_kernel",
    ])
    k = parse(asm)["_ZN1k1fEv"]
    assert k == {"scratch": 2, "scratch_in_loops": 1, "private": 8, "vgpr": 3, "lds": 1024}


def test_every_kernel_is_built(kernels):
    names = " ".join(kernels)
    for kind, n in (("k_verify_keys", 15), ("k_verify_rows", 8), ("k_combine", 3), ("k_append", 1)):
        assert sum(kind in k for k in kernels) == n, (kind, names)


def test_lds_fits_a_compute_unit(kernels):
    for name, k in kernels.items():
        assert 0 <= k["lds"] <= LDS_BYTES, (name, k)


def test_no_scratch_inside_loops(kernels):
    for name, k in kernels.items():
        assert k["scratch_in_loops"] == 0, (name, k)


def test_private_segment_small(kernels):
    for name, k in kernels.items():
        assert k["private"] <= PRIVATE_MAX, (name, k)
        assert k["vgpr"] is not None and k["vgpr"] <= 512, (name, k)
