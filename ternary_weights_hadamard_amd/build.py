"""Build libtb.so from csrc/*.hip with hipcc for gfx950 (in-tree).

Usage: python -m ternary_weights_hadamard_amd.build  (or call build()).
Every HIP source is compiled with packed-fp32 instructions disabled and the
objects are linked into ternary_weights_hadamard_amd/libtb.so.

Sources that use the block-scaled matrix instruction are also compiled to
assembly and checked: its destination must not overlap its A or B source
registers.  The instruction reads its sources over several passes and the
compiler does not always keep the destination apart (an overlapping
destination gives wrong sums), so such a build is rejected.
"""

import concurrent.futures
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtb.so")
PROBE_LIB = os.path.join(PKG, "libtb_probe.so")  # measurement probes (include/tb_probe.h)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _filter(stderr):
    # the host pass does not know the gfx950-only feature name; that note is harmless
    return "\n".join(l for l in stderr.splitlines() if "not a recognized feature" not in l)


def _compile(src, objdir):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _filter(r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


_SCALED_MFMA = "v_mfma_scale_f32_16x16x128_f8f6f4"
_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _reg_range(tok):
    m = _REG.match(tok.strip())
    if not m:
        return None
    lo = int(m.group(2) if m.group(2) is not None else m.group(4))
    hi = int(m.group(3) if m.group(3) is not None else m.group(4))
    return m.group(1), lo, hi


def check_scaled_mfma_operands(asm_text, where):
    """Raise if a block-scaled MFMA writes registers it also reads as A or B."""
    n = 0
    for line in asm_text.splitlines():
        line = line.split(";")[0].strip()
        if not line.startswith(_SCALED_MFMA):
            continue
        n += 1
        ops = [o.strip() for o in line[len(_SCALED_MFMA):].split(",")]
        dst, a, b = (_reg_range(o) for o in ops[:3])
        if dst is None:
            raise RuntimeError(f"{where}: cannot parse {line!r}")
        for src in (a, b):
            if src and src[0] == dst[0] and src[1] <= dst[2] and dst[1] <= src[2]:
                raise RuntimeError(f"{where}: scaled MFMA destination overlaps a source: {line!r}")
    return n


def _check_asm(src):
    with open(src) as f:
        if "mfma_scale" not in f.read():
            return 0
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [HIPCC, *CFLAGS, "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{_filter(r.stderr)}")
        with open(out) as f:
            return check_scaled_mfma_operands(f.read(), os.path.basename(src))


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_filter(r.stderr)}")
    # every kernel launched from host code must have its launch stub defined
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the link: " + ", ".join(missing))
    os.replace(tmp, lib)


def build(verbose=True):
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = _sources()
    probes = _sources(os.path.join(CSRC, "probe"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), srcs))
        pobjs = list(ex.map(lambda s: _compile(s, objdir), probes))
        checked = sum(ex.map(_check_asm, srcs))
    _link(objs, LIB)
    _link(pobjs, PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources ({checked} scaled MFMAs checked), {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
