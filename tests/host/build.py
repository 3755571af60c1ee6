"""Builds the host harness (tests/host/harness.cpp): the library's C ABI and
its row, LM-head and recorder kernels compiled for the CPU against the emulated device
environment in tests/host/hip, with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only: no GPU code is built here).

    python tests/host/build.py [OUTDIR]     (default: _build/host)

Prints the path of the harness executable.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "off_policy_logit_amd", "csrc")
sys.path.insert(0, HERE)
import xform  # noqa: E402


def compiler():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cxx = os.path.join(rocm, "llvm", "bin", "clang++")
    return cxx if os.path.exists(cxx) else "clang++"


FLAGS = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-Wno-unused-command-line-argument",
         "-I", HERE, "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(out_dir=None):
    out_dir = out_dir or os.path.join(ROOT, "_build", "host")
    os.makedirs(out_dir, exist_ok=True)
    units = []
    for name in ("sc_kernels.hip", "sc_lmhead.hip", "sc_record.hip"):
        dst = os.path.join(out_dir, name.replace(".hip", "_host.cpp"))
        with open(os.path.join(CSRC, name)) as f:
            text = xform.transform(f.read())
        with open(dst, "w") as f:
            f.write(text)
        units.append(dst)
    units += [os.path.join(CSRC, "sc_api.cpp"), os.path.join(HERE, "emu.cpp"),
              os.path.join(HERE, "harness.cpp")]
    objs = []
    procs = []
    for u in units:
        obj = os.path.join(out_dir, os.path.basename(u) + ".o")
        cmd = [compiler(), *FLAGS, "-x", "c++", "-c", u, "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                       text=True), cmd))
        objs.append(obj)
    for p, cmd in procs:
        out, _ = p.communicate()
        if p.returncode:
            raise RuntimeError(f"{' '.join(cmd)}\n{out}")
    exe = os.path.join(out_dir, "harness")
    subprocess.run([compiler(), "-fsanitize=address,undefined", *objs, "-o", exe], check=True)
    return exe


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else None))
