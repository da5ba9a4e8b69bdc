"""Build libmla.so (gfx950) from csrc/ with hipcc, with a register-spill gate.

The gate follows the build rule on page "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds"
(the build fails if any kernel spills): every kernel's resource report must show zero scratch memory
and no spilled VGPRs, unless MLA_SKIP_REG_SPILL_CHECK=1 is set. SGPR spills are reported but allowed
while scratch stays at zero: on gfx950 they go to spare VGPR lanes (v_writelane / v_readlane) and
never reach memory. The per-kernel report is written to _build/kernel_resources.txt.

Sources whose kernels contain MFMAs written as inline assembly are also compiled to device
assembly and checked for the wait states gfx950 requires around those MFMAs, and for
compiler-generated uses of m0, which the kernels' LDS copies leave set (asm_check.py); the build
fails on any violation.

Usage: python -m sparse_mla_decode_get_amd.build   (or build() from Python)
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["mla_decode.hip", "mla_decode_wide.hip", "mla_decode_h64.hip", "mla_sched.hip", "mla_combine.hip", "mla_aux.hip",
           "mla_noalloc.hip", "mla_quant.hip", "mla_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed fp32 arithmetic (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# source -> kernel-name fragment whose assembly is checked by asm_check
ASM_CHECKED = {"mla_decode_wide.hip": "sparse_decode_wide_kernel",
               "mla_decode_h64.hip": "sparse_decode_h64_kernel"}


class SpillError(RuntimeError):
    pass


class HazardError(RuntimeError):
    pass


def _asm_check(src, name_part):
    """Compile `src` to gfx950 device assembly and check its inline-assembly MFMAs' wait states."""
    sys.path.insert(0, PKG)
    import asm_check
    out = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    text = open(out).read()
    names = asm_check.kernels(text, name_part)
    if not names:
        raise HazardError(f"no kernel matching {name_part} in {src}")
    problems = []
    for k in names:
        problems += [f"{k}: {m}" for m in asm_check.check(text, k)]
        problems += [f"{k}: {m}" for m in asm_check.m0_outside_inline_asm(text, k)]
    return problems


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    else:
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
               "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


_FIELDS = ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "Occupancy [waves/SIMD]", "SGPRs Spill",
           "VGPRs Spill", "LDS Size [bytes/block]", "SGPRs")


def _parse_resources(text):
    """kernel name -> {field: int} from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in text.splitlines():
        m = re.search(r"remark: .*Function Name: (\S+)", ln)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        if cur is None:
            continue
        for f in _FIELDS:
            m = re.search(r"remark: .*\s" + re.escape(f) + r": (\d+)", ln)
            if m and f not in out[cur]:
                out[cur][f] = int(m.group(1))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(ASM_CHECKED)) as ex:
        checks = [ex.submit(_asm_check, src, part) for src, part in ASM_CHECKED.items()]
        results = list(ex.map(_compile, SOURCES))
        hazards = [m for c in checks for m in c.result()]
    if hazards:
        raise HazardError("MFMA wait-state violations:\n" + "\n".join(hazards[:20]))
    report = {}
    for _, err in results:
        report.update(_parse_resources(err))
    lines = []
    spills = []
    for name, f in sorted(report.items()):
        lines.append(f"{name}: " + ", ".join(f"{k}={v}" for k, v in f.items()))
        if f.get("ScratchSize [bytes/lane]", 0) > 0 or f.get("VGPRs Spill", 0) > 0:
            spills.append(name)
    with open(os.path.join(BUILD, "kernel_resources.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if verbose:
        print("\n".join(lines))
    if spills and os.environ.get("MLA_SKIP_REG_SPILL_CHECK") != "1":
        raise SpillError("register spill / scratch use in: " + ", ".join(spills) +
                         " (set MLA_SKIP_REG_SPILL_CHECK=1 to build anyway)")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
