"""Build the CPU bounds emulation of the kernels (host clang++ with
AddressSanitizer) from the current kernel source.  Returns the binary path.

The kernel file is copied with five mechanical rewrites that only the
emulation needs: each `__shared__` array becomes a pointer from emu_lds(),
the raw `s_barrier` becomes emu_barrier(), the empty asm statement that pins
a value in a register is dropped, the AMDGPU-only occupancy attribute is
dropped, and the single hipLaunchKernel call runs the kernel's workgroups on
the host (emu_launch)."""
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "gemm_epilogues_mlp_amd", "csrc")


def clangxx():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    return None


def rewrite(src: str) -> str:
    src = re.sub(r"__shared__\s+__attribute__\(\(aligned\(\d+\)\)\)\s+uint8_t\s+(\w+)\[([^\]]+)\];",
                 r"uint8_t* \1 = ::emu_lds(\2);", src)
    src = re.sub(r"__shared__\s+__attribute__\(\(aligned\(\d+\)\)\)\s+(\w+)\s+(\w+)\[([^\]]+)\];",
                 r"\1* \2 = reinterpret_cast<\1*>(::emu_lds(sizeof(\1) * (\3)));", src)
    src = src.replace('asm volatile("s_barrier" ::: "memory");', "::emu_barrier();")
    # the empty register-pinning statement has no effect on the host
    src = src.replace('asm volatile("" : "+v"(tid));', "(void)tid;")
    src = re.sub(r"__attribute__\(\(amdgpu_waves_per_eu\([^)]*\)\)\)", "", src)
    # the one hipLaunchKernel call (in launch_kernel) runs the kernel on the host
    launch = ("return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, "
              "shm, stream);")
    if src.count(launch) != 1:
        raise RuntimeError("kernel source: expected exactly one hipLaunchKernel call")
    src = src.replace(launch, "(void)argv; emu_launch(k, grid, block, v...); return hipSuccess;")
    if "__shared__" in src or "asm volatile" in src:
        raise RuntimeError("kernel source has a construct the emulation does not rewrite")
    return src


def build(out_dir: str) -> str:
    cc = clangxx()
    if cc is None:
        raise RuntimeError("clang++ not found")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(CSRC, "swiglu_kernels.hip")) as f:
        src = rewrite(f.read())
    with open(os.path.join(out_dir, "swiglu_kernels_emu.cpp"), "w") as f:
        f.write(src)
    for name in ("swiglu_internal.h",):
        shutil.copy(os.path.join(CSRC, name), out_dir)
    for name in ("swiglu_device.hpp", "emu_driver.cpp"):
        shutil.copy(os.path.join(HERE, name), out_dir)
    exe = os.path.join(out_dir, "emu_driver")
    cmd = [cc, "-std=c++20", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
           "-Wno-unknown-attributes", "-Wno-ignored-attributes", "-Wno-psabi", "-I", out_dir, "-I", HERE,
           os.path.join(out_dir, "emu_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


if __name__ == "__main__":
    import sys
    print(build(sys.argv[1] if len(sys.argv) > 1 else "/tmp/swiglu_emu"))
