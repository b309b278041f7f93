"""Build the CPU bounds emulation of the kernels (host clang++ with
AddressSanitizer) from the current kernel source.  Returns the binary path.

The kernel file is copied with five mechanical rewrites that only the
emulation needs: each `__shared__` array becomes a pointer from emu_lds(),
the raw `s_barrier` becomes emu_barrier(), the empty asm statement that pins
a value in a register is dropped, the AMDGPU-only occupancy attribute is
dropped, and the single hipLaunchKernel call runs the kernel's workgroups on
the host (emu_launch).  Five planted mistakes, off unless the driver is run
with --plant N, show that the LDS ordering check catches what it exists for."""
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
    src = re.sub(r'asm volatile\(""\s*:\s*"\+v"\((\w+)\)\);', r"(void)\1;", src)
    src = re.sub(r"__attribute__\(\(amdgpu_waves_per_eu\([^)]*\)\)\)", "", src)
    # the one hipLaunchKernel call (in launch_kernel) runs the kernel on the host
    launch = ("return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, "
              "shm, stream);")
    if src.count(launch) != 1:
        raise RuntimeError("kernel source: expected exactly one hipLaunchKernel call")
    src = src.replace(launch, "(void)argv; emu_launch(k, grid, block, v...); return hipSuccess;")
    if "__shared__" in src or "asm volatile" in src:
        raise RuntimeError("kernel source has a construct the emulation does not rewrite")
    return plant_points(src)


# Mistakes the LDS ordering check must catch, planted in the emulation copy
# only and switched on at run time (emu_driver --plant N; 0 = none):
#  1: the LDS-tiled K loop waits for one K step fewer of its DMA
#  2: the epilogues reuse the stage ring without the barrier that ends the K loop
#  3: the persistent kernel ends without draining the loads issued past its last tile
#  4: the FP8 tile in MX mode lets the step before a scale group starts leave
#     that group's scale chunks in flight
#  5: the FP8 tile's K loop waits for one K step fewer of its DMA
#  6: the pair tile's Up waves read SiLU(Gate) without the barrier after the
#     Gate waves' writes
PLANTS = [
    (r"^        wait_vmcnt<\(STAGES - 2\) \* C::LOADS>\(\);$",
     "        if (::g_emu_plant == 1) wait_vmcnt<(STAGES - 1) * C::LOADS>();"
     " else wait_vmcnt<(STAGES - 2) * C::LOADS>();", 1),
    (r"^  wait_vmcnt<0>\(\);\n  __syncthreads\(\);\n(?=  const int h32 = lane >> 5;|  // The lane's epilogue)",
     "  wait_vmcnt<0>();\n  if (::g_emu_plant != 2) __syncthreads();\n", 2),
    (r"^(  // the zero loads issued past the last tile still write LDS\n)  wait_vmcnt<0>\(\);$",
     "\\1  if (::g_emu_plant != 3) wait_vmcnt<0>();", 1),
    (r"^    wait_vmcnt<C::in_flight\(T\)>\(\);$",
     "    if (::g_emu_plant == 4 && C::MX && T == 7) wait_vmcnt<C::in_flight(T) + 1>();"
     " else if (::g_emu_plant == 5) wait_vmcnt<C::in_flight(T) + C::LOADS>();"
     " else wait_vmcnt<C::in_flight(T)>();", 1),
    (r"^    __syncthreads\(\);\n(?=    if \(!gate_wave\) \{)",
     "    if (::g_emu_plant != 6) __syncthreads();\n", 1),
]


def plant_points(src: str) -> str:
    for pattern, repl, count in PLANTS:
        src, n = re.subn(pattern, repl, src, flags=re.M)
        if n != count:
            raise RuntimeError(f"plant point found {n} times, expected {count}: {pattern}")
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
    for name in ("swiglu_device.hpp", "emu_driver.cpp", "emu_race.cpp"):
        shutil.copy(os.path.join(HERE, name), out_dir)
    exe = os.path.join(out_dir, "emu_driver")
    common = [cc, "-std=c++20", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
              "-Wno-unknown-attributes", "-Wno-ignored-attributes", "-Wno-psabi", "-I", out_dir,
              "-I", HERE]
    # the kernels' translation unit reports every load and store (the LDS
    # ordering check); the checker itself is built without that
    race_o = os.path.join(out_dir, "emu_race.o")
    subprocess.run(common + ["-c", os.path.join(out_dir, "emu_race.cpp"), "-o", race_o], check=True)
    subprocess.run(common + ["-fsanitize-coverage=func,trace-loads,trace-stores",
                             os.path.join(out_dir, "emu_driver.cpp"), race_o, "-o", exe], check=True)
    return exe


if __name__ == "__main__":
    import sys
    print(build(sys.argv[1] if len(sys.argv) > 1 else "/tmp/swiglu_emu"))
