"""Build the plain-C consumer of libzero_shard.so (test code)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "zs_c_consumer")
PKG = os.path.join(ROOT, "fsdp_sharded_optimizer_zero_amd")
ORACLE = os.path.join(ROOT, "oracle")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ORACLE, "-I", "/opt/rocm/include",
           os.path.join(HERE, "zs_c_consumer.c"), "-o", BIN + ".tmp",
           "-L", PKG, "-lzero_shard", "-L", ORACLE, "-lzs_oracle",
           "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ORACLE}", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
