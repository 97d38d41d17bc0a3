"""Build libattn.so in-tree with hipcc for gfx950.

    python -m exact_tiled_self_amd.build          # build (always recompiles)
    python -m exact_tiled_self_amd.build --sanitize   # libattn_san.so: host code
                                                      # under ASan + UBSan

The library is written to exact_tiled_self_amd/libattn.so via a temporary
file and an atomic rename, so a process that already loaded the old file is
unaffected.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SAN_LIB_PATH = os.path.join(PKG, "libattn_san.so")

SOURCES = ["api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_paged.hip", "prefill_paged.hip",
           "kv_append.hip", "backward_bf16.hip", "fusion.hip"]

# Device-code flags: gfx950 only; packed fp32 instructions disabled.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]

# Per-source additions.  The bf16 prefill kernels never produce or consume a
# NaN in arithmetic (masked scores are -inf; the paged one writes its NaN
# results as bit patterns), so maxima need no NaN canonicalisation.
EXTRA_FLAGS = {
    "prefill_bf16.hip": ["-fno-honor-nans"],
    "prefill_paged.hip": ["-fno-honor-nans"],
    "backward_bf16.hip": ["-fno-honor-nans"],
    # matrix-core accumulators in ordinary VGPRs: the decode loop rescales
    # them every block, which in AGPRs costs a read and a write per element
    "decode_paged.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


# Host-only sanitizer build of the C ABI layer (argument checking, error
# strings, architecture cache).  Every -fsanitize flag is bound to the host
# pass; api.cpp holds no device code, and the kernels are built as usual.
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-shared-libsan",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_SOURCES = {"api.cpp"}


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime, which a process that
    loads the sanitized library must preload."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not out or not os.path.isabs(out) or not os.path.exists(out):
        import glob
        hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not hits:
            raise RuntimeError("no shared AddressSanitizer runtime found")
        out = hits[-1]
    return out


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str | None = None, sanitize: bool = False) -> str:
    """Compile every source (in parallel, each with its own flags), link
    them into `out` and return its path.  With `sanitize`, the host-side ABI
    layer is built under AddressSanitizer and UndefinedBehaviorSanitizer into
    libattn_san.so (by default)."""
    if out is None:
        out = SAN_LIB_PATH if sanitize else LIB_PATH
    from concurrent.futures import ThreadPoolExecutor

    noise = "is not a recognized feature for this target"   # hipcc host-pass noise
    tmpdir = tempfile.mkdtemp(prefix=".attn_build.", dir=os.path.dirname(out))
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, src + ".o")
            san = SAN_FLAGS if sanitize and src in SAN_SOURCES else []
            cmd = [hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *san, "-I", INCLUDE, "-I", CSRC,
                   "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            proc = subprocess.run(cmd, capture_output=True, text=True)
            msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
            return src, obj, proc.returncode, msgs

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(compile_one, SOURCES))
        errors = [f"{src}:\n" + "\n".join(msgs) for src, _, rc, msgs in results if rc != 0]
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        if verbose:
            for src, _, _, msgs in results:
                if msgs:
                    print("\n".join(msgs))
        fd, tmp = tempfile.mkstemp(prefix=".libattn.", suffix=".so.tmp", dir=os.path.dirname(out))
        os.close(fd)
        cmd = [hipcc(), *HIP_FLAGS, *(SAN_FLAGS if sanitize else []), "-shared", "-o", tmp,
               *[obj for _, obj, _, _ in results]]
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            os.unlink(tmp)
            raise RuntimeError("link failed:\n" + proc.stdout + proc.stderr)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
    print(path)
