"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The fp64 oracle (C, gcc) built with -fsanitize=address,undefined runs
  every oracle pin.
- The C-ABI library built with the sanitizers on its host code only (device
  code is untouched) runs the argument-validation tests, which exercise
  every host-side error path without a GPU.

Each run happens in a subprocess with the sanitizer runtime preloaded and
halts on the first report.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _pytest(files, env):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           *files], env=env, capture_output=True, text=True, cwd=ROOT,
                          timeout=600)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-o", str(so),
                    os.path.join(ROOT, "oracle", "gdn_oracle.c"),
                    os.path.join(ROOT, "oracle", "fork_attention_oracle.c"), "-lm"], check=True)
    env = dict(ENV, LD_PRELOAD=f"{asan}:{ubsan}", ORACLE_LIB_OVERRIDE=str(so))
    r = _pytest([os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                 os.path.join(ROOT, "tests", "test_attention_oracle_pins.py")], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rt:
        pytest.skip("hipcc or the clang sanitizer runtime not installed")
    from linear_attention_recurrent_gdn_amd import build as b

    csrc = os.path.join(ROOT, "linear_attention_recurrent_gdn_amd", "csrc")
    # host-side sanitizers only: each -fsanitize= applies to the host pass
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in b.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(csrc, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        cmd = [hipcc, *flags, *b.FILE_FLAGS.get(os.path.basename(src), []), *san, "-c", src,
               "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err.decode()[-3000:]
    so = str(tmp_path / "libgdn_san.so")
    subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *san[:4],
                    "-shared-libsan", "-o", so, *objs], check=True, capture_output=True)
    env = dict(ENV, LD_PRELOAD=rt[-1], GDN_LIB_OVERRIDE=so)
    r = _pytest([os.path.join(ROOT, "tests", "test_abi.py")], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
