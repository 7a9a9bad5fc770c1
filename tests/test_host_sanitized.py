"""The C-ABI host layer (spec_api.hip) built for the CPU under
AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers replaced by host
stand-ins that clear every array carved from the caller's workspace (tests/native/).  Every entry
point runs over the workloads' shapes on both paths and with invalid arguments: a carved array
reaching past the reported workspace size, an out-of-range write or an arithmetic overflow in the
sizing aborts the run.  No GPU and no kernel are involved."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "lossless_draft_verification_row_amd", "csrc")
SANITIZE = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all".split()


def test_host_layer_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    assert os.path.exists(hipcc), "hipcc is needed to build the host layer"
    exe = str(tmp_path / "host_abi_check")
    cmd = [hipcc, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *SANITIZE,
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{os.path.join(HERE, 'native')}",
           "--cuda-host-only", "-x", "hip",
           os.path.join(CSRC, "spec_api.hip"),
           os.path.join(HERE, "native", "host_stubs.cpp"), os.path.join(HERE, "native", "host_abi_check.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
