"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU):
the library's host code (sa_api.hip) is rebuilt with both sanitizers on the host pass only and
test_abi.py runs against it in a child process with the ASan runtime preloaded.  Any invalid
read, write or undefined behaviour in the validation, workspace carve-out or head-map code
aborts the child and fails this test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_abi_validation_under_host_sanitizers():
    from block_sparse_attention_estimate_amd import build as b
    if not all(os.path.exists(os.path.join(b.OBJ, os.path.splitext(s)[0] + ".o"))
               for s in b.SOURCES):
        b.build()
    lib = b.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=b.asan_runtime(), SA_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the sanitized build (not the product library)
    probe = subprocess.run(
        [sys.executable, "-c",
         "import sys; sys.path.insert(0, %r)\n"
         "from block_sparse_attention_estimate_amd import _lib\n"
         "_lib.load()\n"
         "maps = open('/proc/self/maps').read()\n"
         "assert 'libsa_hostsan.so' in maps and 'asan' in maps\n"
         "print('sanitized library loaded')" % ROOT],
        env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0, probe.stdout + probe.stderr
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         env=env, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "passed" in run.stdout
