"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each loaded by a child process with its sanitizer runtime
preloaded (the Python interpreter itself is not instrumented):
  * the FP64 oracle built by gcc with -fsanitize=address,undefined, running
    its pins (tests/test_oracle_pins.py, tests/test_oracle_mixer.py);
  * the C ABI's argument checking (gdn2_api.cpp) built by hipcc with the
    host-only sanitizers and linked with the regular kernel objects, running
    the ABI tests (tests/test_abi_cpu.py), which call every entry point with
    bad and good arguments but launch nothing.
A sanitizer report aborts the child; its log files must stay absent."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, tests, tmp):
    env = dict(os.environ)
    env.update(env_extra)
    log = os.path.join(tmp, "san")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:abort_on_error=1:log_path={log}.asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}.ubsan"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = sorted(glob.glob(log + ".*"))
    text = "".join(open(p).read()[:4000] for p in reports)
    assert r.returncode == 0 and not reports, f"rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-2000:]}\n{text}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    from oracle import build as ob

    lib = ob.compile_oracle(out=str(tmp_path / "liboracle_asan.so"),
                            extra_flags=["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                         "-fno-omit-frame-pointer"])
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    assert os.path.isabs(libasan), "gcc's AddressSanitizer runtime is not installed"
    out = _run({"GDN2_ORACLE_LIB": lib, "LD_PRELOAD": libasan},
               ["tests/test_oracle_pins.py", "tests/test_oracle_mixer.py"], str(tmp_path))
    assert "passed" in out


def test_c_abi_checks_under_sanitizers(tmp_path):
    from delta_rule_linear_gdn2_amd import build as lb

    lib = lb.build_sanitized(str(tmp_path))
    rt = lb.sanitizer_runtime_dir()
    runtime = os.path.join(rt, lb.SAN_RUNTIME)
    if not os.path.exists(runtime):
        pytest.fail(f"{runtime} missing")
    out = _run({"GDN2_LIBRARY": lib, "LD_PRELOAD": runtime,
                "LD_LIBRARY_PATH": rt + os.pathsep + os.environ.get("LD_LIBRARY_PATH", "")},
               ["tests/test_abi_cpu.py"], str(tmp_path))
    assert "passed" in out
