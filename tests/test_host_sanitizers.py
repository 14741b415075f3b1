"""Failure-path evidence on the CPU, under sanitizers.

- tests/host_models/protocol_model.cpp: a thread-per-workgroup model of the
  layer kernel's grid barrier, ticket hand-out and per-slot completion counters
  (the same counting rules as the kernel), built with ThreadSanitizer: every
  unit processed once, no value read before it was written, a missing arrival
  turned into a fault that releases everyone, no data race reported.
- tests/host_models/oracle_sanitize_driver.c: every oracle and host-generator
  entry point, in every storage format, built with AddressSanitizer and
  UndefinedBehaviorSanitizer.
- tests/host_models/abi_sanitize_driver.cpp: the C ABI's host code (mk_api.cpp)
  built with AddressSanitizer and UndefinedBehaviorSanitizer for the host pass,
  driven through its checks and error paths without a GPU.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODELS = os.path.join(ROOT, "tests", "host_models")
CSRC = os.path.join(ROOT, "decoder_megakernel_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _build(cmd):
    rc, out = _run(cmd)
    assert rc == 0, "build failed: %s\n%s" % (" ".join(cmd), out[-3000:])


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_protocol_model_under_thread_sanitizer(tmp_path):
    exe = str(tmp_path / "protocol_model")
    _build(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
            os.path.join(MODELS, "protocol_model.cpp"), "-o", exe])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    rc, out = _run([exe], env=env)
    print(out[-2000:])
    assert rc == 0, out[-4000:]
    assert "all protocol checks passed" in out
    assert "ThreadSanitizer" not in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_and_generator_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all", os.path.join(MODELS, "oracle_sanitize_driver.c"),
            os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth_host.c"),
            "-fopenmp", "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2")
    rc, out = _run([exe], env=env)
    print(out[-2000:])
    assert rc == 0, out[-4000:]
    assert "all calls clean" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    # the device units as the library build leaves them (every source but the host-side API)
    spec = importlib.util.spec_from_file_location("_mk_build", os.path.join(ROOT, "decoder_megakernel_amd", "_build.py"))
    bld = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bld)
    objs = [os.path.join(CSRC, os.path.splitext(n)[0] + ".o") for n in bld.SOURCES if n != "mk_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's kernel objects are not built (run __graft_entry__.build())")
    # sanitizers for the host pass only (the kernels are not instrumented)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    api = str(tmp_path / "mk_api_san.o")
    drv = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_driver")
    _build([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip", "-c",
            os.path.join(CSRC, "mk_api.cpp"), "-o", api, "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san)
    _build([HIPCC, "-O1", "-g", "-std=c++17", "-c", os.path.join(MODELS, "abi_sanitize_driver.cpp"), "-o", drv]
           + san)
    _build([HIPCC, "--offload-arch=gfx950", drv, api] + objs + ["-o", exe] + san)
    # the HIP runtime's own allocations at exit are not this library's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out = _run([exe], env=env)
    print(out[-2000:])
    assert rc == 0, out[-4000:]
    assert "all calls clean" in out
