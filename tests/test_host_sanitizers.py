"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds tests/host_fuzz/jl_host_fuzz.cpp against every libjl source, with
both sanitizers on the host pass of hipcc (the GPU code is built as usual and
never runs), and runs the seeded fuzz of jl_validate, the weight-file parser,
jl_serve_plan and the Router rule on a few seeds; the first sanitizer report
or failed check ends the run with an error.
"""
import os
import subprocess

import pytest

from encoder_transformer_amd import build as jl_build
from encoder_transformer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def fuzzer():
    os.makedirs(OUT, exist_ok=True)
    flags = [f for f in jl_build.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    srcs = [os.path.join(jl_build.CSRC, s) for s in jl_build.SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "host_fuzz", "jl_host_fuzz.cpp"))
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        procs.append((src, subprocess.Popen([jl_build.HIPCC] + flags + ["-c", src, "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{src}:\n{out[-3000:]}"
    exe = os.path.join(OUT, "jl_host_fuzz")
    r = subprocess.run([jl_build.HIPCC, f"--offload-arch={jl_build.ARCH}"] + SAN + objs + ["-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    # a JLW1 header with the model's tensors and no data
    hdr, _, _ = synth.weight_file_header([(n, s, 0) for n, s, _ in synth.weight_spec()])
    hpath = os.path.join(OUT, "header.bin")
    with open(hpath, "wb") as f:
        f.write(hdr)
    return exe, hpath


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_under_sanitizers(fuzzer, seed):
    exe, hpath = fuzzer
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, str(seed), "4000", hpath], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=env, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-6000:]
    assert "ok: seed" in r.stdout
