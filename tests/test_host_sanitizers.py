"""The C-ABI front end under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (validation, shape limits, size and workspace arithmetic) is rebuilt by g++ with
both sanitizers and linked with the regular kernel objects; the host ABI tests then run
against that library in a subprocess with the sanitizer runtimes preloaded. Any sanitizer
report aborts that run.
"""
import os
import shutil
import subprocess
import sys

import pytest

from tensor_transformer_layer_rank_amd import build_sanitized as bs

pytestmark = pytest.mark.skipif(not shutil.which("g++") or not bs.runtimes(),
                                reason="g++ with the ASan/UBSan runtimes is not installed")


@pytest.fixture(scope="module")
def san_lib():
    return bs.build()


def test_front_end_is_instrumented(san_lib):
    out = subprocess.run(["nm", "-D", "--undefined-only", san_lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in out or "__asan_report_store" in out
    assert "__ubsan_handle_" in out


def test_sanitizer_runtime_is_active_in_the_test_process(san_lib):
    code = ("import tensor_transformer_layer_rank_amd as tp; L = tp.load(); assert L.tp_abi_version() == 1; "
            "maps = open('/proc/self/maps').read(); print('libasan' in maps, 'libubsan' in maps, tp.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       env=bs.sanitized_env(), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split()[:3] == ["True", "True", san_lib]


def test_host_abi_tests_pass_under_asan_and_ubsan(san_lib):
    r = bs.run_host_tests()
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-5000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-5000:]
