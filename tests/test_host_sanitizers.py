"""The pool's host bookkeeping (pool.cpp) under AddressSanitizer +
UndefinedBehaviorSanitizer and under ThreadSanitizer: 600 random operations
per seed against a contiguous model with every invariant checked after each,
and four threads driving one pool at once (paged_kv_speculative_amd/csrc/
host_check).  Host code only; built with g++."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_pool_bookkeeping_under_sanitizers():
    path = os.path.join(ROOT, "paged_kv_speculative_amd", "csrc", "host_check", "run.py")
    spec = importlib.util.spec_from_file_location("_pkv_host_check", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    out = m.run(ops=600)
    for name, text in out.items():
        assert "all checks passed" in text, (name, text)
        assert "copy-on-write copies" in text
