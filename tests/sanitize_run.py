"""Runs test files against sanitizer builds (a helper of test_sanitizers.py,
started in its own process with the sanitizer runtime preloaded):
    python sanitize_run.py <moe library or -> <oracle library or -> <test file>...
Each library given replaces the one its module would load."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import block_fp8_mixture_router_amd as moe  # noqa: E402
import oracle  # noqa: E402

if sys.argv[1] != "-":
    moe.LIB_PATH = sys.argv[1]
if sys.argv[2] != "-":
    oracle.LIB_PATH = sys.argv[2]
    oracle.SOURCES = []  # never rebuilt over the sanitizer build

import pytest  # noqa: E402

sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + sys.argv[3:]))
