"""The host side of the library (checks, selector, workspace bookkeeping,
pack utilities) built under AddressSanitizer and UndefinedBehaviorSanitizer
and driven by the C-ABI tests: the run must be clean (CPU only; the prior
art's defects on the pages were of this class: PR #40977 "RDNA hybrid
W4A16", Review section, a bias indexed out of bounds and an LDS size that
disagreed with the host check)."""
import shutil

import pytest

from weight_only_int4_unpack_amd import sanitize


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++ and its sanitizer runtimes")
def test_host_side_clean_under_asan_and_ubsan():
    assert sanitize.main() == 0
