"""Run the host-side ABI and binding tests against a library given on the command line
(the ABI layer built with AddressSanitizer on the host side); started by test_abi_asan.py
in a process that preloads the sanitizer runtime."""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import bit_quantized_grouped_amd as bq  # noqa: E402

lib = ctypes.CDLL(sys.argv[1])
for name, (res, args) in bq._SIGNATURES.items():
    fn = getattr(lib, name)
    fn.restype = res
    fn.argtypes = args
bq._lib = lib   # the binding's calls below go to the instrumented library

import pytest  # noqa: E402

sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", os.path.join(HERE, "test_abi_host.py"),
                      os.path.join(HERE, "test_binding_checks.py")]))
