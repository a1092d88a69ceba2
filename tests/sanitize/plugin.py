"""pytest plugin for the sanitizer run (loaded with -p): points the C ABI
binding and the oracle at their sanitizer builds before any test runs."""
import os

import oracle
import quantized_diffusion_amd as qd

qd.LIB_PATH = os.environ["QD_SANITIZED_LIB"]
qd._lib = None
oracle._default = oracle.Oracle(os.environ["ORACLE_SANITIZED_LIB"])
