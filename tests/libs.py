"""Build-or-load helpers shared by the tests (no arithmetic of the method)."""
import os

import block_wise_bit_amd as dq4
from block_wise_bit_amd import build as dq4_build


def ensure_hip_library():
    """Load libdq4.so, compiling it first only if nothing is built."""
    if not os.path.exists(dq4.LIBRARY_PATH):
        dq4_build.build()
    return dq4.library()
