"""Location of the built HIP library (kept apart so that importing the
binding does not import the build script)."""

import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libcausal_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
