"""Where the in-tree build puts the shared library."""
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_NAME = "libmoe_finalize.so"
LIB_PATH = os.path.join(LIB_DIR, LIB_NAME)
PROBE_LIB_NAME = "libmoe_bandwidth_probes.so"
PROBE_LIB_PATH = os.path.join(LIB_DIR, PROBE_LIB_NAME)
