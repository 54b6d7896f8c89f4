"""CPU oracle for lane-interleaved length-limited Huffman coding and the GEMV
over it.  Test infrastructure only: see oracle.c and oracle.py."""
from .oracle import *  # noqa: F401,F403
from .oracle import build, lib  # noqa: F401
