"""MI355X-native int4 weight-streaming decode.

The compute path is the HIP library libi4decode.so (built from csrc/ for
gfx950); this package holds its thin ctypes binding (`binding`) and the
closed-form byte/FLOP calculator (`roofline`).  The library is loaded on first
use and loading fails loudly if it has not been built.
"""
