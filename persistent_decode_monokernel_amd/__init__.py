"""Persistent batch-1 decode monokernel for AMD MI355X (gfx950).

The HIP library (libkie.so, C ABI in include/kie.h) does all the work; this
package holds its ctypes binding (``kie``), the build step (``build``) and the
seeded synthetic-input generators (``synth``).  Nothing is loaded at import.
"""
