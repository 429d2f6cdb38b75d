"""LongNet dilated attention on AMD MI355X (gfx950).

The compute path is the HIP library ``libdla.so`` built from ``csrc/``; the
module ``dla`` is its thin ctypes binding.  ``inputs`` holds the seeded
synthetic workloads.  Importing the package loads nothing native; the binding
loads the library on first use and raises if it is missing.
"""
