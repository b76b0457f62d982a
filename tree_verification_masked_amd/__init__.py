"""MI355X-native tree verification for EAGLE-style speculative decoding.

The compute path is the HIP library ``libspectree.so`` (built from ``csrc/``),
reached through the thin ctypes binding in :mod:`.binding`.  Importing the
package does not load the library; the first binding call does, and raises if
the library is missing.  The seeded input generators (test and benchmark support)
live outside the package, in the top-level ``synth`` module.
"""
