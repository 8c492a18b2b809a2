"""MI355X-native batched SQP-step linear-algebra core (GATO's form / PCG / merit).

The compute path is the HIP library ``libgato.so`` built from ``csrc/``; its
C ABI is declared in ``include/gato.h``.  ``ops`` is the thin ctypes binding
(argument marshalling only) and ``synth`` draws seeded synthetic inputs.
Importing the package does not load the library; ``ops`` does, and raises if
it is missing.
"""
__all__ = ["ops", "synth"]
