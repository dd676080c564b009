"""Activation-sparse gated FFN forward for MI355X (gfx950).

The compute path is a HIP library behind a C ABI (``include/sffn.h``); the
``sffn`` submodule is its Python binding. Importing this package loads
nothing: ``inputs`` (seeded synthetic data) works without a GPU, and the
binding loads the shared library on first use, failing loudly if it is
missing.
"""
