"""Mel-Band RoFormer mask-estimation core on AMD MI355X (gfx950).

The product is the C-ABI library ``libmbr_core.so`` built from ``csrc/``; this package
holds its thin ctypes binding (``binding``), the seeded synthetic workloads
(``synth``) and the algorithmic FLOP / byte model used to report rooflines
(``roofline``).  Importing the package does not load the library; ``binding.lib()``
does, and raises if the library is missing.
"""
