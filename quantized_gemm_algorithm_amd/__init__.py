"""MiX (Micro-Inverted-Scaling) hot path on MI355X: Python binding over the HIP C-ABI library."""
