"""Echo error-compensated low-bit all-reduce, one GPU's share, for AMD Instinct gfx950."""
