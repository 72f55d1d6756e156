"""Ring AllReduce on one MI355X hosting N virtual ranks (HIP, gfx950)."""
