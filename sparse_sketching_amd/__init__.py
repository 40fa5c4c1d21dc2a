"""Sparse randomized sketching (SparseStack, CountSketch, BlockPerm-SJLT)
on AMD MI355X (gfx950)."""
