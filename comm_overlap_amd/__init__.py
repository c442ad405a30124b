"""Sliced tensor-parallel layer shard for MI355X (gfx950).

The compute path lives in the HIP library libtpslice.so (comm_overlap_amd/csrc); the Python binding
`comm_overlap_amd.tpslice` only marshals tensor pointers and streams into its C ABI.
Import `comm_overlap_amd.tpslice` explicitly: it fails loudly if the library has not been built.
"""
