"""Split-KV (flash-decoding) single-query decode attention for MI355X.

The compute path is the HIP library libfd.so (C ABI, see include/fd.h);
`split_kv_fd_amd.fd` is its thin ctypes binding and `split_kv_fd_amd.decode`
a torch-facing convenience on top of it.  Nothing here falls back to a CPU
implementation: without the built library, the calls raise.
"""
