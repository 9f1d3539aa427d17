"""MI355X-native partial channel-reduce: row-parallel GEMM + partial channel-reduce
(forward, backward) and the standalone reduce, as a C-ABI HIP library with a
thin Python binding.  See `partial_channel_reduce_amd.ops` for the calls."""
__all__ = ["synth"]
