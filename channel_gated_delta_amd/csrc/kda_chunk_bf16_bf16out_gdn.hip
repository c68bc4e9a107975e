// Bf16-input instantiations with bf16 output of the chunkwise prefill with one decay per
// (token, head): the head-wise forget gate of GDN, g [T, H] broadcast to every
// key channel.
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_bf16_bf16out_gdn(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    return chunk_detail::dispatch<bf16, bf16, kGateHead>(a, s, launch, chunk_used);
}
}  // namespace kda
