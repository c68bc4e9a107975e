// bf16-input instantiations of the chunkwise prefill kernel with bf16 output.
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_bf16_bf16out(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    return chunk_detail::dispatch<bf16, bf16, kGatePlain>(a, s, launch, chunk_used);
}
}  // namespace kda
