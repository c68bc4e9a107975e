// Bf16-input instantiations with bf16 output of the chunkwise prefill with the bounded
// forget gate fused in (the kernels form g from the gate's pre-activation).
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_bf16_bf16out_gz(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    return chunk_detail::dispatch<bf16, bf16, kGateFused>(a, s, launch, chunk_used);
}
}  // namespace kda
