// bf16-input instantiations of the chunkwise prefill kernel with fp32 output
// (bf16 MFMA, fp32 accumulate).
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_bf16_f32out(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    return chunk_detail::dispatch<bf16, float, kGatePlain>(a, s, launch, chunk_used);
}
}  // namespace kda
