// fp32 instantiations of the chunkwise prefill kernel (fp32 MFMA throughout).
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_f32(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    return chunk_detail::dispatch<float, float, kGatePlain>(a, s, launch, chunk_used);
}
}  // namespace kda
