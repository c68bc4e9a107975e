// bf16 instantiations of the chunkwise prefill kernel (bf16 MFMA, fp32 accumulate).
#include "kda_chunk_dispatch.cuh"

namespace kda {
hipError_t launch_chunk_bf16(const ChunkArgs &a, hipStream_t s, bool launch, bool *ok) {
    return chunk_detail::dispatch<bf16>(a, s, launch, ok);
}
}  // namespace kda
