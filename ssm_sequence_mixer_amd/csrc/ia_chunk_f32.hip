// ia_chunk_f32.hip — instantiations of the chunked prefill kernels (output and state-only passes) for F = Dv = 32.
#include "ia_chunk.hpp"
#include "ia_chunk_state.hpp"

namespace ia {

template hipError_t launch_chunk_t<32, 32, 32, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<32, 32, 32, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<32, 32, 32, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 32, 32, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 32, 32, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 32, 32, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 32, 32, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 32, 32, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 32, 32, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 32, 32, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 32, 32, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 32, 32, 64>(const ChunkArgs&, int, hipStream_t, int);
template int chunk_occupancy_t<32, 32, 32, 16>();
template int chunk_occupancy_t<32, 32, 32, 32>();
template int chunk_occupancy_t<32, 32, 32, 64>();
template int chunk_occupancy_t<64, 32, 32, 16>();
template int chunk_occupancy_t<64, 32, 32, 32>();
template int chunk_occupancy_t<64, 32, 32, 64>();

}  // namespace ia
