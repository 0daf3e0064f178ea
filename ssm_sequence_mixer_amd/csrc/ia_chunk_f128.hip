// ia_chunk_f128.hip — instantiations of the chunked prefill kernels (output and state-only passes) for F = Dv = 128.
#include "ia_chunk.hpp"
#include "ia_chunk_state.hpp"

namespace ia {

template hipError_t launch_chunk_t<32, 128, 128, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<32, 128, 128, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<32, 128, 128, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 128, 128, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 128, 128, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_chunk_t<64, 128, 128, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 128, 128, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 128, 128, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<32, 128, 128, 64>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 128, 128, 16>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 128, 128, 32>(const ChunkArgs&, int, hipStream_t, int);
template hipError_t launch_state_t<64, 128, 128, 64>(const ChunkArgs&, int, hipStream_t, int);
template int chunk_occupancy_t<32, 128, 128, 16>();
template int chunk_occupancy_t<32, 128, 128, 32>();
template int chunk_occupancy_t<32, 128, 128, 64>();
template int chunk_occupancy_t<64, 128, 128, 16>();
template int chunk_occupancy_t<64, 128, 128, 32>();
template int chunk_occupancy_t<64, 128, 128, 64>();

}  // namespace ia
