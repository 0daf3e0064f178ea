// ia_chunk_g32.hip — instantiations of the gated layer's chunked prefill kernels (output and state-only passes) for F = Dv = 32.
#include "ia_chunk.hpp"
#include "ia_chunk_state.hpp"

namespace ia {

#define IA_INST(C, MM)                                                                    \
  template hipError_t launch_chunk_t<C, 32, 32, MM, false, true>(const ChunkArgs&, int,   \
                                                               hipStream_t, int);         \
  template hipError_t launch_state_t<C, 32, 32, MM, true>(const ChunkArgs&, int,          \
                                                        hipStream_t, int);                \
  template int chunk_occupancy_t<C, 32, 32, MM, false, true>();
IA_INST(32, 16) IA_INST(32, 32) IA_INST(32, 64)
IA_INST(64, 16) IA_INST(64, 32) IA_INST(64, 64)
#undef IA_INST

}  // namespace ia
