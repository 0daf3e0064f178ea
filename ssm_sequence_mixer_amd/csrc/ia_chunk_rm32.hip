// ia_chunk_rm32.hip — instantiations of the chunked prefill's output pass with a readout
// matrix, chunk length 32 (every supported F = Dv and M).
#include "ia_chunk.hpp"

namespace ia {

#define IA_INST(FF, MM)                                                                      \
  template hipError_t launch_chunk_t<32, FF, FF, MM, true>(const ChunkArgs&, int, hipStream_t, \
                                                           int);                             \
  template int chunk_occupancy_t<32, FF, FF, MM, true>();
IA_INST(32, 16) IA_INST(32, 32) IA_INST(32, 64)
IA_INST(64, 16) IA_INST(64, 32) IA_INST(64, 64)
IA_INST(128, 16) IA_INST(128, 32) IA_INST(128, 64)
#undef IA_INST

}  // namespace ia
