// ia_chunk_rm64.hip — instantiations of the chunked prefill's output pass with a readout
// matrix, chunk length 64 (F = Dv = 128 with M = 64 does not fit the LDS: chunk 32 serves it).
#include "ia_chunk.hpp"

namespace ia {

#define IA_INST(FF, MM)                                                                      \
  template hipError_t launch_chunk_t<64, FF, FF, MM, true>(const ChunkArgs&, int, hipStream_t, \
                                                           int);                             \
  template int chunk_occupancy_t<64, FF, FF, MM, true>();
IA_INST(32, 16) IA_INST(32, 32) IA_INST(32, 64)
IA_INST(64, 16) IA_INST(64, 32) IA_INST(64, 64)
IA_INST(128, 16) IA_INST(128, 32)
#undef IA_INST

}  // namespace ia
