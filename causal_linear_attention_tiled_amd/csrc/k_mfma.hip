// MFMA kernels (placeholder until the matrix-core path lands).
#include "la_internal.h"

namespace la {
bool mfma_supported(int, int) { return false; }
void launch_fwd_mfma(const SweepArgs&, const LamArgs&, hipStream_t) {}
void launch_rev_mfma(const SweepArgs&, const LamArgs&, hipStream_t) {}
void launch_chunk_state_mfma(const ChunkStateArgs&, const LamArgs&, hipStream_t) {}
}  // namespace la
