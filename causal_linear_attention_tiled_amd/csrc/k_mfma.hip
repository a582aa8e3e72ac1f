// Reverse (dK, dV) sweep on matrix cores: not built yet, the generic kernel runs instead.
#include "la_internal.h"

namespace la {
bool mfma_rev_supported(int, int) { return false; }
void launch_rev_mfma(const SweepArgs&, const LamArgs&, hipStream_t) {}
}  // namespace la
