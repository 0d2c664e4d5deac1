// MFMA bf16 chunk kernel of libssverify (not built yet in this revision).
#include "ss_common.h"

namespace ssv {
hipError_t launch_chunk_mfma(const ChunkParams&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssv
