// MFMA split-KV decode (placeholder until the tuned kernel lands).
#include "mla_internal.h"

namespace mla {
bool decode_mfma_supported(const DecodeArgs&) { return false; }
hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
