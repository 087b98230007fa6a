// Decode attention over the unquantized BF16 cache (bits 16): the baseline the compressed
// formats are measured against [P2 = llmdaily.org "KV-cache quantization -- making long-context
// inference fit in memory", "Why compression may also improve speed"].
#include "kvq_decode.h"

namespace kvq {
hipError_t launch_decode_b16(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  return launch_decode_bits<16, KVQ_SYM>(p, G, NP, kpc, s);
}
}  // namespace kvq
