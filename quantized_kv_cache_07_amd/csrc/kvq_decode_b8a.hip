// kvq_decode_b8a.hip -- decode-attention kernels for 8-bit asymmetric caches (instantiations of
// kvq_decode.h, one translation unit per format so they compile in parallel).
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_decode_b8a(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  return launch_decode_bits<8, KVQ_ASYM>(p, G, NP, kpc, s);
}

}  // namespace kvq
