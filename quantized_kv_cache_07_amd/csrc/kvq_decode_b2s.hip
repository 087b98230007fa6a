// kvq_decode_b2s.hip -- decode-attention kernels for 2-bit symmetric caches (instantiations of
// kvq_decode.h, one translation unit per format so they compile in parallel).
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_decode_b2s(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  return launch_decode_bits<2, KVQ_SYM>(p, G, NP, kpc, s);
}

}  // namespace kvq
