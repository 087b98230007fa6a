// kvq_decode_mix_k8s.hip -- decode-attention kernels for caches whose keys are 8-bit symmetric
// and whose values use another integer format (instantiations of kvq_decode.h).
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_decode_mixed_k8s(const DecodeParams& p, int vb, int vsch, int G, int NP, bool kpc,
                                  hipStream_t s) {
  return launch_decode_mixed<8, KVQ_SYM>(p, vb, vsch, G, NP, kpc, s);
}

}  // namespace kvq
