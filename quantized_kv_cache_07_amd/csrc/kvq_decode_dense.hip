// kvq_decode_dense.hip -- instantiations of the dense multi-query decode kernel
// (kvq_decode_dense.h) for 2-, 4- and 8-bit symmetric and asymmetric caches with key groups of
// 32, 64 or 128 channels, and for FP8 E4M3 and BF16 caches.
#include "kvq_decode_dense.h"

namespace kvq {

template <int NGK>
hipError_t launch_groups(const DecodeParams& p, int bits, bool asym, hipStream_t s) {
  switch (bits) {
    case 2: return asym ? launch_dense_t<2, KVQ_ASYM, NGK>(p, s) : launch_dense_t<2, KVQ_SYM, NGK>(p, s);
    case 4: return asym ? launch_dense_t<4, KVQ_ASYM, NGK>(p, s) : launch_dense_t<4, KVQ_SYM, NGK>(p, s);
    case 8: return asym ? launch_dense_t<8, KVQ_ASYM, NGK>(p, s) : launch_dense_t<8, KVQ_SYM, NGK>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_dense(const DecodeParams& p, int bits, int scheme, hipStream_t s) {
  if (scheme == KVQ_FP8) return bits == 8 ? launch_dense_t<8, KVQ_FP8, 1>(p, s) : hipErrorInvalidValue;
  if (bits == 16) return launch_dense_t<16, KVQ_SYM, 1>(p, s);
  const bool asym = scheme == KVQ_ASYM;
  switch (p.c.k.group) {
    case 32: return launch_groups<4>(p, bits, asym, s);
    case 64: return launch_groups<2>(p, bits, asym, s);
    case 128: return launch_groups<1>(p, bits, asym, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
