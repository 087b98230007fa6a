// kvq_decode_b8f.hip -- decode-attention kernels for FP8 E4M3 caches with per-tensor or
// per-head scales [P3 = oh-bug.com "KV Cache Quantization in Practice", "Step 3: Deploy a
// Fallback-Capable FP8 First"] (instantiations of kvq_decode.h).
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_decode_b8f(const DecodeParams& p, int G, int NP, bool kpc, hipStream_t s) {
  return launch_decode_bits<8, KVQ_FP8>(p, G, NP, kpc, s);
}

}  // namespace kvq
