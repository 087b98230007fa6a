// host_abi_check.cpp -- drives the host side of libkvq's C ABI (format checks, buffer sizing,
// workspace sizing, argument validation, launch configuration) under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU.  Test infrastructure: built by
// tests/test_sanitizers.py from kvq_host.hip (host code instrumented) and this file, which
// stands in for the kernel translation units: each launch function below checks, on the host,
// that the configuration it is handed stays inside the caller's buffers (the unit-range
// workspace and partial slots inside the workspace, the append grid inside the cache), then
// returns without launching.  Prints "ok" and exits 0.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvq_dev.h"

namespace kvq {

static size_t g_ws_bytes = 0;
static const char* g_ws = nullptr;
static long g_launches = 0;

static void fail(const char* what) {
  std::printf("FAIL: %s\n", what);
  std::exit(1);
}

static hipError_t check_decode(const DecodeParams& p, int G, int NP) {
  g_launches++;
  if (G < 1 || G > 16 || (G > 8 && G != 16) || (NP != 1 && NP != 2)) fail("decode G / NP");
  if (p.nblocks < 1) fail("decode nblocks");
  const char* pre_end = reinterpret_cast<const char*>(p.ws_pre + p.c.B + 2);
  const char* part = reinterpret_cast<const char*>(p.ws_part);
  const size_t part_bytes = static_cast<size_t>(p.nblocks) * 2 * p.qpw * G * PART_STRIDE * 4;
  if (reinterpret_cast<const char*>(p.ws_pre) != g_ws) fail("prefix not at the workspace start");
  if (pre_end > part) fail("prefix overlaps the partials");
  if (part + part_bytes > g_ws + g_ws_bytes) fail("partials beyond the workspace");
  if (G != p.qbs * p.gkv || p.nqb * p.qbs < p.nqt || p.nqs * p.qpw < p.nqb) fail("query blocks");
  return hipSuccess;
}

#define KVQ_STUB(name)                                                                    \
  hipError_t name(const DecodeParams& p, int G, int NP, bool, hipStream_t) { return check_decode(p, G, NP); }
KVQ_STUB(launch_decode_b2s)
KVQ_STUB(launch_decode_b4s)
KVQ_STUB(launch_decode_b8s)
KVQ_STUB(launch_decode_b2a)
KVQ_STUB(launch_decode_b4a)
KVQ_STUB(launch_decode_b8a)
KVQ_STUB(launch_decode_b16)
KVQ_STUB(launch_decode_b8f)
#undef KVQ_STUB
#define KVQ_MIX(name)                                                                     \
  hipError_t name(const DecodeParams& p, int vb, int vs, int G, int NP, bool, hipStream_t) { \
    if ((vb != 2 && vb != 4 && vb != 8) || (vs != KVQ_SYM && vs != KVQ_ASYM)) fail("mixed value format"); \
    return check_decode(p, G, NP);                                                         \
  }
KVQ_MIX(launch_decode_mixed_k2s)
KVQ_MIX(launch_decode_mixed_k2a)
KVQ_MIX(launch_decode_mixed_k4s)
KVQ_MIX(launch_decode_mixed_k4a)
KVQ_MIX(launch_decode_mixed_k8s)
KVQ_MIX(launch_decode_mixed_k8a)
#undef KVQ_MIX
hipError_t launch_decode_dense(const DecodeParams& p, int bits, int scheme, hipStream_t) {
  if (bits != 2 && bits != 4 && bits != 8 && bits != 16) fail("dense bits");
  if (p.qpw != 4 || p.qbs * p.gkv != 16) fail("dense query blocks");
  if (scheme == KVQ_FP8 ? bits != 8
                        : bits != 16 && p.c.k.group != 32 && p.c.k.group != 64 && p.c.k.group != 128)
    fail("dense key format");
  return check_decode(p, 16, 1);
}

hipError_t launch_append(const CacheDev& c, const uint16_t*, const uint16_t*, int n_new, int mode,
                         hipStream_t) {
  g_launches++;
  if (mode == MODE_APPEND && n_new < 1) fail("append n_new");
  if (c.B < 1 || c.H < 1) fail("append cache");
  return hipSuccess;
}

}  // namespace kvq

static kvq_cache fake(const kvq_format& f, int B, int H, int cap, int nblk) {
  kvq_cache c{};
  c.fmt = f;
  c.batch = B;
  c.n_kv_heads = H;
  c.capacity = nblk ? 0 : cap;
  c.num_blocks = nblk;
  c.max_blocks = nblk ? 8 : 0;
  c.block_table = nblk ? reinterpret_cast<const int32_t*>(0x100000) : nullptr;
  uintptr_t a = 0x200000;
  auto next = [&]() { a += 0x10000; return reinterpret_cast<void*>(a); };
  c.k_codes = static_cast<uint8_t*>(next());
  c.v_codes = static_cast<uint8_t*>(next());
  c.k_scale = static_cast<uint16_t*>(next());
  c.v_scale = static_cast<uint16_t*>(next());
  c.k_zero = static_cast<uint16_t*>(next());
  c.v_zero = static_cast<uint16_t*>(next());
  c.k_res = static_cast<uint16_t*>(next());
  c.v_res = static_cast<uint16_t*>(next());
  c.n_quant = static_cast<int32_t*>(next());
  c.n_res = static_cast<int32_t*>(next());
  c.err = static_cast<int32_t*>(next());
  return c;
}

int main() {
  using namespace kvq;
  const int bits_l[] = {2, 3, 4, 8, 16};
  const int sch_l[] = {0, 1, 2, 5};
  const int axis_l[] = {0, 1, 2, 3, 7};
  const int grp_l[] = {0, 16, 32, 48, 64, 128};
  const int res_l[] = {0, 16, 24, 64, 128, 512};
  std::vector<kvq_side> sides;
  for (int b : bits_l)
    for (int s : sch_l)
      for (int ax : axis_l)
        for (int g : grp_l) sides.push_back(kvq_side{b, s, ax, g});
  // every combination through the format check and the buffer sizing
  std::vector<kvq_format> valid;
  for (const kvq_side& k : sides)
    for (const kvq_side& v : sides)
      for (int R : res_l) {
        kvq_format f{k, v, R, 128};
        if (kvq_check_format(&f) != KVQ_OK) continue;
        if (valid.size() < 100000) valid.push_back(f);
        for (int which = -1; which <= 8; which++) {
          (void)kvq_buffer_bytes(&f, 3, 8, 4096, 0, which);
          (void)kvq_buffer_bytes(&f, 3, 8, 0, 1000, which);
          (void)kvq_buffer_bytes(&f, INT_MAX, INT_MAX, INT_MAX - 15, 0, which);
        }
      }
  // launch configurations of a spread of valid formats (every 37th), batch and head counts,
  // query heads, token bounds and query counts: the workspace a call is sized for holds what
  // the launch addresses (the workspace is never dereferenced here)
  char* const wsp = reinterpret_cast<char*>(static_cast<uintptr_t>(1) << 40);
  for (size_t i = 0; i < valid.size(); i += 37) {
    const kvq_format& f = valid[i];
    for (int paged = 0; paged < 2; paged++)
      for (int B : {1, 3, 70})
        for (int H : {1, 2, 8}) {
          kvq_cache c = fake(f, B, H, 256, paged ? 40 : 0);
          for (int g : {1, 2, 4, 8})
            for (int mt : {1, 17, 1000, 131072, INT_MAX})
              for (int nq : {1, 2, 5, 16}) {
                const int hq = g * H;
                const size_t ws = kvq_decode_workspace_bytes_mq(&c, hq, nq, mt);
                if (ws == 0) continue;
                g_ws = wsp;
                g_ws_bytes = ws;
                (void)kvq_decode_attention_mq(&c, reinterpret_cast<void*>(0x1000), nq, hq, 0.1f, mt,
                                              reinterpret_cast<float*>(0x2000), wsp, ws, nullptr);
                if (kvq_decode_attention_mq(&c, reinterpret_cast<void*>(0x1000), nq, hq, 0.1f, mt,
                                            reinterpret_cast<float*>(0x2000), wsp, ws - 1,
                                            nullptr) == KVQ_OK)
                  fail("workspace one byte short accepted");
              }
          (void)kvq_quantize_append(&c, reinterpret_cast<void*>(0x1000), reinterpret_cast<void*>(0x1000),
                                    37, nullptr);
          (void)kvq_flush_residual(&c, nullptr);
        }
  }
  const long n_valid = static_cast<long>(valid.size());
  // argument errors return before any launch
  const long before = g_launches;
  kvq_format f{{4, 0, 0, 64}, {4, 0, 0, 64}, 32, 128};
  kvq_cache c = fake(f, 2, 2, 256, 0);
  if (kvq_quantize_append(nullptr, nullptr, nullptr, 1, nullptr) == KVQ_OK) fail("null cache");
  if (kvq_quantize_append(&c, reinterpret_cast<void*>(0x1008), reinterpret_cast<void*>(0x1000), 1,
                          nullptr) != KVQ_EALIGN) fail("alignment");
  if (kvq_quantize_append(&c, reinterpret_cast<void*>(0x1000), reinterpret_cast<void*>(0x1000), 0,
                          nullptr) != KVQ_EINVAL) fail("n_new 0");
  if (kvq_decode_attention(&c, reinterpret_cast<void*>(0x1000), 5, 0.1f, 100,
                           reinterpret_cast<float*>(0x2000), reinterpret_cast<void*>(0x3000), 1 << 20,
                           nullptr) != KVQ_EINVAL) fail("H_q not a multiple of H_kv");
  (void)kvq_decode_attention_noalloc(&c, reinterpret_cast<void*>(0x1000), 8, 0.1f, 100,
                                     reinterpret_cast<float*>(0x2000), nullptr);
  if (g_launches != before) fail("a refused call launched");
  for (int st = -1; st <= 7; st++) (void)kvq_status_str(static_cast<kvq_status>(st));
  std::printf("ok (%ld valid formats, %ld launches checked)\n", n_valid, g_launches);
  return 0;
}
