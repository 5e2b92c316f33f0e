// Host-side argument checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only).  Every call below is rejected
// by a host check before anything touches a device, so the program runs
// without a GPU; it prints one line per failed expectation and exits 1 if
// there was any.  Built and run by tests/test_host_sanitizer.py.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe_mxfp4.h"

static int g_fail = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      std::printf("FAIL line %d: ", __LINE__);              \
      std::printf(__VA_ARGS__);                             \
      std::printf("\n");                                    \
      ++g_fail;                                             \
    }                                                       \
  } while (0)
#define EXPECT_ST(call, want)                                                               \
  do {                                                                                      \
    const moe_status st_ = (call);                                                          \
    EXPECT(st_ == (want), "%s -> %d (%s), want %d", #call, (int)st_, moe_status_string(st_), \
           (int)(want));                                                                    \
  } while (0)

int main() {
  // stand-in "device" buffers: never dereferenced, only checked for NULL and alignment
  alignas(256) static uint8_t buf[1 << 16];
  uint16_t* x = reinterpret_cast<uint16_t*>(buf);
  float* f = reinterpret_cast<float*>(buf + 4096);
  int32_t* i32 = reinterpret_cast<int32_t*>(buf + 8192);
  uint8_t* u8 = buf + 12288;
  uint16_t* x_odd = reinterpret_cast<uint16_t*>(buf + 2);       // not 16-byte aligned
  void* ws = buf + 16384;

  // status strings: every code and an unknown one
  for (int s = 0; s <= 7; ++s) EXPECT(moe_status_string((moe_status)s) != nullptr, "status %d", s);
  // 6 and 7 are representable in the enumeration (C++) but name no status
  EXPECT(std::strcmp(moe_status_string((moe_status)7), "unknown status") == 0, "unknown status");

  // workspace sizes: valid sizes give a positive multiple of 256 below 64 GiB,
  // invalid ones 0
  const int Ms[] = {1, 2, 4, 5, 8, 9, 15, 16, 17, 63, 64, 65, 512, 4096, 65536};
  const int ks[] = {1, 8, 32};
  const int Es[] = {32, 512, 1024};
  const int Hs[] = {32, 2560, 8192};
  const int Is[] = {32, 768, 4096};
  for (int M : Ms)
    for (int k : ks)
      for (int E : Es)
        for (int H : Hs)
          for (int I : Is) {
            const size_t b = moe_workspace_bytes(M, k, E, H, I);
            EXPECT(b > 0 && b % 256 == 0 && b < (size_t(64) << 30), "workspace(%d,%d,%d,%d,%d) = %zu", M, k, E,
                   H, I, b);
          }
  EXPECT(moe_workspace_bytes(0, 8, 512, 2560, 768) == 0, "M = 0");
  EXPECT(moe_workspace_bytes(MOE_MAX_TOKENS + 1, 8, 512, 2560, 768) == 0, "M too large");
  EXPECT(moe_workspace_bytes(4, 0, 512, 2560, 768) == 0, "k = 0");
  EXPECT(moe_workspace_bytes(4, 9, 8, 2560, 768) == 0, "k > E");
  EXPECT(moe_workspace_bytes(4, 33, 1024, 2560, 768) == 0, "k > MOE_MAX_TOPK");
  EXPECT(moe_workspace_bytes(4, 8, MOE_MAX_EXPERTS + 1, 2560, 768) == 0, "E too large");
  EXPECT(moe_workspace_bytes(4, 8, 512, 2561, 768) == 0, "H not a multiple of 32");
  EXPECT(moe_workspace_bytes(4, 8, 512, MOE_MAX_HIDDEN + 32, 768) == 0, "H too large");
  EXPECT(moe_workspace_bytes(4, 8, 512, 2560, 16) == 0, "I too small");
  EXPECT(moe_workspace_bytes(4, 8, 512, 2560, MOE_MAX_INTER + 32) == 0, "I too large");
  EXPECT(moe_workspace_bytes(-1, 8, 512, 2560, 768) == 0, "negative M");

  moe_mxfp4_weights w{};
  w.w13_q = u8; w.w13_s = u8; w.w2_q = u8; w.w2_s = u8;
  w.num_experts = 512; w.hidden = 2560; w.inter = 768; w.has_shared = 1;
  const size_t wsb = moe_workspace_bytes(4, 8, 512, 2560, 768);

  // moe_layer / moe_layer_ex: each check in turn
  EXPECT_ST(moe_layer(nullptr, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_NULL);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, nullptr, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_NULL);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, &w, 0, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_SHAPE);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, &w, 4, 0, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_SHAPE);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, &w, MOE_MAX_TOKENS + 1, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb,
                      nullptr),
            MOE_ERR_SHAPE);
  EXPECT_ST(moe_layer(x, f, f, 7, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_layer(x_odd, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_ALIGN);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, buf + 16, wsb, nullptr),
            MOE_ERR_ALIGN);
  EXPECT_ST(moe_layer(x, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb - 1, nullptr),
            MOE_ERR_WORKSPACE);
  {
    moe_mxfp4_weights b = w;
    b.hidden = 2561;
    EXPECT_ST(moe_layer(x, f, nullptr, 0, &b, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
              MOE_ERR_SHAPE);
    b = w;
    b.has_shared = 2;
    EXPECT_ST(moe_layer(x, f, nullptr, 0, &b, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
              MOE_ERR_SHAPE);
    b = w;
    b.w2_s = nullptr;
    EXPECT_ST(moe_layer(x, f, nullptr, 0, &b, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
              MOE_ERR_NULL);
    b = w;
    b.w13_q = u8 + 1;
    EXPECT_ST(moe_layer(x, f, nullptr, 0, &b, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
              MOE_ERR_ALIGN);
  }
  {
    moe_exec_opts o{};
    o.act8 = 2;
    EXPECT_ST(moe_layer_ex(x, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, &o, nullptr),
              MOE_ERR_SHAPE);
    o = moe_exec_opts{};
    o.helper_streams[0] = buf;                                  // one helper stream without the other
    EXPECT_ST(moe_layer_ex(x, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, &o, nullptr),
              MOE_ERR_NULL);
    o.helper_streams[1] = buf;                                  // both, but no events
    EXPECT_ST(moe_layer_ex(x, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, &o, nullptr),
              MOE_ERR_NULL);
  }
  // the entry point without a workspace: too large for its static array
  EXPECT_ST(moe_layer_noalloc(x, f, nullptr, 0, &w, 4096, 8, f, i32, f, i32, i32, i32, i32, f, nullptr),
            MOE_ERR_WORKSPACE);
  EXPECT_ST(moe_layer_noalloc(nullptr, f, nullptr, 0, &w, 4, 8, f, i32, f, i32, i32, i32, i32, f, nullptr),
            MOE_ERR_NULL);

  // the three-call route
  EXPECT_ST(moe_route(nullptr, f, nullptr, 0, 4, 2560, 512, 8, f, i32, f, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_route(x, f, nullptr, 0, 4, 2548, 512, 8, f, i32, f, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_route(x_odd, f, nullptr, 0, 4, 2560, 512, 8, f, i32, f, nullptr), MOE_ERR_ALIGN);
  EXPECT_ST(moe_topk_softmax(f, 4, 512, 0, i32, f, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_topk_softmax(nullptr, 4, 512, 8, i32, f, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_sort_by_expert(i32, 4, 8, 4, i32, i32, i32, i32, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_sort_by_expert(i32, 4, 8, 512, nullptr, i32, i32, i32, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_mxfp4_forward(x, &w, 4, 8, f, i32, i32, i32, i32, f, ws, wsb - 256, nullptr), MOE_ERR_WORKSPACE);
  EXPECT_ST(moe_mxfp4_forward(x, &w, 4, 8, nullptr, i32, i32, i32, i32, f, ws, wsb, nullptr), MOE_ERR_NULL);
  {
    moe_exec_opts o{};
    o.act8 = -1;
    EXPECT_ST(moe_mxfp4_forward_ex(x, &w, 4, 8, f, i32, i32, i32, i32, f, ws, wsb, &o, nullptr), MOE_ERR_SHAPE);
  }

  // measurement and auxiliary entry points
  const uint64_t* addrs = reinterpret_cast<const uint64_t*>(buf + 20480);
  const int64_t* sizes = reinterpret_cast<const int64_t*>(buf + 24576);
  uint32_t* out = reinterpret_cast<uint32_t*>(buf + 28672);
  EXPECT_ST(moe_read_probe(addrs, sizes, 0, 16384, out, 1024, nullptr, nullptr, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_read_probe(addrs, sizes, 1, 15, out, 1024, nullptr, nullptr, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_read_probe(addrs, sizes, 1, 16384, out, 1024, buf, nullptr, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_read_probe(nullptr, sizes, 1, 16384, out, 1024, nullptr, nullptr, nullptr), MOE_ERR_NULL);
  EXPECT(moe_layer_probe_stamps(4, 8, 512, 2560, 768) > 0, "probe stamps for the decode path");
  EXPECT(moe_layer_probe_stamps(64, 8, 512, 2560, 768) == 0, "probe stamps outside the decode path");
  EXPECT_ST(moe_layer_hinted(x, f, nullptr, 0, &w, 1, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, i32, nullptr,
                             nullptr, nullptr, nullptr),
            MOE_ERR_NULL);
  EXPECT_ST(moe_mxfp8_quantize(x, 4, 33, u8, u8, nullptr, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_mxfp8_quantize(nullptr, 4, 64, u8, u8, nullptr, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_layer_w4a8(x, f, nullptr, 0, &w, 0, 8, f, i32, f, i32, i32, i32, i32, f, ws, wsb, nullptr),
            MOE_ERR_SHAPE);
  EXPECT_ST(moe_mxfp4_dequantize(u8, u8, 4, 33, f, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_mxfp4_dequantize(nullptr, u8, 4, 64, f, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_prefetch_select(i32, -1, 512, 1, 16, i32, i32, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_prefetch_experts(nullptr, i32, i32, 16, 3, out, nullptr), MOE_ERR_NULL);
  EXPECT_ST(moe_lmhead_fp8_quantize(x, 0, 2560, u8, f, nullptr), MOE_ERR_SHAPE);
  EXPECT_ST(moe_lmhead_fp8_logits(x, u8, f, MOE_LMHEAD_MAX_TOKENS + 1, 1000, 2560, f, nullptr), MOE_ERR_SHAPE);

  std::printf("host checks: %d failed\n", g_fail);
  return g_fail ? 1 : 0;
}
