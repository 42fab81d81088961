// Host-only driver for the C ABI's argument checks, built with AddressSanitizer
// and UndefinedBehaviorSanitizer around the library's host code (api.cpp).
//
// Every call below violates the contract of include/wf.h in one way (or is a
// documented no-op), so each must return its status code from the host
// checks, before any HIP call: the device pointers are fake addresses that
// are never dereferenced.  The launch functions and the few HIP runtime calls
// the host code references are stubs here that abort if reached.  Prints
// "ok <n>" and exits 0 when every call returned what it should.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "wf.h"
#include "wf_internal.h"
#include "wf_mx.h"
#include "wf_qkv.h"
#include "wf_rotate.h"

// ---- stubs: the checks must return before any of these --------------------
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "FAIL: a rejected call reached %s\n", what);
  std::abort();
}
namespace wf {
hipError_t launch_publish(const PublishParams&, int, hipStream_t) { reached("launch_publish"); }
hipError_t launch_attn_bf16(const AttnParams&, int, int, hipStream_t) { reached("launch_attn_bf16"); }
hipError_t launch_attn_fp32(const AttnParams&, int, int, hipStream_t) { reached("launch_attn_fp32"); }
hipError_t launch_publish_mx(const PublishParams&, void*, hipStream_t) { reached("launch_publish_mx"); }
hipError_t launch_attn_mx(const AttnParams&, const void*, hipStream_t) { reached("launch_attn_mx"); }
hipError_t launch_qkv_publish(const QkvParams&, hipStream_t) { reached("launch_qkv_publish"); }
hipError_t launch_rotate(int32_t*, int, int, int, hipStream_t) { reached("launch_rotate"); }
int* status_word_ptr(hipError_t*) { reached("status_word_ptr"); }
}  // namespace wf
extern "C" {
hipError_t hipDeviceSynchronize(void) { reached("hipDeviceSynchronize"); }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { reached("hipMemcpy"); }
const char* hipGetErrorString(hipError_t) { reached("hipGetErrorString"); }
}

// ---- the calls ---------------------------------------------------------------
static const uintptr_t FAKE = 0x7F0000001000ull;   // 16-byte aligned, never touched
static void* fp(uintptr_t off = 0) { return reinterpret_cast<void*>(FAKE + off); }

static int n_checked = 0;
static void expect(int rc, int want, const char* needle, const char* what) {
  const char* err = wf_last_error();
  const bool msg_ok = needle ? std::strstr(err, needle) != nullptr : err[0] == '\0';
  if (rc != want || !msg_ok) {
    std::fprintf(stderr, "FAIL %s: rc %d (want %d), message \"%s\" (want \"%s\")\n", what, rc,
                 want, err, needle ? needle : "");
    std::exit(1);
  }
  ++n_checked;
}

static wf_kv_pool pool(int page_size = 256, int head_dim = 128, int heads = 4) {
  wf_kv_pool p{};
  p.k_pages = fp();
  p.v_pages = fp(0x100000);
  p.page_table = static_cast<const int32_t*>(fp(0x200000));
  p.num_pages = 10;
  p.num_logical_pages = 10;
  p.page_size = page_size;
  p.num_heads = heads;
  p.head_dim = head_dim;
  p.dtype = WF_BF16;
  return p;
}

int main() {
  const wf_rope rope{44, 42, 42, 1e4};
  const int32_t* pos = static_cast<const int32_t*>(fp(0x300000));
  // pool descriptors, through publish and attention
  for (int ps : {8, 48, 2048}) {
    wf_kv_pool p = pool(ps);
    expect(wf_kv_publish(&p, &rope, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
           WF_ERR_INVALID, "page_size", "publish page_size");
  }
  {
    wf_kv_pool p = pool(256, 96);
    expect(wf_kv_publish(&p, &rope, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
           WF_ERR_UNSUPPORTED, "head_dim", "publish head_dim");
    expect(wf_kv_publish(nullptr, &rope, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
           WF_ERR_INVALID, "NULL", "publish null pool");
  }
  wf_kv_pool p = pool();
  // publish
  const wf_rope odd{43, 43, 42, 1e4}, bad_theta{44, 42, 42, -1.0};
  expect(wf_kv_publish(&p, &odd, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "even", "publish odd rope");
  expect(wf_kv_publish(&p, &bad_theta, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "theta", "publish theta");
  expect(wf_kv_publish(&p, &rope, fp(), 512, fp(), 512, nullptr, 100, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "pos_thw", "publish pos");
  expect(wf_kv_publish(&p, &rope, fp(), 500, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "k_row_stride", "publish k stride");
  expect(wf_kv_publish(&p, &rope, fp(), 512, fp(4), 512, pos, 100, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "aligned", "publish v align");
  expect(wf_kv_publish(&p, &rope, fp(), 512, fp(), 512, pos, 61, 2500, nullptr, 0, nullptr),
         WF_ERR_INVALID, "capacity", "publish capacity");
  expect(wf_kv_publish(&p, &rope, fp(), 512, fp(), 512, pos, -1, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "n_tok", "publish n_tok");
  expect(wf_kv_publish(&p, &rope, nullptr, 0, nullptr, 0, pos, 0, 0, nullptr, 0, nullptr), WF_OK,
         nullptr, "publish no-op");
  // attention
  std::vector<wf_segment> segs = {{0, 100, -1}, {100, 50, 0}, {150, 50, 1}};
  int32_t qss[3] = {0, 50, 100};
  expect(wf_chunk_attn(&p, segs.data(), 3, fp(), 512, qss, 2, 0, 0.088f, fp(2), 512, nullptr,
                       nullptr),
         WF_ERR_INVALID, "aligned", "attn out align");
  expect(wf_chunk_attn(&p, segs.data(), 3, fp(), 512, qss, 2, 0, 0.0f, fp(), 512, nullptr, nullptr),
         WF_ERR_INVALID, "scale", "attn scale");
  expect(wf_chunk_attn(&p, segs.data(), 0, fp(), 512, qss, 2, 0, 0.088f, fp(), 512, nullptr,
                       nullptr),
         WF_ERR_INVALID, "n_segs", "attn n_segs");
  int32_t qss_bad[3] = {0, 60, 50};
  expect(wf_chunk_attn(&p, segs.data(), 3, fp(), 512, qss_bad, 2, 0, 0.088f, fp(), 512, nullptr,
                       nullptr),
         WF_ERR_INVALID, "non-decreasing", "attn qss order");
  std::vector<wf_segment> overlap = {{0, 100, -1}, {90, 50, 0}, {150, 50, 1}};
  expect(wf_chunk_attn(&p, overlap.data(), 3, fp(), 512, qss, 2, 0, 0.088f, fp(), 512, nullptr,
                       nullptr),
         WF_ERR_INVALID, "overlap", "attn overlap");
  // many unmergeable ranges: more than the range table holds
  std::vector<wf_segment> many;
  for (int i = 0; i < 32; ++i) many.push_back({i * 20, 10, -1});
  for (int i = 0; i < 32; ++i) many.push_back({1000 + i * 20, 10, i});
  std::vector<int32_t> qss_many;
  for (int i = 0; i <= 32; ++i) qss_many.push_back(i * 10);
  expect(wf_chunk_attn(&p, many.data(), 64, fp(), 512, qss_many.data(), 32, 0, 0.088f, fp(), 512,
                       nullptr, nullptr),
         WF_ERR_UNSUPPORTED, "ranges", "attn too many ranges");
  int32_t qss_empty[3] = {7, 7, 7};
  expect(wf_chunk_attn(&p, segs.data(), 3, nullptr, 512, qss_empty, 2, 0, 0.088f, nullptr, 512,
                       nullptr, nullptr),
         WF_OK, nullptr, "attn no rows");
  // generic query groups
  std::vector<wf_kv_run> runs = {{0, 100}, {100, 50}, {150, 50}};
  std::vector<wf_query_group> groups = {{0, 50, 0, 3}, {40, 100, 0, 2}};
  expect(wf_group_attn(&p, runs.data(), 3, groups.data(), 2, fp(), 512, 0.088f, fp(), 512, nullptr,
                       0, nullptr),
         WF_ERR_INVALID, "overlap at row 40", "group overlap");
  groups = {{0, 50, 1, 4}};
  expect(wf_group_attn(&p, runs.data(), 3, groups.data(), 1, fp(), 512, 0.088f, fp(), 512, nullptr,
                       0, nullptr),
         WF_ERR_INVALID, "runs", "group runs");
  groups = {{0, 50, 0, 3}};
  expect(wf_group_attn(&p, runs.data(), 3, groups.data(), 1, fp(), 512, 0.088f, fp(), 512,
                       static_cast<float*>(fp(0x400000)), 49, nullptr),
         WF_ERR_INVALID, "lse_stride", "group lse stride");
  // MXFP8 keys
  wf_mx_keys keys{fp(0x500000), fp(0x600000)};
  wf_kv_pool p64 = pool(256, 64);
  expect(wf_kv_publish_mx(&p64, &keys, &rope, fp(), 512, fp(), 512, pos, 100, 0, nullptr, 0, nullptr),
         WF_ERR_UNSUPPORTED, "mx keys", "mx head_dim");
  wf_mx_keys null_keys{nullptr, fp(0x600000)};
  expect(wf_chunk_attn_mx(&p, &null_keys, segs.data(), 3, fp(), 512, qss, 2, 0, 0.088f, fp(), 512,
                          nullptr, nullptr),
         WF_ERR_INVALID, "non-NULL", "mx null codes");
  // fused QKV projection
  expect(wf_qkv_publish(&p, &rope, fp(), 256, 100, fp(), nullptr, pos, 10, 0, nullptr, 0, nullptr),
         WF_ERR_UNSUPPORTED, "hidden", "qkv hidden");
  expect(wf_qkv_publish(&p, &rope, fp(), 60, 64, fp(), nullptr, pos, 10, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "x_row_stride", "qkv x stride");
  expect(wf_qkv_publish(&p, &rope, fp(), 64, 64, fp(), fp(1), pos, 10, 0, nullptr, 0, nullptr),
         WF_ERR_INVALID, "bias", "qkv bias align");
  // history rotation
  int32_t* table = static_cast<int32_t*>(fp(0x700000));
  expect(wf_history_rotate(nullptr, 64, 256, 512, 1024, 3, nullptr), WF_ERR_INVALID, "NULL",
         "rotate null");
  expect(wf_history_rotate(table, 64, 256, 100, 1024, 3, nullptr), WF_ERR_INVALID, "window_start",
         "rotate start");
  expect(wf_history_rotate(table, 1 << 20, 16, 0, 16, 16385, nullptr), WF_ERR_UNSUPPORTED,
         "limit", "rotate limit");
  expect(wf_history_rotate(table, 64, 256, 512, 1024, 1, nullptr), WF_OK, nullptr, "rotate noop");
  // status word
  expect(wf_device_status(nullptr, 0), WF_ERR_INVALID, "NULL", "status null");
  std::printf("ok %d\n", n_checked);
  return 0;
}
