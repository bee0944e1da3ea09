// CPU driver of libqstate's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with g++, no
// GPU): the C ABI's validation, planning, handle building and argument checks
// over many configurations, valid and not.  The HIP runtime calls the host
// code makes are replaced by host-memory stand-ins and the kernel launchers
// by stubs that report a launch failure, so every path up to the launch runs.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <vector>

#include "qstate.h"
#include "qstate_internal.hpp"

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
  *p = std::malloc(n ? n : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
  std::memcpy(d, s, n);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stand-in"; }
}

static int g_launches = 0;
namespace qs {
hipError_t launch_step(int, int, int, int, const Args&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_quantize(const Args&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_dequantize(const Args&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
const char* step_kernel_name(int, int, int, int, int) { return "stand-in"; }
}  // namespace qs

static int g_fail = 0;
#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static bool known(qs_status s) {
  return s == QS_OK || s == QS_EINVAL || s == QS_EUNSUPPORTED || s == QS_ENOMEM || s == QS_EHIP;
}

int main() {
  std::mt19937_64 r(12345);
  auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + r() % v.size()); };
  int ok = 0, inited = 0;
  for (int it = 0; it < 4000; ++it) {
    // mostly well-formed configurations; one field in four made malformed
    const bool odd = r() % 4 == 0;
    const int which = (int)(r() % 16);
    auto field = [&](int id, std::initializer_list<int> good, std::initializer_list<int> badv) {
      return (odd && which == id) ? pick(badv) : pick(good);
    };
    qstate_config c{};
    c.abi_version = (odd && which == 0) ? 1u : QSTATE_ABI_VERSION;
    c.kind = field(1, {0, 1}, {2, -1});
    c.decay_mode = field(2, {0, 1}, {5, -3});
    c.B = field(3, {0, 1, 3, 7}, {-2});
    c.H = field(4, {1, 2, 3, 5}, {0, 70});
    c.dk = field(5, {64, 128, 256}, {100, 0, 512});
    c.dv = field(6, {1, 7, 40, 64, 128, 256}, {257, 0});
    c.qbits = field(7, {8, 4}, {2, 16});
    c.hp_dtype = field(8, {0, 1, 2}, {3});
    c.map_mode = field(9, {0, 0, 0, 1, 2}, {4});
    std::vector<uint8_t> map((size_t)std::max(1, std::max(c.H, 1) * std::max(c.dk, 1)));
    for (auto& m : map) m = (r() % 3 == 0);
    c.map = (odd && which == 10) ? nullptr : map.data();
    c.in_dtype = field(11, {0, 1}, {2, 7});
    c.rounding = field(12, {0, 1}, {3});
    c.sr_bits = field(12, {16, 8}, {4});
    c.bdr = pick({0, 1});
    c.bdr_bound = (odd && which == 13) ? NAN : (float)pick({0, 0, 1}) * 0.3f;
    const bool lrb = r() % 3 == 0;
    c.lrb_rank = lrb ? field(14, {1, 4, 8, 12, 16}, {20, -1}) : 0;
    c.lrb_period = pick({64, 3});
    c.lrb_theta = (odd && which == 14) ? 0.0f : 0.5f;
    if (lrb) c.map_mode = 0;
    c.seed = r();
    const bool bf = lrb && c.lrb_rank <= 8 && r() % 2 == 0;
    c.scale_dtype = bf ? 1 : 0;
    c.lrb_dtype = bf ? 1 : 0;
    if (odd && which == 15) c.scale_dtype = pick({1, 2});
    c.scale_axis = (!lrb && c.map_mode == 0 && !bf && r() % 3 == 0) ? pick({1, 2}) : 0;
    if (odd && which == 15 && r() % 2) c.scale_axis = pick({3, -1});
    qstate_sizes z{};
    qs_status s = qstate_plan(&c, &z);
    CHECK(known(s));
    CHECK(s == QS_OK || std::strlen(qstate_last_error()) > 0);
    if (s != QS_OK) continue;
    ++ok;
    CHECK(z.scales > 0 || c.B == 0);
    qstate_handle* h = nullptr;
    qstate_sizes z2{};
    s = qstate_init(&c, &h, &z2);
    CHECK(s == QS_OK && h != nullptr);
    if (s != QS_OK) continue;
    ++inited;
    CHECK(std::memcmp(&z, &z2, sizeof z) == 0);
    CHECK(qstate_kernel_name(h) != nullptr);
    // buffers of the planned sizes (host memory: the stand-in launchers
    // never touch them), then the argument checks of every entry point
    std::vector<uint8_t> pool(z.codes + z.scales + z.hp + z.lrb_W + z.lrb_U + z.lrb_n + 16 * 8 + 4096, 0);
    uintptr_t at = ((uintptr_t)pool.data() + 15u) & ~(uintptr_t)15u;
    auto take = [&](uint64_t n) { void* p = (void*)at; at += (n + 15u) & ~(uint64_t)15u; return n ? p : nullptr; };
    qstate_tensors st{take(z.codes), take(z.scales), take(z.hp), take(z.lrb_W), take(z.lrb_U),
                      (int32_t*)take(z.lrb_n)};
    float* io = (float*)take(1024);
    qstate_inputs in{io, io, io, io, nullptr};
    s = qstate_decode_step(h, &st, &in, io, 0, nullptr);
    CHECK(s == QS_EHIP || (c.B == 0 && s == QS_OK));
    qstate_inputs bad = in;
    bad.q = (const char*)io + 2;
    s = qstate_decode_step(h, &st, &bad, io, 0, nullptr);
    CHECK(s == QS_EINVAL || (c.B == 0 && s == QS_OK));
    s = qstate_decode_step(h, nullptr, &in, io, 0, nullptr);
    CHECK(s == QS_EINVAL || (c.B == 0 && s == QS_OK));
    CHECK(known(qstate_quantize(h, io, &st, 1, nullptr)));
    CHECK(known(qstate_dequantize(h, &st, io, nullptr)));
    int32_t slot[2] = {0, 1};
    uint64_t steps[2] = {0, 1};
    CHECK(known(qstate_decode_step_batch(h, &st, &in, io, c.B > 1 ? 2 : c.B, slot, steps, nullptr)));
    CHECK(qstate_decode_step_batch(h, &st, &in, io, c.B + 1, slot, steps, nullptr) == QS_EINVAL);
    qstate_destroy(h);
  }
  // precision maps: ties, NaN and infinite statistics, fractions at the ends
  for (int it = 0; it < 500; ++it) {
    const int groups = (int)(r() % 4), per = 1 + (int)(r() % 40);
    std::vector<float> stat((size_t)groups * per);
    for (auto& x : stat) x = (float)(r() % 5) * 0.25f;
    if (!stat.empty() && r() % 5 == 0) stat[r() % stat.size()] = NAN;
    if (!stat.empty() && r() % 5 == 0) stat[r() % stat.size()] = INFINITY;
    std::vector<uint8_t> m(stat.size() + 1);
    const float frac = (float)pick({0, 1, 2, 3, 4, -1, 5}) * 0.25f;
    CHECK(known(qstate_build_map(stat.data(), groups, per, frac, m.data())));
  }
  CHECK(qstate_build_map(nullptr, 1, 1, 0.5f, nullptr) == QS_EINVAL);
  for (int s = -8; s <= 2; ++s) CHECK(qstate_strerror((qs_status)s) != nullptr);
  qstate_destroy(nullptr);
  CHECK(qstate_plan(nullptr, nullptr) == QS_EINVAL);
  std::printf("host driver: %d valid plans, %d handles, %d launches reached, %d failed checks\n", ok, inited,
              g_launches, g_fail);
  return g_fail == 0 && ok > 100 && inited > 100 && g_launches > 100 ? 0 : 1;
}
