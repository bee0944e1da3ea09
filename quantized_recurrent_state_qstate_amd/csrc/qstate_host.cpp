// C-ABI host side of libqstate: argument validation, layout planning,
// handle management and kernel launch.  Validation and planning make no HIP
// call, so qstate_plan and every argument error path run without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <vector>

#include "qstate.h"
#include "qstate_internal.hpp"

namespace {

thread_local std::string g_last_error;

qs_status fail(qs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

qs_status ok() {
  g_last_error.clear();
  return QS_OK;
}

constexpr int kMaxRank = 16;
constexpr uint32_t kMaxLds = 64u * 1024u;

uint64_t round16(uint64_t x) { return (x + 15u) & ~uint64_t(15); }
uint64_t round4(uint64_t x) { return (x + 3u) & ~uint64_t(3); }

// Stored row bytes: codes of the quantized channels, values of the protected
// ones, each padded to a multiple of 4 bytes.
uint64_t code_row(uint64_t nq, uint64_t qbits) { return round4((nq * qbits + 7u) / 8u); }
uint64_t hp_row(uint64_t nhp, uint64_t hpb) { return round4(nhp * hpb); }

struct Plan {
  std::vector<uint64_t> code_off, hp_off;
  std::vector<int32_t> nq;
  std::vector<uint8_t> head_type;
  std::vector<uint16_t> slots;
  uint64_t code_bstride = 0, hp_bstride = 0;
  qstate_sizes sizes{};
  int family = qs::kFamDense;
  int row_chunks = 1;
  int dense_rpl = 1;
  int dense_lpr = 8;
  int keymap_eh = 2;
  int keymap_rpl = 1;
  int dense_threads = 256;
  uint32_t lds = 0;
  uint32_t rbuf = 0;            // mixed family: LDS for random bits by slot
  uint64_t prot_mask[4] = {0, 0, 0, 0};   // dense family: protected heads (H <= 256)
  uint64_t code_hblk = 0, hp_hblk = 0;
};

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  if (!e || !*e) return dflt;
  char* end = nullptr;
  long v = std::strtol(e, &end, 10);
  return (end && *end == 0) ? (int)v : dflt;
}

// Shape of the dense kernel: lanes per row (4 for the delta rule at dk 128,
// where the delta term makes the per-row work heavier and 32 keys per lane
// measured faster; 8 otherwise), rows per lane (two with 8 lanes when a head
// has more than 32 rows) and row groups per workgroup (whole waves, at most
// 256 threads).  QSTATE_DENSE_LPR (4, 8; dk 128 only), QSTATE_DENSE_RPL
// (1, 2) and QSTATE_DENSE_GROUPS override for tuning.
void dense_shape(int kind, int dk, int dv, int* lpr, int* rpl, int* threads, int* chunks) {
  int l = dk == 128 ? env_int("QSTATE_DENSE_LPR", kind == QS_KIND_DELTA ? 4 : 8) : 8;
  if (l != 4 && l != 8) l = 8;
  int r = env_int("QSTATE_DENSE_RPL", dv > 32 ? 2 : 1);
  if (r != 1 && r != 2) r = dv > 32 ? 2 : 1;
  if (l == 4) r = 1;                         // 32 keys per lane: one row per lane
  const int gpw = 64 / l;                    // row groups per wave
  const int gmax = 256 / l;                  // row groups per workgroup, at most
  int ng = (dv + r - 1) / r;                 // row groups needed for one head
  ng = std::min(gmax, (ng + gpw - 1) / gpw * gpw);   // whole waves
  const int ng_env = env_int("QSTATE_DENSE_GROUPS", 0);
  if (ng_env > 0 && ng_env <= gmax && ng_env % gpw == 0) ng = ng_env;
  *lpr = l;
  *rpl = r;
  *threads = l * ng;
  *chunks = (dv + ng * r - 1) / (ng * r);
}

bool protected_channel(const qstate_config* c, int h, int k) {
  if (c->map_mode == QS_MAP_NONE) return false;
  if (c->map_mode == QS_MAP_HEAD) return c->map[h] != 0;
  return c->map[(size_t)h * (size_t)c->dk + (size_t)k] != 0;
}

qs_status validate(const qstate_config* c) {
  if (!c) return fail(QS_EINVAL, "config is NULL");
  if (c->abi_version != QSTATE_ABI_VERSION)
    return fail(QS_EINVAL, "abi_version %u, library expects %u", c->abi_version, QSTATE_ABI_VERSION);
  if (c->kind != QS_KIND_ADDITIVE && c->kind != QS_KIND_DELTA) return fail(QS_EINVAL, "kind %d", c->kind);
  if (c->decay_mode != QS_DECAY_HEAD && c->decay_mode != QS_DECAY_KEY)
    return fail(QS_EINVAL, "decay_mode %d", c->decay_mode);
  if (c->B < 0) return fail(QS_EINVAL, "B = %d", c->B);
  if (c->H < 1) return fail(QS_EINVAL, "H = %d", c->H);
  if (c->dk < 1 || c->dv < 1) return fail(QS_EINVAL, "dk = %d, dv = %d", c->dk, c->dv);
  if (c->dk != 64 && c->dk != 128 && c->dk != 256)
    return fail(QS_EUNSUPPORTED, "dk = %d (supported: 64, 128, 256)", c->dk);
  if (c->dv > 256) return fail(QS_EUNSUPPORTED, "dv = %d (supported: 1..256)", c->dv);
  if (c->qbits != 8 && c->qbits != 4) return fail(QS_EUNSUPPORTED, "qbits = %d (supported: 4, 8)", c->qbits);
  if (c->hp_dtype != QS_FP32 && c->hp_dtype != QS_BF16 && c->hp_dtype != QS_FP16)
    return fail(QS_EINVAL, "hp_dtype %d", c->hp_dtype);
  if (c->map_mode != QS_MAP_NONE && c->map_mode != QS_MAP_HEAD && c->map_mode != QS_MAP_KEY)
    return fail(QS_EINVAL, "map_mode %d", c->map_mode);
  if (c->map_mode != QS_MAP_NONE && !c->map) return fail(QS_EINVAL, "map is NULL with map_mode %d", c->map_mode);
  if (c->in_dtype != QS_FP32 && c->in_dtype != QS_BF16)
    return fail(c->in_dtype == QS_FP16 ? QS_EUNSUPPORTED : QS_EINVAL, "in_dtype %d (supported: fp32, bf16)",
                c->in_dtype);
  if (c->rounding != QS_ROUND_NEAREST && c->rounding != QS_ROUND_STOCHASTIC)
    return fail(QS_EINVAL, "rounding %d", c->rounding);
  if (c->rounding == QS_ROUND_STOCHASTIC && c->sr_bits != 16 && c->sr_bits != 8)
    return fail(QS_EUNSUPPORTED, "sr_bits = %d (supported: 8, 16)", c->sr_bits);
  if (c->bdr != 0 && c->bdr != 1) return fail(QS_EINVAL, "bdr %d", c->bdr);
  if (!std::isfinite(c->bdr_bound) || c->bdr_bound < 0.0f) return fail(QS_EINVAL, "bdr_bound %g", c->bdr_bound);
  if (c->lrb_rank < 0) return fail(QS_EINVAL, "lrb_rank %d", c->lrb_rank);
  if (c->lrb_rank > 0) {
    if (c->lrb_rank > kMaxRank) return fail(QS_EUNSUPPORTED, "lrb_rank %d (max %d)", c->lrb_rank, kMaxRank);
    if (c->map_mode != QS_MAP_NONE) return fail(QS_EUNSUPPORTED, "low-rank bypass needs map_mode NONE");
    if (c->lrb_period < 1) return fail(QS_EINVAL, "lrb_period %d", c->lrb_period);
    if (!std::isfinite(c->lrb_theta) || c->lrb_theta <= 0.0f) return fail(QS_EINVAL, "lrb_theta %g", c->lrb_theta);
  }
  if ((c->scale_dtype != QS_FP32 && c->scale_dtype != QS_BF16) || (c->lrb_dtype != QS_FP32 && c->lrb_dtype != QS_BF16))
    return fail(c->scale_dtype == QS_FP16 || c->lrb_dtype == QS_FP16 ? QS_EUNSUPPORTED : QS_EINVAL,
                "scale_dtype %d, lrb_dtype %d (supported: fp32, bf16)", c->scale_dtype, c->lrb_dtype);
  if (c->scale_axis != QS_AXIS_VALUE && c->scale_axis != QS_AXIS_KEY && c->scale_axis != QS_AXIS_HEAD)
    return fail(QS_EINVAL, "scale_axis %d", c->scale_axis);
  if (c->scale_axis != QS_AXIS_VALUE &&
      (c->map_mode != QS_MAP_NONE || c->lrb_rank != 0 || c->scale_dtype != QS_FP32))
    return fail(QS_EUNSUPPORTED, "key-axis and per-head scales: map NONE, no low-rank bypass, fp32 scales");
  if (c->scale_dtype == QS_BF16 || c->lrb_dtype == QS_BF16) {
    // the bf16 layout is the one of int4 states with the low-rank bypass:
    // bf16 scales and bf16 buffer factors together, rank bound 8
    if (c->lrb_rank == 0 || c->scale_dtype != c->lrb_dtype)
      return fail(QS_EUNSUPPORTED, "bf16 scales and bf16 buffer factors come together, with the low-rank bypass");
    if (c->lrb_rank > 8) return fail(QS_EUNSUPPORTED, "bf16 buffer factors: lrb_rank %d (max 8)", c->lrb_rank);
  }
  return QS_OK;
}

qs_status make_plan(const qstate_config* c, Plan* p) {
  qs_status s = validate(c);
  if (s != QS_OK) return s;
  const int H = c->H, dk = c->dk, dv = c->dv;
  const uint64_t hpb = c->hp_dtype == QS_FP32 ? 4u : 2u;
  p->code_off.assign(H, 0);
  p->hp_off.assign(H, 0);
  p->nq.assign(H, 0);
  p->head_type.assign(H, qs::kHeadQuant);
  p->slots.assign((size_t)H * dk, 0);
  uint64_t coff = 0, hoff = 0;
  bool any_mixed = false;
  for (int h = 0; h < H; ++h) {
    int iq = 0, ip = 0;
    for (int k = 0; k < dk; ++k) {
      if (protected_channel(c, h, k)) p->slots[(size_t)h * dk + k] = (uint16_t)(qs::kSlotProt | ip++);
      else p->slots[(size_t)h * dk + k] = (uint16_t)iq++;
    }
    p->nq[h] = iq;
    p->head_type[h] = iq == dk ? qs::kHeadQuant : (iq == 0 ? qs::kHeadProt : qs::kHeadMixed);
    any_mixed = any_mixed || p->head_type[h] == qs::kHeadMixed;
    p->code_off[h] = coff;
    p->hp_off[h] = hoff;
    coff += round16((uint64_t)dv * code_row((uint64_t)iq, (uint64_t)c->qbits));
    hoff += round16((uint64_t)dv * hp_row((uint64_t)ip, hpb));
  }
  p->code_bstride = coff;
  p->hp_bstride = hoff;
  const uint64_t B = (uint64_t)c->B, BH = B * (uint64_t)H, r = (uint64_t)c->lrb_rank;
  p->sizes.codes = B * coff;
  p->sizes.hp = B * hoff;
  const uint64_t sb = c->scale_dtype == QS_BF16 ? 2u : 4u, lb = c->lrb_dtype == QS_BF16 ? 2u : 4u;
  const uint64_t G = c->scale_axis == QS_AXIS_KEY ? (uint64_t)dk : (c->scale_axis == QS_AXIS_HEAD ? 1u : (uint64_t)dv);
  p->sizes.scales = BH * G * sb;
  p->sizes.lrb_W = BH * (uint64_t)dv * r * lb;
  p->sizes.lrb_U = BH * (uint64_t)dk * r * lb;
  p->sizes.lrb_n = r > 0 ? BH * 4u : 0u;

  dense_shape(c->kind, dk, dv, &p->dense_lpr, &p->dense_rpl, &p->dense_threads, &p->row_chunks);
  if (c->scale_axis != QS_AXIS_VALUE) {
    // key-axis or per-head groups: one workgroup per head, two passes
    p->family = qs::kFamGrouped;
  } else if (c->lrb_rank > 0) {
    // one workgroup per head; the buffer and the head's vectors live in
    // static LDS
    p->family = qs::kFamLrb;
  } else if (c->map_mode == QS_MAP_KEY) {
    // key-channel maps (16-bit or fp32 protected values): rows in storage
    // order, 8 lanes per row, each with dk/8 code slots and keymap_eh
    // protected slots, keymap_rpl rows per lane group (4 lanes per row
    // measured slower)
    p->family = qs::kFamKeymap;
    p->dense_lpr = 8;
    p->dense_rpl = 1;
    p->dense_threads = 256;
    int maxhp = 0;
    for (int h = 0; h < H; ++h) maxhp = std::max(maxhp, dk - p->nq[h]);
    p->keymap_eh = 2;
    while (p->keymap_eh * p->dense_lpr < maxhp) p->keymap_eh *= 2;
    int krpl = env_int("QSTATE_KEYMAP_RPL", dv > 32 ? 2 : 1);
    if (krpl != 1 && krpl != 2) krpl = dv > 32 ? 2 : 1;
    p->keymap_rpl = krpl;
    const int rows = 256 / p->dense_lpr * krpl;
    p->row_chunks = (dv + rows - 1) / rows;
  } else if (c->map_mode == QS_MAP_HEAD && H > 256) {
    // head maps over more than 256 heads run the LDS-staged kernel; the dense
    // kernel handles whole-head maps with 16-bit or fp32 protected heads
    // (addressed from a 256-bit head mask in the kernel arguments)
    p->family = qs::kFamMixed;
    uint64_t mx = 0;
    for (int h = 0; h < H; ++h) {
      const uint64_t cb = round16((uint64_t)dv * code_row((uint64_t)p->nq[h], (uint64_t)c->qbits));
      const uint64_t hb = round16((uint64_t)dv * hp_row((uint64_t)(dk - p->nq[h]), hpb));
      mx = std::max(mx, cb + hb);
    }
    p->lds = (uint32_t)std::min<uint64_t>(mx, 0xFFFFFFFFu);
    // stochastic rounding of mixed heads: each lane draws the random bits of
    // a contiguous slot run (one Philox block per 8 or 16 slots) into LDS,
    // 16 bits per slot for the 32 row groups, and gathers its own slots'
    // bits from there; when that does not fit, one block per element
    const uint64_t rb = c->rounding == QS_ROUND_STOCHASTIC ? 32ull * (uint64_t)dk * 2ull : 0ull;
    if (rb > 0 && (uint64_t)p->lds + rb <= kMaxLds) {
      p->rbuf = (uint32_t)rb;
      p->lds += (uint32_t)rb;
    }
    (void)any_mixed;
  } else {
    p->family = qs::kFamDense;
    for (int h = 0; h < H && h < 256; ++h)
      if (p->head_type[h] == qs::kHeadProt) p->prot_mask[h >> 6] |= 1ull << (h & 63);
    p->code_hblk = round16((uint64_t)dv * code_row((uint64_t)dk, (uint64_t)c->qbits));
    p->hp_hblk = round16((uint64_t)dv * hp_row((uint64_t)dk, hpb));
  }
  if (p->lds > kMaxLds)
    return fail(QS_EUNSUPPORTED, "a head needs %u bytes of LDS staging (max %u)", p->lds, kMaxLds);
  const bool chunked = p->family == qs::kFamDense || p->family == qs::kFamKeymap;   // others: one group per head
  const uint64_t grid = BH * (chunked ? (uint64_t)p->row_chunks : 1u);
  if (grid > 0x7FFFFFFFu) return fail(QS_EUNSUPPORTED, "B*H too large for one launch");
  // the kernels form Philox block counters in 32 bits: element indices
  // B*H*dv*dk must stay below 2^35
  if (BH * (uint64_t)dv * (uint64_t)dk >= (1ull << 35))
    return fail(QS_EUNSUPPORTED, "B*H*dv*dk = %llu elements (limit 2^35 per call)",
                (unsigned long long)(BH * (uint64_t)dv * (uint64_t)dk));
  return QS_OK;
}

int rnd_code(const qstate_config* c) {
  if (c->rounding == QS_ROUND_NEAREST) return 0;
  return c->sr_bits == 16 ? 1 : 2;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1u)) == 0u; }

}  // namespace

struct qstate_handle {
  qstate_config cfg{};
  std::vector<uint8_t> map;
  Plan plan;
  void* dev = nullptr;   // one device allocation holding the tables
  qs::DevTables t{};
  int device = -1;
  int rnd = 0;
  std::string kname;
};

namespace {

qs_status check_tensors(const qstate_handle* h, const qstate_tensors* st) {
  if (!st) return fail(QS_EINVAL, "state tensors are NULL");
  const qstate_sizes& z = h->plan.sizes;
  if (z.codes && (!st->codes || !aligned(st->codes, 16))) return fail(QS_EINVAL, "codes NULL or not 16-byte aligned");
  if (z.scales && (!st->scales || !aligned(st->scales, 16))) return fail(QS_EINVAL, "scales NULL or not 16-byte aligned");
  if (z.hp && (!st->hp || !aligned(st->hp, 16))) return fail(QS_EINVAL, "hp NULL or not 16-byte aligned");
  if (z.lrb_W && (!st->lrb_W || !aligned(st->lrb_W, 16))) return fail(QS_EINVAL, "lrb_W NULL or not 16-byte aligned");
  if (z.lrb_U && (!st->lrb_U || !aligned(st->lrb_U, 16))) return fail(QS_EINVAL, "lrb_U NULL or not 16-byte aligned");
  if (z.lrb_n && (!st->lrb_n || !aligned(st->lrb_n, 4))) return fail(QS_EINVAL, "lrb_n NULL or misaligned");
  return QS_OK;
}

qs_status check_device(const qstate_handle* h) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QS_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev != h->device) return fail(QS_EINVAL, "handle was made on device %d, current device is %d", h->device, dev);
  return QS_OK;
}

qs::Args base_args(const qstate_handle* h, const qstate_tensors* st) {
  qs::Args a{};
  const qstate_config& c = h->cfg;
  a.codes = reinterpret_cast<uint8_t*>(st->codes);
  a.scales = reinterpret_cast<float*>(st->scales);   // bf16 elements when scale_bf16
  a.hp = reinterpret_cast<uint8_t*>(st->hp);
  a.W = reinterpret_cast<float*>(st->lrb_W);          // bf16 elements when lrb_bf16
  a.U = reinterpret_cast<float*>(st->lrb_U);
  a.n = st->lrb_n;
  a.B = c.B;
  a.H = c.H;
  a.dk = c.dk;
  a.dv = c.dv;
  a.code_bstride = h->plan.code_bstride;
  a.hp_bstride = h->plan.hp_bstride;
  a.t = h->t;
  a.row_chunks = h->plan.row_chunks;
  a.dense_rpl = h->plan.dense_rpl;
  a.dense_lpr = h->plan.dense_lpr;
  a.keymap_eh = h->plan.keymap_eh;
  a.keymap_rpl = h->plan.keymap_rpl;
  a.load_prio = env_int("QSTATE_LOAD_PRIO", 1) ? 1 : 0;
  a.dense_threads = h->plan.dense_threads;
  for (int w = 0; w < 4; ++w) a.prot_mask[w] = h->plan.prot_mask[w];
  a.code_hblk = h->plan.code_hblk;
  a.hp_hblk = h->plan.hp_hblk;
  a.hp_dtype = c.hp_dtype == QS_FP32 ? 0 : (c.hp_dtype == QS_BF16 ? 1 : 2);
  a.in_bf16 = c.in_dtype == QS_BF16 ? 1 : 0;
  a.decay_key = c.decay_mode == QS_DECAY_KEY ? 1 : 0;
  a.rounding = c.rounding;
  a.sr_bits = c.sr_bits;
  a.bdr = c.bdr;
  a.bdr_bound = c.bdr_bound;
  a.lrb_rank = c.lrb_rank;
  a.lrb_period = c.lrb_period;
  a.lrb_theta = c.lrb_theta;
  a.qbits = c.qbits;
  a.seed_lo = (uint32_t)c.seed;
  a.seed_hi = (uint32_t)(c.seed >> 32);
  a.mixed_lds = h->plan.lds;
  a.mixed_rbuf = h->plan.rbuf;
  a.bf16_layout = c.lrb_dtype == QS_BF16 ? 1 : 0;
  a.scale_axis = c.scale_axis;
  a.nslots = c.B;
  return a;
}

}  // namespace

extern "C" {

qs_status qstate_plan(const qstate_config* cfg, qstate_sizes* sizes) {
  if (!sizes) return fail(QS_EINVAL, "sizes is NULL");
  Plan p;
  qs_status s = make_plan(cfg, &p);
  if (s != QS_OK) return s;
  *sizes = p.sizes;
  return ok();
}

qs_status qstate_init(const qstate_config* cfg, qstate_handle** out, qstate_sizes* sizes) {
  if (!out) return fail(QS_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  qstate_handle* h = new (std::nothrow) qstate_handle();
  if (!h) return fail(QS_ENOMEM, "host allocation failed");
  qs_status s = make_plan(cfg, &h->plan);
  if (s != QS_OK) {
    delete h;
    return s;
  }
  h->cfg = *cfg;
  if (cfg->map_mode != QS_MAP_NONE) {
    const size_t n = cfg->map_mode == QS_MAP_HEAD ? (size_t)cfg->H : (size_t)cfg->H * (size_t)cfg->dk;
    h->map.assign(cfg->map, cfg->map + n);
  }
  h->cfg.map = h->map.empty() ? nullptr : h->map.data();
  h->rnd = rnd_code(cfg);
  h->kname = qs::step_kernel_name(h->plan.family, cfg->qbits, h->rnd, cfg->kind == QS_KIND_DELTA, cfg->dk);

  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return fail(QS_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  const size_t H = (size_t)cfg->H, dk = (size_t)cfg->dk;
  const size_t off_codes = 0, off_hp = off_codes + 8 * H, off_nq = off_hp + 8 * H;
  const size_t off_type = off_nq + 4 * H, off_slots = (off_type + H + 15) & ~size_t(15);
  const size_t total = off_slots + 2 * H * dk;
  std::vector<uint8_t> host(total, 0);
  std::memcpy(host.data() + off_codes, h->plan.code_off.data(), 8 * H);
  std::memcpy(host.data() + off_hp, h->plan.hp_off.data(), 8 * H);
  std::memcpy(host.data() + off_nq, h->plan.nq.data(), 4 * H);
  std::memcpy(host.data() + off_type, h->plan.head_type.data(), H);
  std::memcpy(host.data() + off_slots, h->plan.slots.data(), 2 * H * dk);
  e = hipMalloc(&h->dev, total);
  if (e != hipSuccess) {
    delete h;
    return fail(e == hipErrorOutOfMemory ? QS_ENOMEM : QS_EHIP, "hipMalloc: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(h->dev, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(h->dev);
    delete h;
    return fail(QS_EHIP, "hipMemcpy: %s", hipGetErrorString(e));
  }
  uint8_t* d = reinterpret_cast<uint8_t*>(h->dev);
  h->t.code_off = reinterpret_cast<uint64_t*>(d + off_codes);
  h->t.hp_off = reinterpret_cast<uint64_t*>(d + off_hp);
  h->t.nq = reinterpret_cast<int32_t*>(d + off_nq);
  h->t.head_type = d + off_type;
  h->t.slots = reinterpret_cast<uint16_t*>(d + off_slots);
  if (sizes) *sizes = h->plan.sizes;
  *out = h;
  return ok();
}

qs_status qstate_quantize(qstate_handle* h, const float* S, const qstate_tensors* dst, uint64_t step,
                          void* stream) {
  if (!h) return fail(QS_EINVAL, "handle is NULL");
  qs_status s = check_tensors(h, dst);
  if (s != QS_OK) return s;
  if (h->cfg.B == 0) return ok();
  if (!S || !aligned(S, 16)) return fail(QS_EINVAL, "S NULL or not 16-byte aligned");
  if ((s = check_device(h)) != QS_OK) return s;
  qs::Args a = base_args(h, dst);
  a.S = S;
  a.step_lo = (uint32_t)step;
  a.step_hi = (uint32_t)(step >> 32);
  hipError_t e = qs::launch_quantize(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QS_EHIP, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

qs_status qstate_decode_step(qstate_handle* h, const qstate_tensors* state, const qstate_inputs* in,
                             float* out, uint64_t step, void* stream) {
  if (!h) return fail(QS_EINVAL, "handle is NULL");
  qs_status s = check_tensors(h, state);
  if (s != QS_OK) return s;
  if (!in) return fail(QS_EINVAL, "inputs are NULL");
  if (h->cfg.B == 0) return ok();
  if (!in->q || !in->k || !in->v || !in->decay) return fail(QS_EINVAL, "q, k, v or decay is NULL");
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->v, 16) || !aligned(in->decay, 16))
    return fail(QS_EINVAL, "q, k, v and decay must be 16-byte aligned");
  if (in->beta && !aligned(in->beta, 4)) return fail(QS_EINVAL, "beta misaligned");
  if (!out || !aligned(out, 4)) return fail(QS_EINVAL, "out NULL or misaligned");
  if ((s = check_device(h)) != QS_OK) return s;
  qs::Args a = base_args(h, state);
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.decay = in->decay;
  a.beta = in->beta;
  a.out = out;
  a.step_lo = (uint32_t)step;
  a.step_hi = (uint32_t)(step >> 32);
  hipError_t e = qs::launch_step(h->plan.family, h->cfg.qbits, h->rnd, h->cfg.kind == QS_KIND_DELTA, a,
                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QS_EHIP, "step launch: %s", hipGetErrorString(e));
  return ok();
}

qs_status qstate_decode_step_batch(qstate_handle* h, const qstate_tensors* pool, const qstate_inputs* in,
                                   float* out, int32_t n, const int32_t* slot, const uint64_t* step,
                                   void* stream) {
  if (!h) return fail(QS_EINVAL, "handle is NULL");
  qs_status s = check_tensors(h, pool);
  if (s != QS_OK) return s;
  if (!in) return fail(QS_EINVAL, "inputs are NULL");
  if (n < 0 || n > h->cfg.B) return fail(QS_EINVAL, "batch size %d (pool of %d states)", n, h->cfg.B);
  if (n == 0) return ok();
  if (!slot || !aligned(slot, 4)) return fail(QS_EINVAL, "slot NULL or misaligned");
  if (!step || !aligned(step, 8)) return fail(QS_EINVAL, "step NULL or misaligned");
  if (!in->q || !in->k || !in->v || !in->decay) return fail(QS_EINVAL, "q, k, v or decay is NULL");
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->v, 16) || !aligned(in->decay, 16))
    return fail(QS_EINVAL, "q, k, v and decay must be 16-byte aligned");
  if (in->beta && !aligned(in->beta, 4)) return fail(QS_EINVAL, "beta misaligned");
  if (!out || !aligned(out, 4)) return fail(QS_EINVAL, "out NULL or misaligned");
  if ((s = check_device(h)) != QS_OK) return s;
  qs::Args a = base_args(h, pool);
  a.B = n;                 // the grid covers the batch; the state is addressed through slot
  a.nslots = h->cfg.B;
  a.slot = slot;
  a.seq_step = step;
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.decay = in->decay;
  a.beta = in->beta;
  a.out = out;
  hipError_t e = qs::launch_step(h->plan.family, h->cfg.qbits, h->rnd, h->cfg.kind == QS_KIND_DELTA, a,
                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QS_EHIP, "batch step launch: %s", hipGetErrorString(e));
  return ok();
}

qs_status qstate_dequantize(qstate_handle* h, const qstate_tensors* src, float* S, void* stream) {
  if (!h) return fail(QS_EINVAL, "handle is NULL");
  qs_status s = check_tensors(h, src);
  if (s != QS_OK) return s;
  if (h->cfg.B == 0) return ok();
  if (!S || !aligned(S, 16)) return fail(QS_EINVAL, "S NULL or not 16-byte aligned");
  if ((s = check_device(h)) != QS_OK) return s;
  qs::Args a = base_args(h, src);
  a.S_out = S;
  hipError_t e = qs::launch_dequantize(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QS_EHIP, "dequantize launch: %s", hipGetErrorString(e));
  return ok();
}

qs_status qstate_build_map(const float* stat, int32_t groups, int32_t per_group, float frac, uint8_t* map) {
  if (!stat || !map) return fail(QS_EINVAL, "stat or map is NULL");
  if (groups < 0 || per_group < 1) return fail(QS_EINVAL, "groups %d, per_group %d", groups, per_group);
  if (!(frac >= 0.0f && frac <= 1.0f)) return fail(QS_EINVAL, "frac %g not in [0,1]", frac);
  const int32_t count = (int32_t)std::floor((double)frac * (double)per_group + 0.5);
  std::vector<int32_t> idx((size_t)per_group);
  for (int32_t g = 0; g < groups; ++g) {
    const float* s = stat + (size_t)g * per_group;
    for (int32_t i = 0; i < per_group; ++i)
      if (std::isnan(s[i])) return fail(QS_EINVAL, "stat[%d] is NaN", g * per_group + i);
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [s](int32_t x, int32_t y) { return s[x] < s[y]; });
    uint8_t* m = map + (size_t)g * per_group;
    std::fill(m, m + per_group, 0);
    for (int32_t i = 0; i < count; ++i) m[idx[(size_t)i]] = 1;
  }
  return ok();
}

void qstate_destroy(qstate_handle* h) {
  if (!h) return;
  if (h->dev) (void)hipFree(h->dev);
  delete h;
}

const char* qstate_strerror(qs_status s) {
  switch (s) {
    case QS_OK: return "ok";
    case QS_EINVAL: return "invalid argument";
    case QS_EUNSUPPORTED: return "unsupported configuration";
    case QS_ENOMEM: return "out of memory";
    case QS_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* qstate_last_error(void) { return g_last_error.c_str(); }

const char* qstate_kernel_name(const qstate_handle* h) { return h ? h->kname.c_str() : ""; }

}  // extern "C"
