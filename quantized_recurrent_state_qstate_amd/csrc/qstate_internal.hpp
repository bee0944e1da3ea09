// Internal interface between the C-ABI host code and the gfx950 kernels of
// libqstate.  Not installed; the public ABI is include/qstate.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

// Head storage type in the per-head table.
enum HeadType : uint8_t { kHeadQuant = 0, kHeadProt = 1, kHeadMixed = 2 };

// Slot table entry for key channel k of head h: bit 15 set = protected,
// low 15 bits = slot among the head's quantized (or protected) channels.
constexpr uint16_t kSlotProt = 0x8000u;

// Device-side per-head layout tables (one allocation, owned by the handle).
struct DevTables {
  uint64_t* code_off;   // [H] byte offset of the head's code block in a batch element
  uint64_t* hp_off;     // [H] byte offset of the head's protected block
  int32_t* nq;          // [H] quantized channels of the head
  uint8_t* head_type;   // [H] HeadType
  uint16_t* slots;      // [H*dk]
};

// Everything a kernel needs, passed by value as kernel arguments.
struct Args {
  // stored state
  uint8_t* codes;
  float* scales;
  uint8_t* hp;
  float* W;
  float* U;
  int32_t* n;
  // step inputs / outputs
  const void* q;
  const void* k;
  const void* v;
  const float* decay;
  const float* beta;   // may be null
  float* out;
  const float* S;      // quantize input / dequantize output (fp32 logical)
  float* S_out;
  // geometry and tables
  int32_t B, H, dk, dv;
  uint64_t code_bstride, hp_bstride;
  DevTables t;
  int32_t row_chunks;  // dense kernel: work items (row chunks) per head
  int32_t dense_rpl;   // dense kernel: rows per lane (1, 2)
  int32_t dense_threads;  // dense kernel: threads per workgroup (dense_lpr per row group)
  int32_t dense_lpr;   // dense kernel: lanes per row (8, or 4 for dk 128)
  int32_t keymap_eh;   // key-map kernel: protected slots per lane (2, 4, 8, 16)
  int32_t keymap_rpl;  // key-map kernel: rows per lane group (1, 2)
  int32_t load_prio;   // dense kernel: raised wave priority until the loads are issued
  uint64_t prot_mask[4];  // dense kernel: bit h % 64 of word h / 64 set = head h protected (H <= 256)
  uint64_t code_hblk;  // dense kernel: bytes of one quantized head's code block
  uint64_t hp_hblk;    // dense kernel: bytes of one protected head's block
  int32_t hp_dtype;    // 0 fp32, 1 bf16, 2 fp16
  int32_t in_bf16;     // q,k,v are bf16 (else fp32)
  int32_t decay_key;   // decay per key channel (else per head)
  int32_t rounding;    // 0 nearest, 1 stochastic (quantize kernel)
  int32_t sr_bits;
  int32_t bdr;
  float bdr_bound;
  int32_t lrb_rank, lrb_period;
  float lrb_theta;
  int32_t qbits;
  uint32_t seed_lo, seed_hi;
  uint32_t step_lo, step_hi;
  uint32_t mixed_lds;  // mixed kernel: dynamic LDS bytes
  uint32_t mixed_rbuf; // mixed kernel: bytes of LDS for random bits by slot (0: one Philox block per element)
  int32_t bf16_layout; // scales and low-rank buffer factors stored as bf16 (LRB only)
  int32_t scale_axis;  // scale groups: 0 rows (value axis), 1 columns (key axis), 2 the head
  // batched entry point: batch element b reads its inputs and writes its
  // outputs at b, and its state at slot[b] of a pool of nslots states, with
  // its own step; null = the plain step (slot b, step above)
  const int32_t* slot;
  const uint64_t* seq_step;
  int32_t nslots;
};

// One (batch element, head) of a step: index of its inputs and outputs
// (b*H + h), index of its state (slot*H + h), and its step (Philox counter
// word and merge clock).
struct HeadIx {
  uint64_t in, st;
  uint32_t step_lo, step_hi;
};

// Kernel families chosen at init.
enum StepFamily : int { kFamDense = 0, kFamMixed = 1, kFamLrb = 2, kFamKeymap = 3, kFamGrouped = 4 };

// Launchers.  Step kernels, one launcher per family, instantiated per
// (qbits, rounding) in qstate_step_<family>.hip (the low-rank-bypass one per
// kind too, the key-map one per dk); launch_step (qstate_misc.hip) dispatches to them.  Return hipSuccess or the launch error.  `rnd`: 0
// nearest, 1 stochastic 16-bit, 2 stochastic 8-bit.
template <int QB, int RND>
hipError_t launch_dense(int delta, const Args& a, hipStream_t s);
template <int QB, int RND>
hipError_t launch_mixed(int delta, const Args& a, hipStream_t s);
template <int QB, int RND, int DK>
hipError_t launch_keymap(int delta, const Args& a, hipStream_t s);
template <int QB, int RND, int DELTA>
hipError_t launch_lrb(const Args& a, hipStream_t s);
template <int QB, int RND>
hipError_t launch_grouped(int delta, const Args& a, hipStream_t s);
hipError_t launch_step(int family, int qbits, int rnd, int delta, const Args& a,
                       hipStream_t s);
hipError_t launch_quantize(const Args& a, hipStream_t s);
hipError_t launch_dequantize(const Args& a, hipStream_t s);
const char* step_kernel_name(int family, int qbits, int rnd, int delta, int dk);

}  // namespace qs
