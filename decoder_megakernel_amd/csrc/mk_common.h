// Definitions shared by the host side (mk_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

constexpr int kThreads = 512;            // threads per workgroup (8 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxT = MK_MAX_T;          // verify rows the LDS budget is sized for
constexpr int kXPad = 8;                 // LDS row padding of activation operands (elements)
constexpr int kBarriers = 11;            // grid barrier slots of one layer launch (trace stamps)
constexpr int kTraceX = 16;              // extra per-workgroup timestamps (sub-phase marks)
constexpr int kTraceStride = 2 + 2 * kBarriers + kTraceX;
constexpr int kLdsBytes = 160 * 1024 - 256;
constexpr int kMaxTopK = 16;
constexpr int kIdxCtrStride = 64;        // words between two rows' top-k part counters (two each)
constexpr int kGateCnt = 128;            // index of the first of 8 gate/up ticket counters in att_cnt,
constexpr int kCntStride = 64;           // which sit 256 bytes apart (device-scope atomics on one
                                         // line are serialised where they are performed)
constexpr int kDownCnt = kGateCnt + 8 * kCntStride;   // the 8 down-projection ticket counters
constexpr int kSlotCnt = kDownCnt + 8 * kCntStride;   // per-slot gate/up completion counters,
constexpr int kSlotStride = 16;                       // 64 bytes apart
constexpr int kMaxSlots = MK_MAX_T * kMaxTopK + 8;
constexpr int kCntWords = kSlotCnt + kSlotStride * kMaxSlots;   // words of the counter area
constexpr int kMaxExperts = 1024;        // routed experts per layer (16 logits per lane)
constexpr int kStageCh = 18;             // float4s per lane when staging one activation row
constexpr int kMaxStageK = kStageCh * 64 * 4;   // longest activation row (elements)
constexpr int kNormCh = 16;              // float4s per lane when normalising one hidden row
constexpr int kMaxModel = kNormCh * 64 * 4;     // longest hidden row (d_model)

// Packed tile geometry: one tile = 16 rows x kTileK[fmt] columns = 1 KiB,
// lane l holds row (l % 16) and 16 consecutive bytes of columns
// (l / 16) * (kTileK / 4) ... ; tiles of a matrix are row-tile major.
// MXFP4 tiles hold 16 rows x 128 columns of 4-bit codes: lane l's 16 bytes are
// the 32 elements (one MX scale group) of row l % 16 at columns (l / 16) * 32.
__host__ __device__ constexpr int tile_k(int fmt) {
  return fmt == MK_FMT_F32 ? 16 : (fmt == MK_FMT_BF16 ? 32 : (fmt == MK_FMT_FP8_B128 ? 64 : 128));
}
// Bytes per element in the tiles (MXFP4: two elements per byte, see launch_pack).
__host__ __device__ constexpr int elem_bytes(int fmt) { return fmt == MK_FMT_F32 ? 4 : (fmt == MK_FMT_BF16 ? 2 : 1); }
// Formats whose tiles carry scales: fp8 (fp32 per 128x128 block) and MXFP4 (E8M0 per 32 elements of a row).
// Bytes of one KV cache row of kvw values (fp8 rows: codes, fp32 scale, padding to 16).
__host__ __device__ constexpr int kv_row_bytes(int fmt, int kvw) {   // kvw: values per row
  return fmt == MK_FMT_FP8_ROW ? (kvw + 4 + 15) / 16 * 16 : kvw * (fmt == MK_FMT_F32 ? 4 : 2);
}
__host__ __device__ constexpr bool scaled_fmt(int fmt) { return fmt == MK_FMT_FP8_B128 || fmt == MK_FMT_MXFP4; }

// Per-layer device state (persistent across steps; zeroed at init).
// The grid barrier is two-level: workgroups arrive on the counter of their
// group (the workgroups of one XCD, b % 8, when the grid is a multiple of 8;
// else kBarGroup consecutive workgroups); the last of a group arrives on
// `top`; the last group leader advances `gen`, which releases everyone.  The
// 32-bit counters only grow (wrapping), and every barrier adds a power of two
// to each: the next power of two >= the group size to a group counter (the
// first workgroup of a smaller group adds the missing arrivals), and the next
// power of two >= the number of groups to `top` (group 0's leader adds the
// missing ones).  The last arriver is the one whose addition makes the count a
// multiple of that power, so nothing is reset between barriers or launches
// (a layer keeps one grouping for its lifetime).
// Fault words (the layer's own, in BarrierState, and a stack's): 0 = none.
constexpr uint32_t kFaultTimeout = 1;      // a bounded wait gave up
constexpr uint32_t kFaultKvRange = 2;      // KV length + T beyond the cache capacity
constexpr uint32_t kFaultToken = 3;        // a token id outside [0, vocab)
constexpr uint32_t kFaultXcd = 4;          // a workgroup found itself on another XCD than its barrier group's
constexpr int kBarGroup = 16;
static_assert((kBarGroup & (kBarGroup - 1)) == 0, "the group size must be a power of two");
constexpr int kMaxBarGroups = 64;        // grids of up to 1024 workgroups
constexpr int kMaxGrid = kBarGroup * kMaxBarGroups;
struct alignas(256) BarrierLine {
  uint32_t n;
  uint32_t pad[63];
};
struct alignas(256) BarrierState {
  uint32_t gen;
  uint32_t pad1[63];
  uint32_t fault;          // kFault* below
  uint32_t pad2[63];
  unsigned long long slots_sum;   // sum over launches of experts streamed (routed distinct + shared)
  unsigned long long launches;    // launches that reached the expert phase
  uint32_t pad3[60];
  BarrierLine top;
  BarrierLine grp[kMaxBarGroups];
};

// Schedule chosen at init for this device and shape.
struct Schedule {
  int nwg;                 // persistent grid (all co-resident)
  int s_q;                 // k-splits of the Q / latent-KV projection
  int grid_min;            // a lower bound of nwg fixed at compile time (0: none)
};
// Instances for fixed layer shapes assume at least this many workgroups (one
// per CU on MI355X), so that choices depending on the grid size fold.
constexpr int kSpecMinGrid = 256;

// Kernel parameters (passed by value).
struct LayerParams {
  // shape
  int d, nh, dh, dc, dr, qw, kvw, nq, E, topk, nshared, f, T;
  int L;                   // cached positions before the step (host value) ...
  const int32_t* L_dev;    // ... or read from device memory when non-null
  float eps, scale;
  double rope_base;
  double rope_step;        // rope_base^(-2 / d_rope): pair i turns by pos * rope_step^i radians
  // tensors
  const float* H;          // [T][d]
  float* out;              // [T][d]
  void* kv;                // [cap][kvw]
  int kv_capacity;         // rows of `kv`
  const float* g1;
  const float* g2;
  const uint8_t* wq;
  const uint8_t* wdkv;
  const uint8_t* wuk;
  const uint8_t* wuv;
  const uint8_t* wo;
  const uint8_t* wr;
  const float* rbias;
  // low-rank query (ql > 0): W_DQ [ql][d], q-norm gain, W_UQ [nq][ql]; latent norm gain (kv_norm)
  int ql, kv_norm;
  const uint8_t* wdq;
  const uint8_t* wuq;
  const float* gq;
  const float* gkv;
  // sparse attention (itopk > 0): indexer heads and key dims, rows kept per query row
  int ihead, idim, itopk;
  int kv_row;                      // values per cache row (kvw, + idim with sparse attention)
  const uint8_t* widx;             // [W_IQ; W_IW; W_IK] tiles
  const uint8_t* const* experts;   // [E + nshared] packed expert blocks
  // packed expert block geometry (bytes)
  long long exp_w13_bytes;         // interleaved W1/W3 tiles
  long long exp_w2_bytes;          // W2 tiles
  // workspace
  float* qkv_part;         // [s_q][T][nq + kvw] (low-rank query: [s_q][T][ql + kvw])
  float* qbuf;             // low-rank query: q [T][nq]
  void* iq;                // sparse: index queries, bf16 [T][ihead][idim]
  float* iw;               // sparse: index head weights [T][ihead]
  float* iscore;           // sparse: index scores [T][idx_max_rows]
  uint16_t* ik16;          // sparse: the scores' order keys, top 16 bits [T][idx_max_rows]
  uint32_t* ihist;         // sparse: the top-k's first-digit histogram of each row [kMaxT][2048]
  uint32_t* ictr;          // sparse: the top-k's part counters [kMaxT][kIdxCtrStride]
  uint32_t* icnt;          // sparse: pairs per part [kMaxT][512]
  uint32_t* icand;         // sparse: (row, 32-bit key) pairs of the parts [kMaxT][idx_max_rows][2]
  int32_t* isel;           // sparse: kept rows [T][itopk], ascending
  int imax;                // sparse: idx_max_rows
  int att_share;           // long contexts may take the four-tile attention units (partials sized for them)
  float* qrope;            // [T][nh][dr]
  float* qabs;             // [T][nh][dc]
  float* att_part;         // [units][16][dc]
  float* att_ml;           // [units][16][2]
  float* z;                // [T][nh][dc]
  float* o;                // [T][nh*dh] in the activation type (fp32 or bf16)
  float* hp;               // [T][d]
  int32_t* route_sel;      // [T][topk]
  float* route_gate;       // [T][topk]
  float* route_cand;       // router candidates: [T][E/16][16] biased logits, then [T][E/16][16] int expert ids
  float* logits;           // [T][E] (written by workgroup 0)
  float* hbuf;             // [slots][T][f] in the expert activation type (fp32 or bf16)
  float* ybuf;             // [slots][T][d]
  const uint8_t* dummy;    // 32 KiB scratch read by the streams' last (discarded) prefetch
  // state
  BarrierState* bar;
  uint32_t* model_fault;   // stack-wide fault word (null for a layer run on its own): a launch
                           // that finds it set does nothing, and one that fails sets it
  uint32_t* att_cnt;       // ticket counters (gate/up at kGateCnt, down at kDownCnt)
  long long* trace;        // [nwg][2 + 2*kBarriers] or null
  long long timeout_ticks; // 100 MHz ticks
  int xcd_release;         // grid barrier groups = XCDs, one L2 write-back per XCD (grid a multiple of 8)
  Schedule sch;
};

}  // namespace mk
