// launch.h -- interface between the C-ABI host layer (damp_api.hip) and the gfx950 kernels
// (step_kernels.hip). Internal to libdamp.so; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace damp {

enum Fmt : int { FMT_F32 = 0, FMT_Q = 1 };  // fp32 state / FP16 + INT8 rows (DAMP, uniform INT8)

// Where one unit's (slot, head) state lives. Unit u = slot * H + head.
//   FMT_F32: fp32 rows at hbase + u * hstride (d x d floats, key rows in original order)
//   FMT_Q:   storage row p < r is FP16 at hbase + u * hstride + 2 p d,
//            storage row p >= r is INT8 at cbase + u * cstride + (p - r) d,
//            with its fp32 scale at sbase + u * sstride + 4 (p - r);
//            rowmap[head * d + p] = the key row held in storage row p (nullptr = identity).
//   contiguous: the three regions of a unit are adjacent (DAMP pool blocks).
//   heads (per-head DAMP layout; nullptr otherwise): heads[h] = {byte offset of head h's block
//     inside a slot, r of head h}; the block of (slot, h) is at hbase + slot * slot_stride +
//     heads[h].x and holds that head's FP16 rows, INT8 rows and scales as above (cbase, sbase,
//     the strides and r are unused). heads_r_or / heads_r_max: bitwise OR and maximum of the
//     heads' r, for the launcher's choice of kernel instance.
struct StateRef {
  uint8_t* hbase;
  uint8_t* cbase;
  uint8_t* sbase;
  int64_t hstride;
  int64_t cstride;
  int64_t sstride;
  int32_t r;
  const uint8_t* rowmap;
  int32_t contiguous;
  const int2* heads;
  int64_t slot_stride;
  int32_t heads_r_or;
  int32_t heads_r_max;
  int32_t num_slots;          // slots in the pool: a slot index outside [0, num_slots) is skipped
};

struct StepArgs {
  StateRef st;
  const int32_t* slot_idx;  // [B]
  int32_t B;
  int32_t H;
  const void* q;            // [B][H][d], fp32 or bf16
  const void* k;
  const void* v;
  const float* alpha;       // [B][H] or [B][H][d]
  const float* beta;        // [B][H]
  float* out;               // [B][H][d]
  int32_t prestep;          // 1: q, k are normalised here and alpha, beta are logits
  uint8_t* win;             // per-window requantization: the window buffers (else nullptr)
  int64_t win_stride;       //   bytes per (slot, head) buffer
  int32_t window;           //   tokens per window, 1 .. 8
  const int32_t* order;     // [B]: workgroups take batch positions in this order (nullptr: 0 .. B-1)
};

struct PackArgs {
  StateRef st;
  const int32_t* slot_idx;  // [n]
  int32_t n;
  int32_t H;
  float* S;                 // [n][H][d][d] fp32, key rows in original order
};

// Each returns hipSuccess or the launch error. d must be 16, 32, 64 or 128 (checked by caller).
hipError_t launch_step(int fmt, int d, int per_key, int bf16, const StepArgs& a, hipStream_t s);
hipError_t launch_quantize(int d, const PackArgs& a, hipStream_t s);
hipError_t launch_dequantize(int d, const PackArgs& a, hipStream_t s);
// Per-window requantization: one token of a window (flush_only = false; q..out as the step) or
// the flush of every listed unit with pending tokens (flush_only = true; B units, no vectors).
hipError_t launch_window(int d, int per_key, int bf16, bool flush_only, const StepArgs& a,
                         hipStream_t s);
int window_max();

// Batch order (order_kernels.hip): order[0..B) = the batch positions by ascending slot bucket,
// bucket = clamp(slot, 0, num_slots - 1) >> order_shift(num_slots), at most kOrderBuckets buckets.
constexpr int kOrderBuckets = 4096;
int order_shift(int32_t num_slots);
hipError_t launch_batch_order(const int32_t* slot_idx, int32_t B, int32_t num_slots, int32_t* order,
                              hipStream_t s);

// STEPQuant-style state (stq_kernels.hip). The block of (slot, head) is at pool + slot *
// slot_stride + heads[head].x; heads[head] = {offset, n16 | n8 << 8 | n6 << 16 | n4 << 24, and
// in .z/.w the bits of the binary64 sum of w_i^2 over the head's integer rows}; rowmap [H][d]
// storage row -> key row; w1 [H][d] row-impact weights in storage order (0 on pivot rows; 1 on
// every integer row of a head whose weights are all 0).
struct StqArgs {
  StepArgs step;            // q, k, v, alpha, beta, out and st.rowmap for the step's staging
  uint8_t* pool;            // source state
  uint8_t* dst;             // destination state (nullptr = in place)
  int64_t slot_stride;
  const int4* heads;
  const float* w1;
  const uint8_t* rowmap;
  const int32_t* slot_idx;
  int32_t num_slots;        // a slot index outside [0, num_slots) is skipped
  int32_t B;                // units = B * H
  int32_t H;
  float* S;                 // pack / unpack: fp32 [B][H][d][d], key rows in original order
  int32_t max_pivots;       // the largest number of pivot rows in one head
};
// mode 0 = decode step, 1 = pack, 2 = unpack; d is 64 or 128.
hipError_t launch_stq(int mode, int d, int per_key, int bf16, const StqArgs& a, hipStream_t s);

// Calibration (calib_kernels.hip). Sizes are validated by the caller: d in {16, 32, 64, 128},
// H * d <= alloc_max_rows(), H * (r_max / g) <= alloc_max_groups(), R % g == 0.
hipError_t launch_risk_scores(int d, const float* S, int32_t n, int32_t H, const float* abar,
                              double* row_err, double* score, hipStream_t s);
hipError_t launch_allocate_rows(const double* score, int32_t H, int32_t d, int64_t R, int32_t g,
                                int32_t r_max, int32_t* r_out, int32_t* map_out, hipStream_t s);
int alloc_max_rows();
int alloc_max_groups();

}  // namespace damp
