// Host-side internals of libkda: kernel parameter blocks and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// Record a one-line reason for the calling thread's last failure.
int fail(int status, const char* fmt, ...);

// ---------------------------------------------------------------- recurrent
// One pass of the token recurrence on register-resident state tiles; serves
// kda_decode (T_spec = 1) and kda_verify.
struct StepParams {
  const void *q, *k, *v, *g, *beta;
  void* o;                        // NULL: no outputs
  float* pool;
  const int32_t *src_slot, *dst_slot;
  const int32_t* accepted_len;    // NULL: no commit (outputs only) unless commit_all
  int32_t* committed_len_out;
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride;  // per token
  int64_t n_slots;
  int32_t n_seq, T_spec, H;
  int32_t commit_all;             // decode: store after T_spec tokens
  float scale;
};

int launch_step(const StepParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream);
// verify at d = 128 with bf16 inputs and 2..16 tokens on matrix cores
int launch_verify_mfma(const StepParams& p, int out_dtype, hipStream_t stream);

// decode step with the short convolution fused in
struct DecodeConvParams {
  const void *x, *w, *bias, *g, *beta;
  void* cpool;
  void* o;
  float* pool;
  const int32_t *csrc, *cdst, *src_slot, *dst_slot;
  int64_t x_stride, g_stride, beta_stride, o_stride;
  int64_t n_slots, n_cslots;
  int32_t n_seq, H, W, act, qk_l2norm;
  float eps, scale;
  // verify only: tokens per sequence (x, g, beta, o strides are per token)
  // and the commit at the accepted length (NULL: outputs only, no commit)
  int32_t T_spec;
  const int32_t* accepted_len;
  int32_t* committed_len_out;
  // gated RMS norm of the output: NULL ogate = none
  const void* ogate;
  const void* onorm_w;
  int64_t ogate_stride;           // per sequence (decode) or per token (verify)
  float onorm_eps;
};

int launch_decode_conv(const DecodeConvParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream);
int launch_verify_conv(const DecodeConvParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream);
// verify_conv at d = 128 with bf16 inputs and 2..16 tokens on matrix cores
int launch_verify_conv_mfma(const DecodeConvParams& p, int out_dtype, hipStream_t stream);

// ---------------------------------------------------------------- plan
// device-side checkpoint plan (kda_ckpt_plan_device)
struct PlanParams {
  const int32_t *cu, *start_pos, *free_slots;
  int32_t *ckpt_cu, *ckpt_pos, *ckpt_slot, *n_total;
  int64_t T_tot;
  int32_t n_seq, interval, cap, n_free;
};

int launch_plan(const PlanParams& p, hipStream_t stream);

// ---------------------------------------------------------------- conv
struct ConvParams {
  const void* x;
  void* y;
  const void* w;
  const void* bias;
  const int32_t* cu;
  void* pool;
  const int32_t *src_slot, *dst_slot, *adv;
  int64_t x_stride, y_stride, T_tot, n_slots;
  int32_t n_seq, C, W, act;
  int32_t n_tiles;                // body tiles of TT tokens
  // per-head L2 normalisation of the outputs (the prefill's q and k): the
  // channels below norm_channels, in groups of norm_d; norm_d = 0 = none
  int64_t norm_channels;
  int32_t norm_d;
  float norm_eps;
};

int launch_conv(const ConvParams& p, int dtype, hipStream_t stream);

// Conv history at the interval checkpoints of a prefill: checkpoint j of
// sequence s (ckpt_cu[s] <= j < ckpt_cu[s + 1]) at absolute position
// (start / I + 1 + j - ckpt_cu[s]) * I gets the W-1 raw inputs of
// history ++ tokens before it, in conv_pool[ckpt_slot[j]].
struct ConvCkptParams {
  const void* x;
  void* pool;
  const int32_t *cu, *start_pos, *src_slot, *ckpt_cu, *ckpt_slot;
  int64_t x_stride, T_tot, n_slots, n_ckpt;
  int32_t n_seq, C, W, interval;
};
int launch_conv_ckpt(const ConvCkptParams& p, int dtype, hipStream_t stream);

// ---------------------------------------------------------------- prefill
struct PrefillParams {
  const void *q, *k, *v, *g, *beta;
  void* o;
  const int32_t* cu;
  float* pool;
  const int32_t *src_slot, *dst_slot, *start_pos, *ckpt_cu, *ckpt_slot;
  int32_t* ckpt_pos_out;
  void* workspace;
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride;
  int64_t T_tot, n_slots, n_ckpt, workspace_bytes;
  int32_t n_seq, H, chunk, ckpt_interval;
  float scale;
  // segment scan (long sequences): set by launch_prefill
  int32_t segment_len;            // effective length (> 0), or <= 0 = no split
  int32_t mode;                   // kModeFull / kModeLocal / kModeTransition / kModePassA / kModeFixup
  const int32_t* seg_cu;          // [n_seq + 1] first work item of each sequence, or NULL
  const int32_t* blk_cu;          // [n_seq + 1] first workspace block of each sequence
  float* ws_states;               // 3 d x d blocks per head for every block index
  int32_t* ws_zero;               // per block index and head: chunks after which the transition is exactly 0, or -1
  int32_t* item_order;            // work items by decreasing token count (segment plan), or NULL
  int64_t max_items;              // capacity of item_order
  int64_t ws_max_blocks;
};

// work modes of the prefill kernel
enum { kModeFull = 0, kModeLocal = 1, kModeTransition = 2, kModePassA = 3, kModeFixup = 4 };
constexpr int32_t kDefaultSegmentLen = 32768;

int64_t prefill_workspace_bytes(const PrefillParams& p, int D);
int launch_prefill(const PrefillParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream);

}  // namespace kda
