// Host-side plan, workspace layout and kernel launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flce.h"

namespace flce {

// Everything the launchers need, derived from flce_params on the host.
struct Plan {
  int64_t N, H, V, ignore_index;
  int dtype, gw_dtype, reduction;
  bool has_bias;
  bool accum_gw, accum_gb;       // backward adds into grad_weight / grad_bias
  bool tgt_i32;                  // targets are int32 (else int64)
  float scale, cap, z_loss;

  int64_t n_tt, n_vt, n_ht;      // 256-wide tiles over tokens, vocabulary, hidden
  int64_t N_pad, V_pad;          // padded to whole tiles
  int esize;                     // bytes per input element

  // forward
  int S;                         // vocabulary splits per token tile
  size_t f_part, f_blk, f_bytes; // workspace offsets / total

  // backward
  int64_t Vc;                    // vocabulary chunk width (multiple of 256)
  int n_chunks;
  int gh_parts;                  // grad_hidden: K (vocabulary) splits per chunk when there are few output tiles
  int gh_kt_per_part;            // 64-row stages per split
  size_t b_coefA, b_coefB, b_lseL, b_tgt, b_D, b_xt, b_ghacc, b_ghpart, b_gbpart, b_bytes;
};

constexpr size_t kStatusBytes = 256;   // status word at workspace offset 0
// Backward: the dlogits scale factor and its inverse (two fp32 words) follow
// the status word.  Powers of two: 1 except for fp16 dlogits (bwd_prep_kernel).
constexpr size_t kDscaleOffset = 16;

// Partial sums of one finalize block (forward).
struct BlockPart {
  double loss;
  double entropy;
  int n_valid;
  int n_correct;
  int bad_target;
  int pad;
};

int make_plan(const flce_params* p, Plan* plan);

hipError_t launch_forward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                          const void* targets, float* loss, float* lse, int64_t* num_correct,
                          float* entropy_sum, char* ws, hipStream_t st);

hipError_t launch_backward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                           const void* targets, const float* lse, const float* grad_loss,
                           void* grad_hidden, void* grad_weight, void* grad_bias, char* ws,
                           hipStream_t st);

}  // namespace flce
