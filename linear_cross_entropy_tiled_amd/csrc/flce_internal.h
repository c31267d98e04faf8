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
  bool gw_accum_out;             // one-pass path: sum grad_weight over the blocks in its own dtype
  float scale, cap, z_loss;
  flce_launch_timer* timer;      // optional event pairs around the matrix-core launches (caller-owned)

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

  // one-pass forward + backward (plan_forward_backward): blocks of fb_rows rows
  int64_t fb_rows;               // rows per block, a multiple of 256
  int fb_blocks;
  int64_t fb_Vc;                 // vocabulary chunk of the grad_hidden contraction (32-bit weight offsets)
  int fb_vchunks;
  bool fb_gw_acc32;              // grad_weight summed over the blocks in an fp32 workspace accumulator
  size_t fb_part, fb_blk, fb_coefA, fb_coefB, fb_lseL, fb_tgt, fb_Z, fb_xt, fb_ghacc, fb_gwacc, fb_ghpart,
      fb_gbpart, fb_bytes;
};

// Vocabulary splits of the forward tile kernel for n_tt token tiles: about
// one workgroup per CU.
int forward_splits(int64_t n_tt, int64_t n_vt);
// Fills the fb_* fields of a plan made by make_plan; block_rows 0 = library choice.
int plan_forward_backward(Plan* plan, int64_t block_rows);

// flce_launch_timer: one event pair around a launch.  Nothing without a timer
// or once its capacity is used up; a failed record leaves its error for the
// hipGetLastError that ends every entry point.
inline bool timer_open(const Plan& pl) { return pl.timer && pl.timer->count < pl.timer->capacity; }
inline void time_begin(const Plan& pl, hipStream_t st) {
  if (timer_open(pl)) (void)hipEventRecord(static_cast<hipEvent_t>(pl.timer->events[2 * pl.timer->count]), st);
}
inline void time_end(const Plan& pl, int kernel, hipStream_t st) {
  if (!timer_open(pl)) return;
  flce_launch_timer* t = pl.timer;
  (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * t->count + 1]), st);
  t->kernel[t->count] = kernel;
  t->count++;
}

constexpr size_t kStatusBytes = 256;   // status word at workspace offset 0
// Backward: the dlogits scale factor and its inverse (two fp32 words) follow
// the status word.  Powers of two: 1 except for fp16 dlogits (bwd_prep_kernel).
constexpr size_t kDscaleOffset = 16;
// One-pass forward + backward: two fp32 ones (a unit factor for kernels that
// take a dlogits factor pointer).
constexpr size_t kOnesOffset = 32;

// Partial sums of one finalize block (forward).
struct BlockPart {
  double loss;
  double entropy;
  int n_valid;
  int n_correct;
  int bad_target;
  int pad;
};

// ---------------------------------------------------------------------------
// Gradient contractions, shared by the fused backward (one vocabulary chunk of
// D per launch) and the generic chunked loss (one block of rows per launch).
// D is a [rows][ldD] scratch in the input dtype, zero outside the valid
// rows and columns.
// ---------------------------------------------------------------------------

// grad_weight[v][:] for the vocabulary rows [cv0, cv0 + 256 n_vt_c):
// sum over t < N_pad of D[t][v - cv0] hiddenT[:][t], times dscale[1].
// mode 3: out (+)= C (accumulate), rounded once; with K blocks in several
// launches: mode 0 acc32 = C, 1 acc32 += C, 2 out (+)= acc32 + C.
struct GwArgs {
  const char* hiddenT;   // hidden transposed: [H][N_pad], zero past the valid rows
  const char* D;
  int ldD;
  int N, H, V, N_pad;
  int cv0;
  int n_ht, n_vt_c;
  void* gw;
  int gw_type;      // flce_dtype of grad_weight
  int accumulate;   // add to grad_weight's current contents (modes 2, 3)
  const float* dscale;   // [1]: 2^-s, undoes the factor D is stored with
  float* acc32;     // fp32 V x H accumulator (modes 0-2)
  int mode;
};

// grad_hidden[t][:] = sum over the chunk's vocabulary rows of D[t][v] W[v][:],
// times dscale[1].  mode 0: first of several chunks (store the fp32
// accumulator), 1: middle (accumulator += C), 2: last (out = cast(acc + C)),
// 3: only chunk (out = cast(C)).
struct GhArgs {
  const char* weight;
  const char* D;
  int ldD;
  int N, H, V;
  int cv0, cvn;     // chunk start and padded width
  int n_ht, n_tt;
  float* accb;      // fp32 N x H accumulator (may alias out when out is fp32)
  void* out;
  int out_f32;
  int mode;
  int parts;        // > 1: K split; split p covers stages [p kt_per_part, (p+1) kt_per_part)
  int kt_per_part;
  float* part;      // parts x N x H fp32 partials (parts > 1)
  const float* dscale;   // [1]: 2^-s, undoes the factor D is stored with
};

// hiddenT[h][t] = hidden[t][h] for t < N, 0 for N <= t < N_pad.
void launch_transpose_hidden(int dtype, const void* hidden, int N, int H, int N_pad, void* hiddenT,
                             hipStream_t st);
void launch_gw(int dtype, const GwArgs& g, hipStream_t st);
void launch_gh(int dtype, const GhArgs& h, hipStream_t st);
// grad_hidden K-split planning (parts, 64-row stages per part) for a chunk of
// width cvn over n_tiles output tiles.
void plan_gh_split(int64_t n_tiles, int64_t cvn, int esize, int64_t N, int64_t H, int* parts, int* kt_per_part);

int make_plan(const flce_params* p, Plan* plan);

// Generic chunked loss (flce_chunked_linear_loss): blocks of rows_c rows.
struct ChunkPlan {
  int64_t N, H, V;
  int dtype, gw_dtype, esize;
  bool accum_gw;                 // FLCE_ACCUMULATE_GRAD_WEIGHT
  bool gw_acc32;                 // grad_weight summed over blocks in an fp32 workspace accumulator
  int64_t n_ht, n_vt, V_pad;
  int64_t rows_c;                // rows per block (multiple of 256)
  int n_chunks;
  int64_t Vc;                    // vocabulary chunk of the grad_inputs contraction
  int n_vchunks;
  size_t b_L, b_xt, b_giacc, b_gwacc, b_ghpart, b_bytes;
};

int make_chunk_plan(const flce_chunked_params* p, ChunkPlan* plan);
int launch_chunked(const ChunkPlan& pl, const void* inputs, const void* weight, flce_chunk_loss_fn fn, void* user,
                   float* loss, void* grad_inputs, void* grad_weight, char* ws, hipStream_t st);
int launch_wmse(const flce_wmse_args& a, int64_t row0, int rows, int V, void* L, int ld, int dtype, float* loss,
                hipStream_t st);

void launch_forward_rows(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                         const void* targets, int64_t r0, int rows, int S, float* part, float* loss, float* lse,
                         BlockPart* blk, void* z, int ldz, hipStream_t st);
void launch_forward_scalars(const Plan& pl, const BlockPart* blk, int nblk, float* loss, int64_t* num_correct,
                            float* entropy_sum, int* status, hipStream_t st);
void launch_prep_rows(const Plan& pl, const void* targets, const float* lse, const float* grad_loss, float* coefA,
                      float* coefB, float* lseL, int* tgt, int* status, float* dscale, int64_t row0, int64_t row1,
                      hipStream_t st);
void launch_gb_reduce(int dtype, const float* part, int n_tt, int ld, int V, void* gb, int accumulate,
                      const float* dscale, hipStream_t st);
hipError_t launch_forward_backward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                                   const void* targets, const float* grad_loss, float* loss, float* lse,
                                   int64_t* num_correct, float* entropy_sum, void* grad_hidden, void* grad_weight,
                                   void* grad_bias, char* ws, hipStream_t st);

hipError_t launch_scale_gradients(const Plan& pl, const float* g, void* grad_hidden, void* grad_weight,
                                  void* grad_bias, hipStream_t st);

hipError_t launch_forward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                          const void* targets, float* loss, float* lse, int64_t* num_correct,
                          float* entropy_sum, char* ws, hipStream_t st);

hipError_t launch_backward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                           const void* targets, const float* lse, const float* grad_loss,
                           void* grad_hidden, void* grad_weight, void* grad_bias, char* ws,
                           hipStream_t st);

}  // namespace flce
