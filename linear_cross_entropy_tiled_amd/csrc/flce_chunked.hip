// Generic chunked linear loss: the projection logits = inputs . weight^T is
// formed one block of rows at a time, a caller-supplied function turns each
// logits block into its loss and logits gradient G in place, and the block's
// G is folded back into grad_inputs (G . weight) and grad_weight
// (+= G^T . inputs) with the same contraction kernels as the fused backward.
//
// Method: "Chunked Linear Loss" page ("Why chunk the projection?": the five
// steps per chunk; "Loss function contract": the callback returns the scalar
// loss and a gradient of the logits' shape; "Weight-gradient accumulation
// dtype").  The built-in weighted squared error is the page's "Direct logits
// gradients" example.
#include "flce_device.h"
#include "flce_internal.h"

namespace flce {

// ---------------------------------------------------------------------------
// Logits of one block of rows: L[t][v] = sum_k inputs[t][k] weight[v][k],
// rounded to the input dtype, for t < rows and v < V; 0 elsewhere in the
// block's Np x V_pad buffer (the contractions read the padding).
// One 256 (vocab) x 256 (token) tile per workgroup.
// ---------------------------------------------------------------------------
struct LogitsArgs {
  const char* weight;
  const char* inputs;   // row 0 of the block
  int rows, H, V;
  int ld;               // buffer row stride in elements (V_pad)
  int n_vt, n_tt;
  void* L;
};

__device__ __forceinline__ void store4_t(float* p, const float* c) {
  *reinterpret_cast<f32x4*>(p) = f32x4{c[0], c[1], c[2], c[3]};
}
__device__ __forceinline__ void store4_t(bf16* p, const float* c) {
  bf16x4 v;
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = (bf16)c[j];
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4_t(f16* p, const float* c) {
  f16x4 v;
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = (f16)c[j];
  *reinterpret_cast<f16x4*>(p) = v;
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void chunk_logits_kernel(LogitsArgs a) {
  constexpr int E = sizeof(T);
  const int L = xcd_logical_id(blockIdx.x, gridDim.x);
  int vt, tt;
  grouped_tile(L, a.n_vt, a.n_tt, 4, vt, tt);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int v0 = vt * 256, t0 = tt * 256;
  const uint32_t ld = (uint32_t)a.H * E;
  OperandDesc da;   // weight rows
  da.base = a.weight + (size_t)v0 * ld;
  da.ld_bytes = ld;
  da.nrec = (uint32_t)max(min(a.V - v0, 256), 0) * ld;
  da.cols_valid = 0;
  da.k_bytes = a.H * E;
  OperandDesc db;   // input rows of the block
  db.base = a.inputs + (size_t)t0 * ld;
  db.ld_bytes = ld;
  db.nrec = (uint32_t)max(min(a.rows - t0, 256), 0) * ld;
  db.cols_valid = 0;
  db.k_bytes = a.H * E;
  Acc acc[kMI][kNI];
  zero_acc(acc);
  tile_mainloop<T, true, true>(da, db, (a.H * E + kBKB - 1) / kBKB, grouped_share(vt, tt), acc);

  T* out = reinterpret_cast<T*>(a.L);
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    const int t = t0 + wn * kWaveN + acc_col(ni, lane);
    const bool t_ok = t < a.rows;
#pragma unroll
    for (int mi = 0; mi < kMI; mi++) {
      const int v = v0 + wm * kWaveM + acc_row(mi, 0, lane);
      float c[4];
#pragma unroll
      for (int j = 0; j < 4; j++) c[j] = (t_ok && v + j < a.V) ? acc[mi][ni][j] : 0.0f;
      store4_t(out + (size_t)t * a.ld + v, c);
    }
  }
}

// Zeroes the caller's loss and sets the dlogits scale factors to 1 (the
// callback's gradient is used as it is).
__global__ void chunk_init_kernel(float* loss, float* dscale) {
  if (threadIdx.x == 0) {
    loss[0] = 0.0f;
    dscale[0] = 1.0f;
    dscale[1] = 1.0f;
  }
}

// ---------------------------------------------------------------------------
// Weighted squared error ("Direct logits gradients" example):
//   e = z - y,  w = row_weight[i] feature_weight[j],
//   loss = sum e^2 w,  grad = 2 e w  (rounded to the logits dtype).
// One workgroup per row: the row's loss goes to row_loss[row0 + i]
// (fixed-order tree); a second one-workgroup kernel adds the block's row
// losses to *loss in row order.
// ---------------------------------------------------------------------------
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef f32x4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<f16> { typedef f16x4 type; };

// vec_yf: the target rows and feature_weight allow 16-byte loads.
template <typename T>
__global__ __launch_bounds__(256) void wmse_rows_kernel(T* L, int ld, int V, const float* target, int64_t ld_target,
                                                        const float* row_weight, const float* feature_weight,
                                                        float* row_loss, int64_t row0, int vec_yf) {
  typedef typename Vec4<T>::type V4;
  __shared__ float red[256];
  const int i = blockIdx.x;
  T* z = L + (size_t)i * ld;
  const float* y = target + (size_t)(row0 + i) * ld_target;
  const float rw = row_weight[row0 + i];
  float s = 0.0f;
  for (int v = 4 * threadIdx.x; v < V; v += 4 * 256) {
    if (v + 4 <= V) {
      const V4 zv = *reinterpret_cast<const V4*>(z + v);
      f32x4 yv, fv;
      if (vec_yf) {
        yv = *reinterpret_cast<const f32x4*>(y + v);
        fv = *reinterpret_cast<const f32x4*>(feature_weight + v);
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          yv[j] = y[v + j];
          fv[j] = feature_weight[v + j];
        }
      }
      V4 gv;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float e = (float)zv[j] - yv[j];
        const float w = rw * fv[j];
        s = fmaf(e * e, w, s);
        gv[j] = (T)(2.0f * e * w);
      }
      *reinterpret_cast<V4*>(z + v) = gv;
    } else {
      for (int j = v; j < V; j++) {
        const float e = (float)z[j] - y[j];
        const float w = rw * feature_weight[j];
        s = fmaf(e * e, w, s);
        z[j] = (T)(2.0f * e * w);
      }
    }
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) row_loss[row0 + i] = red[0];
}

__global__ __launch_bounds__(256) void wmse_sum_kernel(const float* row_loss, int64_t row0, int rows, float* loss) {
  __shared__ float red[256];
  float s = 0.0f;
  for (int i = threadIdx.x; i < rows; i += 256) s += row_loss[row0 + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] += red[0];
}

template <typename T>
static void launch_wmse_t(const flce_wmse_args& a, int64_t row0, int rows, int V, void* L, int ld, float* loss,
                          hipStream_t st) {
  const int vec_yf = a.ld_target % 4 == 0 && (reinterpret_cast<uintptr_t>(a.target) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.feature_weight) & 15) == 0;
  wmse_rows_kernel<T><<<rows, 256, 0, st>>>(reinterpret_cast<T*>(L), ld, V, a.target, a.ld_target, a.row_weight,
                                            a.feature_weight, a.row_loss, row0, vec_yf);
  wmse_sum_kernel<<<1, 256, 0, st>>>(a.row_loss, row0, rows, loss);
}

// ---------------------------------------------------------------------------
// The row-block loop.
// ---------------------------------------------------------------------------
template <typename T>
static void launch_chunk_logits_t(const LogitsArgs& a, hipStream_t st) {
  chunk_logits_kernel<T><<<a.n_vt * a.n_tt, kThreads, 0, st>>>(a);
}

int launch_chunked(const ChunkPlan& pl, const void* inputs, const void* weight, flce_chunk_loss_fn fn, void* user,
                   float* loss, void* grad_inputs, void* grad_weight, char* ws, hipStream_t st) {
  float* dscale = reinterpret_cast<float*>(ws + kDscaleOffset);
  chunk_init_kernel<<<1, 64, 0, st>>>(loss, dscale);
  if (hipGetLastError() != hipSuccess) return FLCE_ERR_HIP;
  const char* in = static_cast<const char*>(inputs);
  char* gi = static_cast<char*>(grad_inputs);
  char* Lbuf = ws + pl.b_L;
  const bool gi_f32 = pl.dtype == FLCE_F32;
  if (pl.n_chunks == 0) {
    // no rows: grad_weight is zero (or left as it is when accumulating)
    GwArgs g;
    g.hiddenT = ws + pl.b_xt;
    g.D = Lbuf;
    g.ldD = (int)pl.V_pad;
    g.N = 0;
    g.H = (int)pl.H;
    g.V = (int)pl.V;
    g.N_pad = 0;
    g.cv0 = 0;
    g.n_ht = (int)pl.n_ht;
    g.n_vt_c = (int)pl.n_vt;
    g.gw = grad_weight;
    g.gw_type = pl.gw_dtype;
    g.accumulate = pl.accum_gw ? 1 : 0;
    g.dscale = dscale;
    g.acc32 = nullptr;
    g.mode = 3;
    launch_gw(pl.dtype, g, st);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  for (int c = 0; c < pl.n_chunks; c++) {
    const int64_t r0 = (int64_t)c * pl.rows_c;
    const int rows = (int)(pl.N - r0 < pl.rows_c ? pl.N - r0 : pl.rows_c);
    const int n_tt = (rows + 255) / 256;
    const int Np = n_tt * 256;

    LogitsArgs la;
    la.weight = static_cast<const char*>(weight);
    la.inputs = in + (size_t)r0 * pl.H * pl.esize;
    la.rows = rows;
    la.H = (int)pl.H;
    la.V = (int)pl.V;
    la.ld = (int)pl.V_pad;
    la.n_vt = (int)pl.n_vt;
    la.n_tt = n_tt;
    la.L = Lbuf;
    if (pl.dtype == FLCE_BF16) launch_chunk_logits_t<bf16>(la, st);
    else if (pl.dtype == FLCE_F16) launch_chunk_logits_t<f16>(la, st);
    else launch_chunk_logits_t<float>(la, st);
    if (hipGetLastError() != hipSuccess) return FLCE_ERR_HIP;

    if (fn(user, r0, rows, pl.V, Lbuf, pl.V_pad, pl.dtype, loss, st) != 0) return FLCE_ERR_CALLBACK;

    // grad_inputs[rows] = G . weight, over vocabulary chunks of width Vc
    launch_transpose_hidden(pl.dtype, la.inputs, rows, (int)pl.H, Np, ws + pl.b_xt, st);
    char* gi_blk = gi + (size_t)r0 * pl.H * (gi_f32 ? 4 : pl.esize);
    float* accb = gi_f32 ? reinterpret_cast<float*>(gi_blk) : reinterpret_cast<float*>(ws + pl.b_giacc);
    for (int k = 0; k < pl.n_vchunks; k++) {
      const int cv0 = (int)(k * pl.Vc);
      const int cvn = (int)(pl.V_pad - cv0 < pl.Vc ? pl.V_pad - cv0 : pl.Vc);
      GhArgs h;
      h.weight = static_cast<const char*>(weight);
      h.D = Lbuf + (size_t)cv0 * pl.esize;
      h.ldD = (int)pl.V_pad;
      h.N = rows;
      h.H = (int)pl.H;
      h.V = (int)pl.V;
      h.cv0 = cv0;
      h.cvn = cvn;
      h.n_ht = (int)pl.n_ht;
      h.n_tt = n_tt;
      h.accb = accb;
      h.out = gi_blk;
      h.out_f32 = gi_f32;
      h.mode = pl.n_vchunks == 1 ? 3 : (k == 0 ? 0 : (k == pl.n_vchunks - 1 ? 2 : 1));
      plan_gh_split((int64_t)pl.n_ht * n_tt, cvn, pl.esize, rows, pl.H, &h.parts, &h.kt_per_part);
      h.part = reinterpret_cast<float*>(ws + pl.b_ghpart);
      h.dscale = dscale;
      launch_gh(pl.dtype, h, st);
    }

    // grad_weight (+)= G^T . inputs[rows]
    GwArgs g;
    g.hiddenT = ws + pl.b_xt;
    g.D = Lbuf;
    g.ldD = (int)pl.V_pad;
    g.N = rows;
    g.H = (int)pl.H;
    g.V = (int)pl.V;
    g.N_pad = Np;
    g.cv0 = 0;
    g.n_ht = (int)pl.n_ht;
    g.n_vt_c = (int)pl.n_vt;
    g.gw = grad_weight;
    g.gw_type = pl.gw_dtype;
    g.dscale = dscale;
    g.acc32 = reinterpret_cast<float*>(ws + pl.b_gwacc);
    const bool first = c == 0, last = c == pl.n_chunks - 1;
    if (pl.gw_acc32) {   // fp32 sum over the row blocks, rounded once at the end
      g.mode = first && last ? 3 : (first ? 0 : (last ? 2 : 1));
      g.accumulate = pl.accum_gw ? 1 : 0;
    } else {             // summed in the output buffer (exact for fp32, rounded per block otherwise)
      g.mode = 3;
      g.accumulate = (!first || pl.accum_gw) ? 1 : 0;
    }
    launch_gw(pl.dtype, g, st);
    if (hipGetLastError() != hipSuccess) return FLCE_ERR_HIP;
  }
  return FLCE_OK;
}

int launch_wmse(const flce_wmse_args& a, int64_t row0, int rows, int V, void* L, int ld, int dtype, float* loss,
                hipStream_t st) {
  if (dtype == FLCE_BF16) launch_wmse_t<bf16>(a, row0, rows, V, L, ld, loss, st);
  else if (dtype == FLCE_F16) launch_wmse_t<f16>(a, row0, rows, V, L, ld, loss, st);
  else launch_wmse_t<float>(a, row0, rows, V, L, ld, loss, st);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // namespace flce
