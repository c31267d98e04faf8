// One-pass forward + backward: the row-chunked schedule.  For each block of
// rows, the logit tiles are computed once: their online-softmax state gives
// LSE, the loss and the metrics (exactly as in the forward pass), and the same
// tiles, stored in the input dtype, are turned in place into the logit
// gradient, which the two contractions of the backward pass consume right
// away.  Nothing is recomputed; the upstream gradient must be known up front.
//
// Method: "Chunked Linear Cross-Entropy" page, "Kernel design" (per row chunk:
// logits tile, a fused cross-entropy-and-logits-gradient step that overwrites
// the tile with dlogits, then the input and weight gradients from it) and the
// quack-kernels chunked_linear_cross_entropy_fwd (gradients formed inside the
// forward chunk loop); "Chunked Linear Loss" page, "Weight-gradient
// accumulation dtype" (grad_weight summed over the blocks in fp32, rounded
// once).  Per block of rows [r0, r0 + rows):
//   tiles     z = softcap(scale (x W^T + b)) -> Z (input dtype), split partials;
//   finalize  LSE, per-row loss and metric partials (fp32 state, not Z);
//   prep      c_t, (1 + 2 lam LSE_t) c_t for the block's rows;
//   dlogits   D = scale softcap'(z) (coefA p - [v = t] coefB) over Z, in place,
//             plus the block's per-256-row column sums for grad_bias;
//   gh        grad_hidden[rows] = D W           (written once);
//   gw        grad_weight (+)= D^T x[rows]       (fp32 over the blocks).
#include "flce_device.h"
#include "flce_internal.h"

namespace flce {

__global__ void fb_init_kernel(float* ones) {
  if (threadIdx.x == 0) {
    ones[0] = 1.0f;
    ones[1] = 1.0f;
  }
}

template <typename T> struct Quad;
template <> struct Quad<float> { typedef f32x4 type; };
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<f16> { typedef f16x4 type; };

struct FbDlogitsArgs {
  void* Z;               // the block's logits in, D out: [rows_pad][ldz]
  int ldz;
  int rows, V;           // valid rows of the block; vocabulary
  int64_t r0;            // batch row of the block's row 0
  const float* coefA;    // per batch row (see bwd_prep_kernel)
  const float* coefB;
  const float* lseL;
  const int* tgt;
  float scale, inv_cap;  // inv_cap = 1/cap, 0 without the cap
  const float* dscale;   // [0]: factor D is stored with
  float* gb_part;        // [batch row group][ld_gb]: column sums of D (without the factor)
  int ld_gb;
};

// One 256-row x 256-column patch per workgroup: wave w takes 64 rows, lane l
// four consecutive columns, so every row is read and written as one
// contiguous 512-byte (16-bit types) segment per wave.
template <typename T, bool SOFTCAP>
__global__ __launch_bounds__(256) void fb_dlogits_kernel(FbDlogitsArgs a) {
  typedef typename Quad<T>::type Q;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int v = blockIdx.x * 256 + 4 * lane;
  const int g = blockIdx.y;
  const float ds = a.dscale[0];
  T* Z = reinterpret_cast<T*>(a.Z);
  float cs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  bool vok[4];
#pragma unroll
  for (int j = 0; j < 4; j++) vok[j] = v + j < a.V;
#pragma unroll 4
  for (int i = 0; i < 64; i++) {
    const int tl = g * 256 + w * 64 + i;   // row within the block
    const int64_t tb = a.r0 + tl;          // batch row
    Q* zp = reinterpret_cast<Q*>(Z + (size_t)tl * a.ldz + v);
    const Q zq = *zp;
    const bool row_ok = tl < a.rows;
    const float cA = a.coefA[tb], cB = a.coefB[tb], lL = a.lseL[tb];
    const int tg = a.tgt[tb];
    Q out;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float z = (float)zq[j];
      const float p = fast_exp2(fmaf(z, kLog2e, -lL));
      float d = cA * p - (v + j == tg ? cB : 0.0f);
      if constexpr (SOFTCAP) {
        const float zc = z * a.inv_cap;
        d *= fmaf(-zc, zc, 1.0f);
      }
      d = (row_ok && vok[j]) ? d * a.scale : 0.0f;
      cs[j] += d;
      out[j] = (T)(d * ds);
    }
    *zp = out;
  }
  __shared__ float red[4][256];
#pragma unroll
  for (int j = 0; j < 4; j++) red[w][4 * lane + j] = cs[j];
  __syncthreads();
  if (w == 0) {
    float* dst = a.gb_part + (size_t)(a.r0 / 256 + g) * a.ld_gb + v;
#pragma unroll
    for (int j = 0; j < 4; j++) dst[j] = ((red[0][4 * lane + j] + red[1][4 * lane + j]) + red[2][4 * lane + j]) +
                                         red[3][4 * lane + j];
  }
}

template <typename T>
static void launch_fb_dlogits_t(const FbDlogitsArgs& a, int n_vt, int n_tt, bool softcap, hipStream_t st) {
  const dim3 grid((unsigned)n_vt, (unsigned)n_tt);
  if (softcap) fb_dlogits_kernel<T, true><<<grid, 256, 0, st>>>(a);
  else fb_dlogits_kernel<T, false><<<grid, 256, 0, st>>>(a);
}

hipError_t launch_forward_backward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                                   const void* targets, const float* grad_loss, float* loss, float* lse,
                                   int64_t* num_correct, float* entropy_sum, void* grad_hidden, void* grad_weight,
                                   void* grad_bias, char* ws, hipStream_t st) {
  int* status = reinterpret_cast<int*>(ws);
  float* dscale = reinterpret_cast<float*>(ws + kDscaleOffset);
  float* ones = reinterpret_cast<float*>(ws + kOnesOffset);
  float* part = reinterpret_cast<float*>(ws + pl.fb_part);
  BlockPart* blk = reinterpret_cast<BlockPart*>(ws + pl.fb_blk);
  float* coefA = reinterpret_cast<float*>(ws + pl.fb_coefA);
  float* coefB = reinterpret_cast<float*>(ws + pl.fb_coefB);
  float* lseL = reinterpret_cast<float*>(ws + pl.fb_lseL);
  int* tgt = reinterpret_cast<int*>(ws + pl.fb_tgt);
  char* Z = ws + pl.fb_Z;
  char* xt = ws + pl.fb_xt;
  float* gb_part = reinterpret_cast<float*>(ws + pl.fb_gbpart);
  const int ldz = (int)pl.V_pad;
  const bool gh_f32 = pl.dtype == FLCE_F32;
  const size_t gh_esize = gh_f32 ? 4 : (size_t)pl.esize;
  fb_init_kernel<<<1, 64, 0, st>>>(ones);

  if (pl.fb_blocks == 0) {
    // no rows: loss and metrics from one empty row group; grad_weight and
    // grad_bias zero (or left as they are when accumulating)
    launch_forward_rows(pl, hidden, weight, bias, targets, 0, 0, 1, part, loss, lse, blk, nullptr, 0, st);
    launch_forward_scalars(pl, blk, 1, loss, num_correct, entropy_sum, status, st);
    GwArgs g;
    g.hiddenT = xt;
    g.D = Z;
    g.ldD = ldz;
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
    g.dscale = ones;
    g.acc32 = nullptr;
    g.mode = 3;
    launch_gw(pl.dtype, g, st);
    if (grad_bias)
      launch_gb_reduce(pl.dtype, gb_part, 0, ldz, (int)pl.V, grad_bias, pl.accum_gb ? 1 : 0, ones, st);
    return hipGetLastError();
  }

  for (int b = 0; b < pl.fb_blocks; b++) {
    const int64_t r0 = (int64_t)b * pl.fb_rows;
    const int rows = (int)(pl.N - r0 < pl.fb_rows ? pl.N - r0 : pl.fb_rows);
    const int n_tt = (rows + 255) / 256;
    const int rows_pad = n_tt * 256;
    const int S = forward_splits(n_tt, pl.n_vt);

    // logits of the block (stored) and their softmax state -> LSE, loss, metrics
    launch_forward_rows(pl, hidden, weight, bias, targets, r0, rows, S, part, loss, lse, blk, Z, ldz, st);
    // per-row gradient coefficients of the block's rows
    launch_prep_rows(pl, targets, lse, grad_loss, coefA, coefB, lseL, tgt, status, dscale, r0, r0 + rows_pad, st);

    FbDlogitsArgs d;
    d.Z = Z;
    d.ldz = ldz;
    d.rows = rows;
    d.V = (int)pl.V;
    d.r0 = r0;
    d.coefA = coefA;
    d.coefB = coefB;
    d.lseL = lseL;
    d.tgt = tgt;
    d.scale = pl.scale;
    d.inv_cap = pl.cap > 0 ? 1.0f / pl.cap : 0.0f;
    d.dscale = dscale;
    d.gb_part = gb_part;
    d.ld_gb = ldz;
    if (pl.dtype == FLCE_BF16) launch_fb_dlogits_t<bf16>(d, (int)pl.n_vt, n_tt, pl.cap > 0, st);
    else if (pl.dtype == FLCE_F16) launch_fb_dlogits_t<f16>(d, (int)pl.n_vt, n_tt, pl.cap > 0, st);
    else launch_fb_dlogits_t<float>(d, (int)pl.n_vt, n_tt, pl.cap > 0, st);

    // grad_hidden[rows] = D . weight, over vocabulary chunks of width fb_Vc
    const char* x_blk = static_cast<const char*>(hidden) + (size_t)r0 * pl.H * pl.esize;
    launch_transpose_hidden(pl.dtype, x_blk, rows, (int)pl.H, rows_pad, xt, st);
    char* gh_blk = static_cast<char*>(grad_hidden) + (size_t)r0 * pl.H * gh_esize;
    float* accb = gh_f32 ? reinterpret_cast<float*>(gh_blk) : reinterpret_cast<float*>(ws + pl.fb_ghacc);
    for (int k = 0; k < pl.fb_vchunks; k++) {
      const int cv0 = (int)(k * pl.fb_Vc);
      const int cvn = (int)(pl.V_pad - cv0 < pl.fb_Vc ? pl.V_pad - cv0 : pl.fb_Vc);
      GhArgs h;
      h.weight = static_cast<const char*>(weight);
      h.D = Z + (size_t)cv0 * pl.esize;
      h.ldD = ldz;
      h.N = rows;
      h.H = (int)pl.H;
      h.V = (int)pl.V;
      h.cv0 = cv0;
      h.cvn = cvn;
      h.n_ht = (int)pl.n_ht;
      h.n_tt = n_tt;
      h.accb = accb;
      h.out = gh_blk;
      h.out_f32 = gh_f32;
      h.mode = pl.fb_vchunks == 1 ? 3 : (k == 0 ? 0 : (k == pl.fb_vchunks - 1 ? 2 : 1));
      plan_gh_split((int64_t)pl.n_ht * n_tt, cvn, pl.esize, rows, pl.H, &h.parts, &h.kt_per_part);
      h.part = reinterpret_cast<float*>(ws + pl.fb_ghpart);
      h.dscale = dscale;
      launch_gh(pl.dtype, h, st);
    }

    // grad_weight (+)= D^T . hidden[rows]
    GwArgs g;
    g.hiddenT = xt;
    g.D = Z;
    g.ldD = ldz;
    g.N = rows;
    g.H = (int)pl.H;
    g.V = (int)pl.V;
    g.N_pad = rows_pad;
    g.cv0 = 0;
    g.n_ht = (int)pl.n_ht;
    g.n_vt_c = (int)pl.n_vt;
    g.gw = grad_weight;
    g.gw_type = pl.gw_dtype;
    g.dscale = dscale;
    g.acc32 = reinterpret_cast<float*>(ws + pl.fb_gwacc);
    const bool first = b == 0, last = b == pl.fb_blocks - 1;
    if (pl.fb_gw_acc32) {   // fp32 sum over the blocks, rounded once at the end
      g.mode = first && last ? 3 : (first ? 0 : (last ? 2 : 1));
      g.accumulate = pl.accum_gw ? 1 : 0;
    } else {                // fp32 output, one block, or summed in the output's dtype on request
      g.mode = 3;
      g.accumulate = (!first || pl.accum_gw) ? 1 : 0;
    }
    launch_gw(pl.dtype, g, st);
  }
  launch_forward_scalars(pl, blk, (int)pl.n_tt, loss, num_correct, entropy_sum, status, st);
  if (grad_bias)
    launch_gb_reduce(pl.dtype, gb_part, (int)pl.n_tt, ldz, (int)pl.V, grad_bias, pl.accum_gb ? 1 : 0, ones, st);
  return hipGetLastError();
}

// In-place x *= g over n elements of type T, four per thread step; all threads
// return at once when g == 1.
template <typename T>
__global__ __launch_bounds__(256) void scale_kernel(T* x, int64_t n, const float* g) {
  typedef typename Quad<T>::type Q;
  const float s = g[0];
  if (s == 1.0f) return;
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    Q v = reinterpret_cast<Q*>(x)[i];
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = (T)((float)v[j] * s);
    reinterpret_cast<Q*>(x)[i] = v;
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = (T)((float)x[i] * s);
}

static void launch_scale(int dtype, void* x, int64_t n, const float* g, hipStream_t st) {
  if (n <= 0) return;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (dtype == FLCE_BF16) scale_kernel<bf16><<<(int)blocks, 256, 0, st>>>(reinterpret_cast<bf16*>(x), n, g);
  else if (dtype == FLCE_F16) scale_kernel<f16><<<(int)blocks, 256, 0, st>>>(reinterpret_cast<f16*>(x), n, g);
  else scale_kernel<float><<<(int)blocks, 256, 0, st>>>(reinterpret_cast<float*>(x), n, g);
}

hipError_t launch_scale_gradients(const Plan& pl, const float* g, void* grad_hidden, void* grad_weight,
                                  void* grad_bias, hipStream_t st) {
  launch_scale(pl.dtype, grad_hidden, pl.N * pl.H, g, st);
  launch_scale(pl.gw_dtype, grad_weight, pl.V * pl.H, g, st);
  if (grad_bias) launch_scale(pl.dtype, grad_bias, pl.V, g, st);
  return hipGetLastError();
}

}  // namespace flce
