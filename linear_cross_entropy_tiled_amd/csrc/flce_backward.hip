// Backward pass: recompute each logit tile, form the logit gradient, and feed
// the two gradient contractions, one vocabulary chunk at a time.
//
// Method: fused-linear-ce README, "Algorithm" (recompute each tile, form
// p - onehot, accumulate grad_hidden = (p - onehot) @ weight and
// grad_weight = (p - onehot)^T @ hidden).  The weight gradient is accumulated
// in fp32 and cast once ("Chunked Linear Loss", "Weight-gradient accumulation
// dtype").  Per vocabulary chunk of width Vc:
//   dlogits  D[t][v] = scale * softcap'(z) * c_t * ((1 + 2 lam LSE_t) p_tv - [v = t_t])
//            into a scratch of N x Vc in the input dtype, plus per
//            token-tile column sums of D for grad_bias;
//   gw       grad_weight[v][:] = sum_t D[t][v] hidden[t][:]    (written once per row);
//   gh       grad_hidden[t][:] += sum_v D[t][v] weight[v][:]   (fp32, fixed chunk order).
// No float atomics: every output element has exactly one writer per launch,
// so results are bitwise reproducible.
//
// fp16 dlogits: with "mean" over thousands of tokens most entries of D are
// far below fp16's smallest normal (p ~ 1/V times c ~ 1/n_valid), so D is
// stored multiplied by a power of two 2^s chosen per call from the largest
// possible |D| (|scale| max_t (|coefA_t| + |coefB_t|)) to put that bound just
// under 2^14.  The contractions accumulate in fp32 and their epilogues
// multiply by 2^-s, which is exact, so the results are those of an unscaled
// D with fp16's full precision.  For bf16 and fp32 the factor is 1.
#include "flce_device.h"
#include "flce_internal.h"

namespace flce {

// ---------------------------------------------------------------------------
// Per-row coefficients: n_valid, c_i, and the constants the dlogits epilogue
// needs.  One block; N is at most a few hundred thousand rows.
// ---------------------------------------------------------------------------
struct PrepArgs {
  const void* targets;
  int tgt_i32;
  const float* lse;
  const float* grad_loss;
  int N, V, N_pad, reduction;
  int64_t ignore_index;
  float z_loss;
  float* coefA;   // c_i (1 + 2 lam LSE_i), 0 if ignored
  float* coefB;   // c_i, 0 if ignored
  float* lseL;    // LSE_i * log2(e); +inf on padding rows
  int* tgt;       // target or -1
  int* status;
  float* dscale;  // [0] = 2^s, [1] = 2^-s (see above)
  int f16_d;      // dlogits are fp16: choose s; else s = 0
  float abs_scale;
  int row0, row1; // coefficients (and the fp16 bound) for rows [row0, row1) only; n_valid counts all N
};

__global__ __launch_bounds__(1024) void bwd_prep_kernel(PrepArgs a) {
  __shared__ int sv[1024], sb[1024];
  __shared__ float sm[1024];
  const int tid = threadIdx.x;
  int nv = 0, bad = 0;
  for (int i = tid; i < a.N; i += 1024) {
    const int64_t t = load_target(a.targets, i, a.tgt_i32);
    const bool in_range = t >= 0 && t < a.V;
    nv += (t != a.ignore_index && in_range) ? 1 : 0;
    bad |= (t != a.ignore_index && !in_range) ? 1 : 0;
  }
  sv[tid] = nv;
  sb[tid] = bad;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) {
      sv[tid] += sv[tid + w];
      sb[tid] |= sb[tid + w];
    }
    __syncthreads();
  }
  const int n_valid = sv[0];
  const float g0 = a.reduction == FLCE_REDUCTION_NONE ? 0.0f : a.grad_loss[0];
  const float c_all = a.reduction == FLCE_REDUCTION_SUM ? g0 : (n_valid > 0 ? g0 / (float)n_valid : 0.0f);
  float dmax = 0.0f;
  for (int i = a.row0 + tid; i < a.row1; i += 1024) {
    // padding rows (i >= N) take LSE = +inf: their logit tiles are the bias
    // alone, and exp(z - LSE) must be 0 there however large that is (a finite
    // LSE of 0 overflows exp to inf once |scale * bias| passes ~88, and
    // inf * coefA = inf * 0 would put NaN into grad_bias and grad_weight)
    float ca = 0.0f, cb = 0.0f, ll = INFINITY;
    int tg = -1;
    if (i < a.N) {
      const int64_t t = load_target(a.targets, i, a.tgt_i32);
      const bool valid = t != a.ignore_index && t >= 0 && t < a.V;
      const float lse = a.lse[i];
      ll = lse * kLog2e;
      if (valid) {
        const float c = a.reduction == FLCE_REDUCTION_NONE ? a.grad_loss[i] : c_all;
        ca = c * (1.0f + 2.0f * a.z_loss * lse);
        cb = c;
        tg = (int)t;
      }
    }
    a.coefA[i] = ca;
    a.coefB[i] = cb;
    a.lseL[i] = ll;
    a.tgt[i] = tg;
    dmax = fmaxf(dmax, fabsf(ca) + fabsf(cb));
  }
  if (a.f16_d) {
    sm[tid] = dmax;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w) sm[tid] = fmaxf(sm[tid], sm[tid + w]);
      __syncthreads();
    }
  }
  if (tid == 0) {
    a.status[0] = sb[0] ? FLCE_ERR_TARGET_OUT_OF_RANGE : FLCE_OK;
    int s = 0;
    const float bound = a.f16_d ? sm[0] * a.abs_scale : 0.0f;   // >= every |D|
    if (bound > 0.0f && isfinite(bound)) {
      int e;
      frexpf(bound, &e);   // bound < 2^e
      s = min(max(14 - e, -120), 120);
    }
    a.dscale[0] = ldexpf(1.0f, s);
    a.dscale[1] = ldexpf(1.0f, -s);
  }
}

// ---------------------------------------------------------------------------
// Stores of 4 consecutive values (one lane, 4 consecutive rows of a tile),
// rounded to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(f16* p, float a, float b, float c, float d) {
  f16x4 v;
  v[0] = (f16)a;
  v[1] = (f16)b;
  v[2] = (f16)c;
  v[3] = (f16)d;
  *reinterpret_cast<f16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a;
  v[1] = b;
  v[2] = c;
  v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}

// Four consecutive elements from global memory, widened to fp32.
template <typename T> __device__ __forceinline__ void load4(const T* p, float* out);
template <> __device__ __forceinline__ void load4<float>(const float* p, float* out) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = v[j];
}
template <> __device__ __forceinline__ void load4<bf16>(const bf16* p, float* out) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = (float)v[j];
}
template <> __device__ __forceinline__ void load4<f16>(const f16* p, float* out) {
  const f16x4 v = *reinterpret_cast<const f16x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = (float)v[j];
}

// grad_weight element types (FLCE_F32, FLCE_BF16, FLCE_F16): 4 consecutive
// values added to (when accumulating) and stored in the buffer's type.
__device__ __forceinline__ void update4(void* base, size_t o, int type, bool accumulate, float* c) {
  if (accumulate) {
    float prev[4];
    if (type == FLCE_F32) load4<float>(reinterpret_cast<const float*>(base) + o, prev);
    else if (type == FLCE_BF16) load4<bf16>(reinterpret_cast<const bf16*>(base) + o, prev);
    else load4<f16>(reinterpret_cast<const f16*>(base) + o, prev);
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] += prev[j];
  }
  if (type == FLCE_F32) store4(reinterpret_cast<float*>(base) + o, c[0], c[1], c[2], c[3]);
  else if (type == FLCE_BF16) store4(reinterpret_cast<bf16*>(base) + o, c[0], c[1], c[2], c[3]);
  else store4(reinterpret_cast<f16*>(base) + o, c[0], c[1], c[2], c[3]);
}

// ---------------------------------------------------------------------------
// dlogits: one 256 (vocab) x 256 (token) tile per workgroup.
// ---------------------------------------------------------------------------
struct DlogitsArgs {
  const char* hidden;
  const char* weight;
  const void* bias;
  int N, H, V;
  float scale, cap, two_log2e_over_cap, two_cap;
  int cv0;          // first vocabulary row of the chunk
  int n_vt_c;       // vocabulary tiles in the chunk
  int n_tt;
  const float* coefA;
  const float* coefB;
  const float* lseL;
  const int* tgt;
  void* D;          // D[t][v - cv0], row stride ldD elements
  int ldD;
  float* gb_part;   // [n_tt][ld_gb]
  int ld_gb;
  const float* dscale;   // [0]: factor D is stored with
};

// DPP lane permutations within each 16-lane row, each an involution that
// pairs lanes differing in one bit of the lane index (and keeps the bits
// above it): row mirror (i <-> 15 - i: bit 3), half-row mirror (i <-> 7 - i
// within 8: bit 2), and the quad permutations [2 3 0 1] (bit 1) and
// [1 0 3 2] (bit 0).
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1;

// One halving step of an exchange reduction over the 16 lanes of a row: the
// lane and its partner (CTRL, which flips lane bit BIT) each keep one half of
// the 2 HALF values, the lane with bit BIT set the upper half, and add the
// partner's copy of that half.
template <int HALF, int BIT, int CTRL>
__device__ __forceinline__ void halve_exchange(float (&h)[32], int lane) {
  const bool hi = (lane & BIT) != 0;
#pragma unroll
  for (int k = 0; k < HALF; k++) {
    const float give = hi ? h[k] : h[HALF + k];
    const float keep = hi ? h[HALF + k] : h[k];
    const int got = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), CTRL, 0xF, 0xF, false);
    h[k] = keep + __builtin_bit_cast(float, got);
  }
}

template <typename T, bool HAS_BIAS, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd_dlogits_kernel(DlogitsArgs a) {
  constexpr int E = sizeof(T);
  const int L = xcd_logical_id(blockIdx.x, gridDim.x);
  int vt, tt;
  grouped_tile(L, a.n_vt_c, a.n_tt, 4, vt, tt);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int v0 = a.cv0 + vt * 256, t0 = tt * 256;

  const uint32_t ld = (uint32_t)a.H * E;
  OperandDesc da;     // weight rows
  OperandDesc db;     // hidden rows
  da.base = a.weight + (size_t)v0 * ld;
  da.ld_bytes = ld;
  da.nrec = (uint32_t)max(min(a.V - v0, 256), 0) * ld;
  da.cols_valid = 0;
  da.k_bytes = a.H * E;
  db.base = a.hidden + (size_t)t0 * ld;
  db.ld_bytes = ld;
  db.nrec = (uint32_t)max(min(a.N - t0, 256), 0) * ld;
  db.cols_valid = 0;
  db.k_bytes = a.H * E;
  const int KT = (a.H * E + kBKB - 1) / kBKB;

  // per-token coefficients (coefA, coefB, lseL, target) of the 256 tokens
  // and the bias of the 256 vocabulary rows, staged in LDS by DMA; the main
  // loop's first stage wait covers them
  static __shared__ __attribute__((aligned(16))) char vec_lds[4 * 1024 + 256 * sizeof(T)];
  {
    const uint32_t tok_bytes = 1024;   // the per-token arrays hold N_pad (a multiple of 256) entries
    if (wave == 0) dma_vector(a.coefA + t0, tok_bytes, vec_lds, 1024, lane);
    if (wave == 1) dma_vector(a.coefB + t0, tok_bytes, vec_lds + 1024, 1024, lane);
    if (wave == 2) dma_vector(a.lseL + t0, tok_bytes, vec_lds + 2048, 1024, lane);
    if (wave == 3) dma_vector(a.tgt + t0, tok_bytes, vec_lds + 3072, 1024, lane);
    // rounded up to whole words: an odd last bf16 entry shares its word
    // (same page) with a masked row
    if (HAS_BIAS && wave == 4)
      dma_vector(reinterpret_cast<const T*>(a.bias) + v0, ((uint32_t)max(min(a.V - v0, 256), 0) * E + 3u) & ~3u,
                 vec_lds + 4096, 256 * E, lane);
  }

  Acc acc[kMI][kNI];
  zero_acc(acc);
  tile_mainloop<T, true, true>(da, db, KT, no_share(), acc);

  // ---- epilogue, one 16-row MFMA tile at a time:
  //   D = 2^s * scale * softcap'(z) * (coefA * p - [row = target] * coefB),
  // stored as 4 consecutive vocabulary rows per lane, plus the column sums
  // over this tile's 256 tokens for grad_bias
  const int vw = v0 + wm * kWaveM;
  const bool ragged = vw + kWaveM > a.V;
  // With the cap, everything is written in r = 1 / (exp(2v/cap) + 1), where v
  // is the scaled logit: z = cap (1 - 2r), softcap'(z) = 1 - (z/cap)^2 =
  // 4 r (1 - r) and p = exp2(r * (-2 cap log2e) + cap log2e - LSE log2e).
  // Per token: cAs = scale coefA (4x with the cap), cBs likewise, k0 = the
  // exponent's constant term (or -LSE log2e without the cap).
  const float s2 = SOFTCAP ? a.scale * a.two_log2e_over_cap : a.scale;   // scale folded into the exp argument
  const float k1 = -a.two_cap * kLog2e;
  const float cmul = (SOFTCAP ? 4.0f * a.scale : a.scale) * a.dscale[0];
  float cAs[kNI], cBs[kNI], k0[kNI];
  int rel[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    const int tl = wn * kWaveN + acc_col(ni, lane);
    cAs[ni] = reinterpret_cast<const float*>(vec_lds)[tl] * cmul;
    cBs[ni] = reinterpret_cast<const float*>(vec_lds + 1024)[tl] * cmul;
    const float lL = reinterpret_cast<const float*>(vec_lds + 2048)[tl];
    k0[ni] = SOFTCAP ? fmaf(a.cap, kLog2e, -lL) : -lL;
    rel[ni] = reinterpret_cast<const int*>(vec_lds + 3072)[tl] - vw;
  }
  // whether any lane's target row lies in this wave's 128 rows, per column tile
  // (uniform; at large V almost never, so the per-row-tile test below is skipped)
  bool col_hit[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) col_hit[ni] = __builtin_amdgcn_ballot_w64(rel[ni] >= 0 && rel[ni] < kWaveM) != 0;
  T* D = reinterpret_cast<T*>(a.D);
  float cs[kMI][4];   // per vocabulary row of the lane: the sum over its kNI token columns
#pragma unroll
  for (int mi = 0; mi < kMI; mi++) {
    float sb[4];
    if constexpr (HAS_BIAS) {
      lds_vec4<T>(vec_lds + 4096, wm * kWaveM + acc_row(mi, 0, lane), sb);
#pragma unroll
      for (int j = 0; j < 4; j++) sb[j] *= s2;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) cs[mi][r] = 0.0f;
#pragma unroll
    for (int ni = 0; ni < kNI; ni++) {
      float f[4], d[4];   // f: softcap' / 4 with the cap, else unused
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float v = HAS_BIAS ? fmaf(acc[mi][ni][r], s2, sb[r]) : acc[mi][ni][r] * s2;
        if constexpr (SOFTCAP) {
          const float rr = fast_rcp(fast_exp2(v) + 1.0f);
          const float p = fast_exp2(fmaf(rr, k1, k0[ni]));
          f[r] = fmaf(-rr, rr, rr);
          d[r] = (p * cAs[ni]) * f[r];
        } else {
          d[r] = fast_exp2(fmaf(v, kLog2e, k0[ni])) * cAs[ni];
        }
      }
      // the target row, where some lane of the wave holds it here
      if (col_hit[ni]) {
        const int rt = rel[ni] - mi * 16;
        const bool hit = rt >= 0 && rt < 16 && (rt >> 2) == (lane >> 4);
        if (__builtin_amdgcn_ballot_w64(hit)) {
#pragma unroll
          for (int r = 0; r < 4; r++)
            if (acc_row(0, r, lane) == rt) d[r] -= SOFTCAP ? cBs[ni] * f[r] : cBs[ni];
        }
      }
      if (ragged) {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (vw + acc_row(mi, r, lane) >= a.V) d[r] = 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 4; r++) cs[mi][r] += d[r];
      if constexpr (sizeof(T) == 2) {
        // into this wave's 16 KiB of LDS (64 token rows x 128 logits; 16-byte
        // chunk q of row t at chunk q ^ (t & 15)), stored as whole rows below;
        // the lane's 4 values are half of chunk 2 mi + lane/32; the key is
        // opaque so that the offsets are not held across the main loop
        const int tl = acc_col(ni, lane);
        int key = (tl & 15) << 4;
        asm volatile("" : "+v"(key));
        char* dst = g_lds + wave * 16384 + tl * 256 + 8 * ((lane >> 4) & 1);
        const int q = mi * 2 + (lane >> 5);
        store4(reinterpret_cast<T*>(dst + ((q << 4) ^ key)), d[0], d[1], d[2], d[3]);
      } else {
        const int t = t0 + wn * kWaveN + acc_col(ni, lane);
        store4(D + (size_t)t * a.ldD + (vw - a.cv0) + acc_row(mi, 0, lane), d[0], d[1], d[2], d[3]);
      }
    }
  }
  if constexpr (sizeof(T) == 2) {
    // the staged logit gradient leaves as whole rows, four 256-byte rows per
    // store instruction (each lane reads rows other lanes wrote); non-temporal,
    // since only later launches read it back (a chunk is far larger than L2),
    // so that it does not displace operand lines other workgroups still read
    wave_lds_sync();
    const char* src = g_lds + wave * 16384;
    const int q = lane & 15;
    T* dbase = D + (size_t)(t0 + wn * kWaveN + (lane >> 4)) * a.ldD + (vw - a.cv0) + 8 * q;
#pragma unroll 2
    for (int k = 0; k < 16; k++) {
      const int r = 4 * k + (lane >> 4);
      const i32x4 v = *reinterpret_cast<const i32x4*>(src + r * 256 + ((q ^ (r & 15)) << 4));
      __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dbase + (size_t)(4 * k) * a.ldD));
    }
  }
  if constexpr (HAS_BIAS) {
    // grad_bias partial of this token tile: each vocabulary row's sum over the
    // tile's 256 tokens.  The 16 lanes of a lane group hold the same 32 rows
    // for 16 tokens each; an exchange that halves the values over lane bits
    // 3, 2, 1, 0 (partners from DPP permutations within the 16-lane row)
    // leaves lane i of group g the sums of its wave's 64 tokens for values
    // v = 2i, 2i + 1 (v = 4 mi + r: row 16 mi + 4 g + r).  The four waves
    // along the tokens then add through LDS.  Every step is in a fixed order,
    // so the sums are reproducible.
    static __shared__ float gbs[kWaves][kWaveM];
    float h[4 * kMI];
#pragma unroll
    for (int mi = 0; mi < kMI; mi++)
#pragma unroll
      for (int r = 0; r < 4; r++) h[4 * mi + r] = cs[mi][r];
    halve_exchange<16, 8, kDppRowMirror>(h, lane);
    halve_exchange<8, 4, kDppRowHalfMirror>(h, lane);
    halve_exchange<4, 2, kDppQuadXor2>(h, lane);
    halve_exchange<2, 1, kDppQuadXor1>(h, lane);
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int v = 2 * (lane & 15) + k;
      gbs[wave][(v >> 2) * 16 + 4 * (lane >> 4) + (v & 3)] = h[k];
    }
    __syncthreads();
    const int tid2 = threadIdx.x;
    if (tid2 < 256) {
      const int wm2 = tid2 / kWaveM, row = tid2 % kWaveM;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWavesN; w++) sum += gbs[wm2 * kWavesN + w][row];
      a.gb_part[(size_t)tt * a.ld_gb + v0 + tid2] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// grad_weight epilogue for a wave whose 128 (h) x 64 (v) block lies inside the
// matrix: straight-line code per (mode, output type, accumulate), and per half
// MFMA tile every read (the fp32 accumulator, the prior output) is issued
// before the first store, so the reads overlap instead of each waiting for the
// stores before it.  Lane: 4 consecutive h of one v per 4-register group.
// ---------------------------------------------------------------------------
template <typename OutT> __device__ __forceinline__ f32x4 load4v(const OutT* p);
template <> __device__ __forceinline__ f32x4 load4v<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <> __device__ __forceinline__ f32x4 load4v<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ __forceinline__ f32x4 load4v<f16>(const f16* p) {
  const f16x4 v = *reinterpret_cast<const f16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename T> constexpr bool is_f16() { return false; }
template <> constexpr bool is_f16<f16>() { return true; }

// MODE 0: acc32 = C; 1: acc32 += C; 2: out = acc32 + C; 3: out = C; ACC (modes
// 2, 3): plus out's prior contents.  C = the accumulator times `inv`; row r of
// the wave's block is row rbase + r of the ld-wide matrices, column c is
// column cbase + c.
template <typename OutT, int MODE, bool ACC>
__device__ __forceinline__ void block_store_t(float* acc32, OutT* out, int ld,
                                              const Acc (&acc)[kMI][kNI], float inv, int rbase, int cbase,
                                              int lane) {
  constexpr bool READ_ACC = MODE == 1 || MODE == 2;
  constexpr bool READ_OUT = ACC && MODE >= 2;
  // The accumulator holds, per lane and tile, 4 consecutive columns of one row
  // (16 rows per store instruction, 16 bytes each).  It goes through a 16 KiB
  // LDS region of this wave's own, one 16-row MFMA tile column at a time, and
  // leaves as whole rows: two 128-column rows per instruction, every cache
  // line written whole.  Rows are 512 bytes; the 16-byte chunk c of row r sits
  // at chunk c ^ r, so both the scattered writes and the row reads are free of
  // bank conflicts.  Every LDS read of the main loop whose value is used has
  // completed before it returns, and a wave reads back only what it wrote.
  char* stage = g_lds + (threadIdx.x >> 6) * 16384;
  const int r_w = lane & 15;
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
#pragma unroll
    for (int mi = 0; mi < kMI; mi++) {
      const int ch = mi * 4 + (lane >> 4);   // columns 4 ch .. 4 ch + 3
      *reinterpret_cast<f32x4*>(stage + r_w * 512 + ((ch ^ r_w) << 4)) = acc[mi][ni];
    }
    wave_lds_sync();   // the rows below were written by other lanes
    const int c = lane & 31;
#pragma unroll
    for (int k0 = 0; k0 < 8; k0 += 4) {
      f32x4 pa[4], po[4], cv[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int rr = 2 * (k0 + k) + (lane >> 5);
        const size_t o = (size_t)(rbase + ni * 16 + rr) * ld + cbase + 4 * c;
        if constexpr (READ_ACC) pa[k] = *reinterpret_cast<const f32x4*>(acc32 + o);
        if constexpr (READ_OUT) po[k] = load4v<OutT>(out + o);
        cv[k] = *reinterpret_cast<const f32x4*>(stage + rr * 512 + ((c ^ rr) << 4));
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int rr = 2 * (k0 + k) + (lane >> 5);
        const size_t o = (size_t)(rbase + ni * 16 + rr) * ld + cbase + 4 * c;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[j] = cv[k][j] * inv;
          if constexpr (READ_ACC) v[j] += pa[k][j];
          if constexpr (READ_OUT) v[j] += po[k][j];
        }
        if constexpr (MODE <= 1) store4(acc32 + o, v[0], v[1], v[2], v[3]);
        else store4(out + o, v[0], v[1], v[2], v[3]);
      }
    }
    wave_lds_sync();   // every lane has read the area before the next tile column is written over it
  }
}

// Modes 2 and 3 into an output of type OutT.
template <typename OutT>
__device__ __forceinline__ void block_store_out(float* acc32, void* out, int ld, int mode, bool accumulate,
                                                const Acc (&acc)[kMI][kNI], float inv, int rbase, int cbase,
                                                int lane) {
  OutT* o = reinterpret_cast<OutT*>(out);
  if (mode == 2) {
    if (accumulate) block_store_t<OutT, 2, true>(acc32, o, ld, acc, inv, rbase, cbase, lane);
    else block_store_t<OutT, 2, false>(acc32, o, ld, acc, inv, rbase, cbase, lane);
  } else {
    if (accumulate) block_store_t<OutT, 3, true>(acc32, o, ld, acc, inv, rbase, cbase, lane);
    else block_store_t<OutT, 3, false>(acc32, o, ld, acc, inv, rbase, cbase, lane);
  }
}

// Any mode; out_type is the flce_dtype of `out` (modes 2, 3).
__device__ __forceinline__ void block_store(float* acc32, void* out, int out_type, int ld, int mode, bool accumulate,
                                            const Acc (&acc)[kMI][kNI], float inv, int rbase, int cbase,
                                            int lane) {
  if (mode == 0) block_store_t<float, 0, false>(acc32, nullptr, ld, acc, inv, rbase, cbase, lane);
  else if (mode == 1) block_store_t<float, 1, false>(acc32, nullptr, ld, acc, inv, rbase, cbase, lane);
  else if (out_type == FLCE_BF16) block_store_out<bf16>(acc32, out, ld, mode, accumulate, acc, inv, rbase, cbase, lane);
  else if (out_type == FLCE_F16) block_store_out<f16>(acc32, out, ld, mode, accumulate, acc, inv, rbase, cbase, lane);
  else block_store_out<float>(acc32, out, ld, mode, accumulate, acc, inv, rbase, cbase, lane);
}

// ---------------------------------------------------------------------------
// grad_weight for one chunk: C[h][v] = sum_t hidden[t][h] D[t][v]
// A = hidden (MNMAJOR: rows t, cols h), B = D (MNMAJOR: rows t, cols v).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_gw_kernel(GwArgs a) {
  constexpr int E = sizeof(T);
  const int L = xcd_logical_id(blockIdx.x, gridDim.x);
  int ht, vt;
  grouped_tile(L, a.n_ht, a.n_vt_c, 4, ht, vt);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int h0 = ht * 256, vl0 = vt * 256;

  OperandDesc da;     // hidden^T rows h, K = tokens
  const uint32_t ldt = (uint32_t)a.N_pad * E;
  da.base = a.hiddenT + (size_t)h0 * ldt;
  da.ld_bytes = ldt;
  da.nrec = (uint32_t)min(a.H - h0, 256) * ldt;
  da.cols_valid = 0;
  da.k_bytes = a.N_pad * E;
  OperandDesc db;     // dlogits rows t (K), columns v: transposing reads
  const uint32_t ldd = (uint32_t)a.ldD * E;
  db.base = a.D + (size_t)vl0 * E;
  db.ld_bytes = ldd;
  db.nrec = a.N_pad > 0 ? (uint32_t)((size_t)a.N_pad * ldd - (size_t)vl0 * E) : 0u;
  db.cols_valid = a.ldD - vl0;
  db.k_bytes = 0;
  const int KT = (a.N_pad * E + kBKB - 1) / kBKB;

  Acc acc[kMI][kNI];
  zero_acc(acc);
  tile_mainloop<T, true, false>(da, db, KT, no_share(), acc);

  const float inv = a.dscale[1];
  const int vbase = a.cv0 + vl0 + wn * kWaveN, hbase = h0 + wm * kWaveM;
  if (vbase + kWaveN <= a.V && hbase + kWaveM <= a.H) {   // the wave's block lies inside grad_weight
    block_store(a.acc32, a.gw, a.gw_type, a.H, a.mode, a.accumulate != 0, acc, inv, vbase, hbase, lane);
    return;
  }
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    const int v = a.cv0 + vl0 + wn * kWaveN + acc_col(ni, lane);
    if (v >= a.V) continue;
#pragma unroll
    for (int mi = 0; mi < kMI; mi++) {
      const int h = h0 + wm * kWaveM + acc_row(mi, 0, lane);   // 4 consecutive h; H % 8 == 0
      if (h >= a.H) continue;
      const size_t o = (size_t)v * a.H + h;
      float c[4] = {acc[mi][ni][0] * inv, acc[mi][ni][1] * inv, acc[mi][ni][2] * inv, acc[mi][ni][3] * inv};
      if (a.mode == 1 || a.mode == 2) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(a.acc32 + o);
#pragma unroll
        for (int j = 0; j < 4; j++) c[j] += prev[j];
      }
      if (a.mode <= 1) store4(a.acc32 + o, c[0], c[1], c[2], c[3]);
      else update4(a.gw, o, a.gw_type, a.accumulate != 0, c);
    }
  }
}

// ---------------------------------------------------------------------------
// grad_hidden for one chunk: C[h][t] = sum_v weight[v][h] D[t][v]
// A = weight (MNMAJOR: rows v, cols h), B = D (KMAJOR: rows t, K = v).
// mode 0: first of several chunks (store fp32 accumulator)
// mode 1: middle chunk (accumulator += C)
// mode 2: last chunk (out = cast(accumulator + C))
// mode 3: only chunk (out = cast(C))
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_gh_kernel(GhArgs a) {
  constexpr int E = sizeof(T);
  const int L = xcd_logical_id(blockIdx.x, gridDim.x);
  // the split is the slow index, so the workgroups one XCD runs together
  // share a K range and the grouped tile order still applies within it
  const int n_tiles = a.n_ht * a.n_tt;
  const int split = L / n_tiles;
  int ht, tt;
  grouped_tile(L - split * n_tiles, a.n_ht, a.n_tt, 4, ht, tt);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int h0 = ht * 256, t0 = tt * 256;

  // this split's K range: stages [kt0, kt0 + KT) of the chunk (64 vocabulary rows each)
  const int KT_all = (a.cvn * E + kBKB - 1) / kBKB;
  const int kt0 = split * a.kt_per_part;
  const int KT = max(min(KT_all - kt0, a.kt_per_part), 0);
  const int v_off = kt0 * (kBKB / E);   // first vocabulary row of the split within the chunk

  OperandDesc da;     // weight rows v (K) of the split, columns h: transposing reads
  const uint32_t ldw = (uint32_t)a.H * E;
  const int vrows = max(min(a.V - a.cv0, a.cvn) - v_off, 0);
  da.base = a.weight + ((size_t)(a.cv0 + v_off) * a.H + h0) * E;
  da.ld_bytes = ldw;
  da.nrec = vrows > 0 ? (uint32_t)((size_t)vrows * ldw - (size_t)h0 * E) : 0u;
  da.cols_valid = a.H - h0;
  da.k_bytes = 0;
  OperandDesc db;     // dlogits rows t, K = v
  const uint32_t ldd = (uint32_t)a.ldD * E;
  db.base = a.D + (size_t)t0 * ldd + (size_t)v_off * E;
  db.ld_bytes = ldd;
  db.nrec = 256u * ldd - (uint32_t)v_off * E;
  db.cols_valid = 0;
  db.k_bytes = (a.cvn - v_off) * E;

  Acc acc[kMI][kNI];
  zero_acc(acc);
  tile_mainloop<T, false, true>(da, db, KT, grouped_share(ht, tt), acc);

  const float inv = a.dscale[1];
  const int tbase = t0 + wn * kWaveN, hbase = h0 + wm * kWaveM;
  if (tbase + kWaveN <= a.N && hbase + kWaveM <= a.H) {   // the wave's block lies inside grad_hidden
    if (a.parts > 1)   // partial of this split; bwd_gh_reduce applies the mode
      block_store(a.part + (size_t)split * a.N * a.H, nullptr, FLCE_F32, a.H, 0, false, acc, inv, tbase, hbase, lane);
    else
      block_store(a.accb, a.out, a.out_f32 ? FLCE_F32 : (sizeof(T) == 2 ? (is_f16<T>() ? FLCE_F16 : FLCE_BF16) : FLCE_F32),
                  a.H, a.mode, false, acc, inv, tbase, hbase, lane);
    return;
  }
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    const int t = t0 + wn * kWaveN + acc_col(ni, lane);
    if (t >= a.N) continue;
#pragma unroll
    for (int mi = 0; mi < kMI; mi++) {
      const int h = h0 + wm * kWaveM + acc_row(mi, 0, lane);   // 4 consecutive h; H % 8 == 0
      if (h >= a.H) continue;
      const size_t o = (size_t)t * a.H + h;
      float c0 = acc[mi][ni][0] * inv, c1 = acc[mi][ni][1] * inv;
      float c2 = acc[mi][ni][2] * inv, c3 = acc[mi][ni][3] * inv;
      if (a.parts > 1) {   // partial of this split; bwd_gh_reduce applies the mode
        store4(a.part + (size_t)split * a.N * a.H + o, c0, c1, c2, c3);
        continue;
      }
      if (a.mode == 1 || a.mode == 2) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(a.accb + o);
        c0 += prev[0];
        c1 += prev[1];
        c2 += prev[2];
        c3 += prev[3];
      }
      if (a.mode <= 1 || a.out_f32) {
        float* dst = (a.mode <= 1) ? a.accb + o : reinterpret_cast<float*>(a.out) + o;
        store4(dst, c0, c1, c2, c3);
      } else {
        store4(reinterpret_cast<T*>(a.out) + o, c0, c1, c2, c3);
      }
    }
  }
}

// grad_hidden with a K split: out = (mode 1, 2: accumulator +) sum of the
// partials in split order, stored like bwd_gh_kernel's epilogue (mode 0, 1 ->
// accumulator; 2, 3 -> output, cast).  Four consecutive elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void bwd_gh_reduce(const float* part, int parts, int64_t n4, int64_t stride,
                                                     float* accb, void* out, int out_f32, int mode) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 s = (mode == 1 || mode == 2) ? reinterpret_cast<const f32x4*>(accb)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < parts; p++) s += reinterpret_cast<const f32x4*>(part + (size_t)p * stride)[i];
  if (mode <= 1 || out_f32) {
    float* dst = mode <= 1 ? accb : reinterpret_cast<float*>(out);
    reinterpret_cast<f32x4*>(dst)[i] = s;
  } else {
    store4(reinterpret_cast<T*>(out) + 4 * i, s[0], s[1], s[2], s[3]);
  }
}

// hidden^T [H][N_pad] (zero for t >= N): the token-contiguous copy of hidden
// that the grad_weight contraction reads as its register operand.
template <typename T>
__global__ __launch_bounds__(256) void transpose_hidden_kernel(const T* x, int N, int H, int N_pad, T* xt) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r, h = h0 + tx;
    tile[r][tx] = (t < N && h < H) ? load_elem<T>(x, (int64_t)t * H + h) : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int h = h0 + r, t = t0 + tx;
    if (h < H && t < N_pad) xt[(size_t)h * N_pad + t] = (T)tile[tx][r];
  }
}

// grad_bias[v] = sum over token tiles of the per-tile column sums, in order
// (sums of the stored D, so times 2^-s).
template <typename T>
__global__ __launch_bounds__(256) void bwd_gb_reduce(const float* part, int n_tt, int ld, int V, T* gb,
                                                     int accumulate, const float* dscale) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float s = 0.0f;
  for (int i = 0; i < n_tt; i++) s += part[(size_t)i * ld + v];
  s *= dscale[1];
  if (accumulate) s += load_elem<T>(gb, v);
  gb[v] = (T)s;
}

// Per-row coefficients of rows [row0, row1) (n_valid over all rows) and the
// fp16 dlogits factor from those rows.
void launch_prep_rows(const Plan& pl, const void* targets, const float* lse, const float* grad_loss, float* coefA,
                      float* coefB, float* lseL, int* tgt, int* status, float* dscale, int64_t row0, int64_t row1,
                      hipStream_t st) {
  PrepArgs pa;
  pa.targets = targets;
  pa.tgt_i32 = pl.tgt_i32 ? 1 : 0;
  pa.lse = lse;
  pa.grad_loss = grad_loss;
  pa.N = (int)pl.N;
  pa.V = (int)pl.V;
  pa.N_pad = (int)pl.N_pad;
  pa.reduction = pl.reduction;
  pa.ignore_index = pl.ignore_index;
  pa.z_loss = pl.z_loss;
  pa.coefA = coefA;
  pa.coefB = coefB;
  pa.lseL = lseL;
  pa.tgt = tgt;
  pa.status = status;
  pa.dscale = dscale;
  pa.f16_d = pl.dtype == FLCE_F16;
  pa.abs_scale = fabsf(pl.scale);
  pa.row0 = (int)row0;
  pa.row1 = (int)row1;
  bwd_prep_kernel<<<1, 1024, 0, st>>>(pa);
}

template <typename T>
static hipError_t launch_backward_t(const Plan& pl, const void* hidden, const void* weight,
                                    const void* bias, const void* targets, const float* lse,
                                    const float* grad_loss, void* grad_hidden, void* grad_weight,
                                    void* grad_bias, char* ws, hipStream_t st) {
  float* coefA = reinterpret_cast<float*>(ws + pl.b_coefA);
  float* coefB = reinterpret_cast<float*>(ws + pl.b_coefB);
  float* lseL = reinterpret_cast<float*>(ws + pl.b_lseL);
  int* tgt = reinterpret_cast<int*>(ws + pl.b_tgt);
  char* D = ws + pl.b_D;
  float* gb_part = reinterpret_cast<float*>(ws + pl.b_gbpart);

  float* dscale = reinterpret_cast<float*>(ws + kDscaleOffset);
  launch_prep_rows(pl, targets, lse, grad_loss, coefA, coefB, lseL, tgt, reinterpret_cast<int*>(ws), dscale, 0,
                   pl.N_pad, st);

  T* hiddenT = reinterpret_cast<T*>(ws + pl.b_xt);
  if (pl.N > 0) launch_transpose_hidden(pl.dtype, hidden, (int)pl.N, (int)pl.H, (int)pl.N_pad, hiddenT, st);
  const bool gh_f32 = pl.dtype == FLCE_F32;
  float* accb = gh_f32 ? reinterpret_cast<float*>(grad_hidden) : reinterpret_cast<float*>(ws + pl.b_ghacc);
  const int ldD = (int)pl.Vc;

  for (int c = 0; c < pl.n_chunks; c++) {
    const int cv0 = (int)(c * pl.Vc);
    const int cvn = (int)(pl.V_pad - cv0 < pl.Vc ? pl.V_pad - cv0 : pl.Vc);
    const int n_vt_c = cvn / 256;
    if (pl.N > 0) {
      DlogitsArgs d;
      d.hidden = static_cast<const char*>(hidden);
      d.weight = static_cast<const char*>(weight);
      d.bias = bias;
      d.N = (int)pl.N;
      d.H = (int)pl.H;
      d.V = (int)pl.V;
      d.scale = pl.scale;
      d.cap = pl.cap;
      d.two_log2e_over_cap = pl.cap > 0 ? 2.0f * kLog2e / pl.cap : 0.0f;
      d.two_cap = 2.0f * pl.cap;
      d.cv0 = cv0;
      d.n_vt_c = n_vt_c;
      d.n_tt = (int)pl.n_tt;
      d.coefA = coefA;
      d.coefB = coefB;
      d.lseL = lseL;
      d.tgt = tgt;
      d.D = D;
      d.ldD = ldD;
      d.gb_part = gb_part;
      d.ld_gb = (int)pl.V_pad;
      d.dscale = dscale;
      const int nwg = n_vt_c * (int)pl.n_tt;
      time_begin(pl, st);
      if (pl.has_bias) {
        if (pl.cap > 0) bwd_dlogits_kernel<T, true, true><<<nwg, kThreads, 0, st>>>(d);
        else bwd_dlogits_kernel<T, true, false><<<nwg, kThreads, 0, st>>>(d);
      } else {
        if (pl.cap > 0) bwd_dlogits_kernel<T, false, true><<<nwg, kThreads, 0, st>>>(d);
        else bwd_dlogits_kernel<T, false, false><<<nwg, kThreads, 0, st>>>(d);
      }
      time_end(pl, FLCE_KERNEL_DLOGITS, st);
    }
    {
      GwArgs g;
      g.hiddenT = reinterpret_cast<const char*>(hiddenT);
      g.D = D;
      g.ldD = ldD;
      g.N = (int)pl.N;
      g.H = (int)pl.H;
      g.V = (int)pl.V;
      g.N_pad = (int)pl.N_pad;
      g.cv0 = cv0;
      g.n_ht = (int)pl.n_ht;
      g.n_vt_c = n_vt_c;
      g.gw = grad_weight;
      g.gw_type = pl.gw_dtype;
      g.dscale = dscale;
      g.accumulate = pl.accum_gw ? 1 : 0;
      g.acc32 = nullptr;
      g.mode = 3;   // each vocabulary row belongs to one chunk: written once
      time_begin(pl, st);
      launch_gw(pl.dtype, g, st);
      time_end(pl, FLCE_KERNEL_GRAD_WEIGHT, st);
    }
    if (pl.N > 0) {
      GhArgs h;
      h.weight = static_cast<const char*>(weight);
      h.D = D;
      h.ldD = ldD;
      h.N = (int)pl.N;
      h.H = (int)pl.H;
      h.V = (int)pl.V;
      h.cv0 = cv0;
      h.cvn = cvn;
      h.n_ht = (int)pl.n_ht;
      h.n_tt = (int)pl.n_tt;
      h.accb = accb;
      h.out = grad_hidden;
      h.out_f32 = gh_f32;
      h.mode = pl.n_chunks == 1 ? 3 : (c == 0 ? 0 : (c == pl.n_chunks - 1 ? 2 : 1));
      h.parts = pl.gh_parts;
      h.kt_per_part = pl.gh_kt_per_part;
      h.part = reinterpret_cast<float*>(ws + pl.b_ghpart);
      h.dscale = dscale;
      time_begin(pl, st);
      launch_gh(pl.dtype, h, st);
      time_end(pl, FLCE_KERNEL_GRAD_HIDDEN, st);
    }
  }
  if (grad_bias) {
    bwd_gb_reduce<T><<<(int)((pl.V + 255) / 256), 256, 0, st>>>(gb_part, (int)pl.n_tt, (int)pl.V_pad,
                                                               (int)pl.V, reinterpret_cast<T*>(grad_bias),
                                                               pl.accum_gb ? 1 : 0, dscale);
  }
  return hipGetLastError();
}

void launch_gb_reduce(int dtype, const float* part, int n_tt, int ld, int V, void* gb, int accumulate,
                      const float* dscale, hipStream_t st) {
  const int nwg = (V + 255) / 256;
  if (dtype == FLCE_BF16)
    bwd_gb_reduce<bf16><<<nwg, 256, 0, st>>>(part, n_tt, ld, V, reinterpret_cast<bf16*>(gb), accumulate, dscale);
  else if (dtype == FLCE_F16)
    bwd_gb_reduce<f16><<<nwg, 256, 0, st>>>(part, n_tt, ld, V, reinterpret_cast<f16*>(gb), accumulate, dscale);
  else
    bwd_gb_reduce<float><<<nwg, 256, 0, st>>>(part, n_tt, ld, V, reinterpret_cast<float*>(gb), accumulate, dscale);
}

template <typename T>
static void launch_transpose_t(const void* hidden, int N, int H, int N_pad, void* hiddenT, hipStream_t st) {
  dim3 grid((unsigned)(N_pad / 64), (unsigned)((H + 63) / 64));
  transpose_hidden_kernel<T><<<grid, 256, 0, st>>>(reinterpret_cast<const T*>(hidden), N, H, N_pad,
                                                   reinterpret_cast<T*>(hiddenT));
}

void launch_transpose_hidden(int dtype, const void* hidden, int N, int H, int N_pad, void* hiddenT,
                             hipStream_t st) {
  if (dtype == FLCE_BF16) launch_transpose_t<bf16>(hidden, N, H, N_pad, hiddenT, st);
  else if (dtype == FLCE_F16) launch_transpose_t<f16>(hidden, N, H, N_pad, hiddenT, st);
  else launch_transpose_t<float>(hidden, N, H, N_pad, hiddenT, st);
}

void launch_gw(int dtype, const GwArgs& g, hipStream_t st) {
  const int nwg = g.n_ht * g.n_vt_c;
  if (dtype == FLCE_BF16) bwd_gw_kernel<bf16><<<nwg, kThreads, 0, st>>>(g);
  else if (dtype == FLCE_F16) bwd_gw_kernel<f16><<<nwg, kThreads, 0, st>>>(g);
  else bwd_gw_kernel<float><<<nwg, kThreads, 0, st>>>(g);
}

template <typename T>
static void launch_gh_t(const GhArgs& h, hipStream_t st) {
  bwd_gh_kernel<T><<<h.n_ht * h.n_tt * h.parts, kThreads, 0, st>>>(h);
  if (h.parts > 1) {
    const int64_t nh = (int64_t)h.N * h.H, n4 = nh / 4;
    bwd_gh_reduce<T><<<(int)((n4 + 255) / 256), 256, 0, st>>>(h.part, h.parts, n4, nh, h.accb, h.out, h.out_f32,
                                                              h.mode);
  }
}

void launch_gh(int dtype, const GhArgs& h, hipStream_t st) {
  if (dtype == FLCE_BF16) launch_gh_t<bf16>(h, st);
  else if (dtype == FLCE_F16) launch_gh_t<f16>(h, st);
  else launch_gh_t<float>(h, st);
}

hipError_t launch_backward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                           const void* targets, const float* lse, const float* grad_loss,
                           void* grad_hidden, void* grad_weight, void* grad_bias, char* ws,
                           hipStream_t st) {
  if (pl.dtype == FLCE_BF16)
    return launch_backward_t<bf16>(pl, hidden, weight, bias, targets, lse, grad_loss, grad_hidden,
                                   grad_weight, grad_bias, ws, st);
  if (pl.dtype == FLCE_F16)
    return launch_backward_t<f16>(pl, hidden, weight, bias, targets, lse, grad_loss, grad_hidden,
                                  grad_weight, grad_bias, ws, st);
  return launch_backward_t<float>(pl, hidden, weight, bias, targets, lse, grad_loss, grad_hidden,
                                  grad_weight, grad_bias, ws, st);
}

}  // namespace flce
