// Forward pass: vocabulary-tiled logit GEMM with an online-softmax epilogue,
// then a fixed-order merge of the vocabulary splits and of the scalar sums.
//
// Method: fused-linear-ce README, "Algorithm" (tile over the vocabulary,
// fp32 accumulator, bias / logit_scale / softcap, online log-sum-exp merge,
// nothing of size (N, V) written) and "Metrics for free" (argmax carried with
// the running max; sum_j p_j z_j carried with the same rescaling).
#include "flce_device.h"
#include "flce_internal.h"

namespace flce {

struct FwdTileArgs {
  const char* hidden;
  const char* weight;
  const void* bias;
  const void* targets;
  int tgt_i32;
  int N, H, V;
  int64_t ignore_index;
  float scale, cap, two_log2e_over_cap, two_cap;
  int n_vt, S, N_pad;
  float* part_m;
  float* part_l;
  float* part_T;
  int* part_idx;
  float* part_zt;
  void* z;          // STORE_Z: logits of the tile rows, z[t - t_first][v], row stride ldz elements
  int ldz;
};

// Per-lane running softmax state for one token column.
struct RowState {
  float m, l, T, zt;
  int idx;
};

__device__ __forceinline__ void merge_state(RowState& a, const RowState& b) {
  const float mn = fmaxf(a.m, b.m);
  const float fa = fast_exp2((a.m - mn) * kLog2e);
  const float fb = fast_exp2((b.m - mn) * kLog2e);
  a.l = a.l * fa + b.l * fb;
  a.T = a.T * fa + b.T * fb;
  a.idx = b.m > a.m ? b.idx : (a.m > b.m ? a.idx : min(a.idx, b.idx));
  a.m = mn;
  a.zt = fmaxf(a.zt, b.zt);
}

// Four consecutive logits of one token, rounded to the input type.
__device__ __forceinline__ void store_z4(float* p, const float* z) {
  *reinterpret_cast<f32x4*>(p) = f32x4{z[0], z[1], z[2], z[3]};
}
__device__ __forceinline__ void store_z4(bf16* p, const float* z) {
  bf16x4 v;
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = (bf16)z[j];
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store_z4(f16* p, const float* z) {
  f16x4 v;
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = (f16)z[j];
  *reinterpret_cast<f16x4*>(p) = v;
}

// STORE_Z: also write every transformed logit z of the tiles to a.z (the row
// block's logits for the one-pass forward + backward); rows past V and tokens
// past N get finite values that the logit-gradient pass overwrites.
template <typename T, bool HAS_BIAS, bool SOFTCAP, bool STORE_Z>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiles_kernel(FwdTileArgs a) {
  constexpr int E = sizeof(T);
  const int L = xcd_logical_id(blockIdx.x, gridDim.x);
  // Token tiles x splits.  With whole groups of 4 token tiles, splits in
  // multiples of 8 and at least 256 workgroups, ids walk 4 token tiles, then
  // the next split, so the 32 ids one XCD runs at once are 4 token tiles x 8
  // splits: each hidden tile is read by 8 of them and each weight tile by 4,
  // the least fabric traffic for 32 resident tiles.  Otherwise token-tile
  // major: the 32 ids are 32/S token tiles x S splits.
  const int n_tt = (int)gridDim.x / a.S;
  const bool grouped = a.S % 8 == 0 && n_tt % 4 == 0 && gridDim.x >= 256;
  int tt, s;
  if (grouped) {
    grouped_tile(L, n_tt, a.S, 4, tt, s);
  } else {
    tt = L / a.S;
    s = L % a.S;
  }
  const int vt_begin = (int)((int64_t)s * a.n_vt / a.S);
  const int vt_end = (int)((int64_t)(s + 1) * a.n_vt / a.S);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int t0 = tt * 256;

  // Running state of the lane's kNI token columns: m and l in registers, the
  // rest (sum e z, the target logit, the argmax) and the tile's targets in
  // LDS, where they wait out the main loop without taking its registers.
  // Every lane reads and writes only its own state slots.
  static __shared__ float st_T[kWaves][kNI][64], st_zt[kWaves][kNI][64];
  static __shared__ int st_idx[kWaves][kNI][64], tile_tgt[256];
  float st_m[kNI], st_l[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    st_m[ni] = kMasked;
    st_l[ni] = 0.0f;
    st_T[wave][ni][lane] = 0.0f;
    st_zt[wave][ni][lane] = -INFINITY;
    st_idx[wave][ni][lane] = 0;
  }
  if (tid < 256) {   // visible to all waves after the main loop's first barrier
    const int t = t0 + tid;
    const int64_t tv = t < a.N ? load_target(a.targets, t, a.tgt_i32) : a.ignore_index;
    tile_tgt[tid] = (tv != a.ignore_index && tv >= 0 && tv < a.V) ? (int)tv : -1;
  }

  const uint32_t ld = (uint32_t)a.H * E;
  OperandDesc db;     // hidden rows of this token tile
  db.base = a.hidden + (size_t)t0 * ld;
  db.ld_bytes = ld;
  db.nrec = (uint32_t)min(a.N - t0, 256) * ld;
  db.cols_valid = 0;
  db.k_bytes = a.H * E;
  const int KT = (a.H * E + kBKB - 1) / kBKB;

  // One XCD runs `win` consecutive ids at once.  The splits of a token tile
  // share its hidden rows; the token tiles of a split read the same weight
  // tile at the same time.
  const int win = min(32, max(1, (int)gridDim.x / 8));
  L2Share sh;
  if (grouped) {
    sh.a_n = 4;
    sh.a_rank = tt & 3;
    sh.b_n = 8;
    sh.b_rank = s & 7;
  } else {
    sh.b_n = min(a.S, win);
    sh.b_rank = s % sh.b_n;
    sh.a_n = a.S <= win ? win / a.S : 1;
    sh.a_rank = tt % sh.a_n;
    if (sh.a_n < 2) sh.a_n = 0;
    if (sh.b_n < 2) sh.b_n = 0;
  }

  // the bias of each vocabulary tile is staged in LDS (two buffers, by tile
  // parity: a tile's bias is written only after every wave has passed the
  // barriers of the tile in between, i.e. finished reading the older one)
  static __shared__ __attribute__((aligned(16))) char bias_lds[2][256 * sizeof(T)];

  // scale of the accumulator into u (see the epilogue) and the exponent slope in r
  const float s_u = SOFTCAP ? a.scale * a.two_log2e_over_cap : a.scale;
  const float k1 = -a.two_cap * kLog2e;

  Acc acc[kMI][kNI];
  for (int vt = vt_begin; vt < vt_end; ++vt) {
    const int v0 = vt * 256;
    const char* bias_tile = bias_lds[(vt - vt_begin) & 1];
    // the range is rounded up to whole 4-byte words so that an odd last 16-bit
    // entry still arrives: its word lies in the same page as the entry (the
    // bias is 16-byte aligned), and its other half only feeds masked rows
    if (HAS_BIAS && wave == 0)
      dma_vector(reinterpret_cast<const T*>(a.bias) + v0, ((uint32_t)min(a.V - v0, 256) * E + 3u) & ~3u,
                 bias_lds[(vt - vt_begin) & 1], 256 * E, lane);
    OperandDesc da;     // weight rows of this vocabulary tile
    da.base = a.weight + (size_t)v0 * ld;
    da.ld_bytes = ld;
    da.nrec = (uint32_t)min(a.V - v0, 256) * ld;
    da.cols_valid = 0;
    da.k_bytes = a.H * E;
    zero_acc(acc);
    tile_mainloop<T, true, true>(da, db, KT, sh, acc);

    // ---- epilogue: per token column, transform the lane's 32 vocabulary rows of
    // the tile (4 of each of the 8 row tiles) and merge them into the running
    // state of the column.  Rows are visited in ascending order, so taking an
    // index only on a strict improvement of the running max keeps the lowest
    // index on ties.
    //
    // With the cap, the per-element work is written in u = 2 v log2(e) / cap
    // (v the scaled logit) and r = 1 / (2^u + 1): z = cap (1 - 2r) rises with
    // u, so the block max and argmax are taken on u; e^(z - m) =
    // 2^(r (-2 cap log2e) + (cap - m) log2e); and sum e z = cap sum e -
    // 2 cap sum e r.  Without the cap, u = z.
    //
    // Pass 1 overwrites the accumulator with u and takes the lane's max over
    // the rows below V; pass 2 forms r, the exponentials and the stored
    // logits.  Nothing but the accumulator holds the column (the registers are
    // the main loop's).  Rows at or past V (only in the last vocabulary tile)
    // keep their finite u for the stored logits and are left out of the max,
    // the argmax and the sums.
    // Row tests compare the compile-time offset 16 mi + r of an element with a
    // per-lane bound (acc_row(mi, r, lane) = 16 mi + r + 4 (lane / 16)), so
    // that no per-element row index is formed and kept in a register.
    const int vw = v0 + wm * kWaveM;
    const int n_valid = a.V - vw;   // rows of the wave block below V
    const bool ragged = n_valid < kWaveM;
    const int lane_row = acc_row(0, 0, lane);
    const int lim = n_valid - lane_row;   // element (mi, r) is below V iff 16 mi + r < lim
#pragma unroll
    for (int ni = 0; ni < kNI; ni++) {
      float mu = kMasked;
#pragma unroll
      for (int mi = 0; mi < kMI; mi++) {
        float sb[4];
        if constexpr (HAS_BIAS) {
          lds_vec4<T>(bias_tile, wm * kWaveM + acc_row(mi, 0, lane), sb);
#pragma unroll
          for (int j = 0; j < 4; j++) sb[j] *= s_u;
        }
#pragma unroll
        for (int r = 0; r < 4; r++)
          acc[mi][ni][r] = HAS_BIAS ? fmaf(acc[mi][ni][r], s_u, sb[r]) : acc[mi][ni][r] * s_u;
      }
      if (ragged) {
#pragma unroll
        for (int mi = 0; mi < kMI; mi++)
#pragma unroll
          for (int r = 0; r < 4; r++)
            if (16 * mi + r < lim) mu = fmaxf(mu, acc[mi][ni][r]);
      } else {
#pragma unroll
        for (int mi = 0; mi < kMI; mi++)
#pragma unroll
          for (int r = 0; r < 4; r++) mu = fmaxf(mu, acc[mi][ni][r]);
      }
      // the block max in z; a block that is all masked rows keeps kMasked
      float mx = mu;
      if constexpr (SOFTCAP) mx = mu == kMasked ? kMasked : fmaf(-a.two_cap, fast_rcp(fast_exp2(mu) + 1.0f), a.cap);
      // the target logit, where a lane of the wave holds its row here
      const int rel = tile_tgt[wn * kWaveN + acc_col(ni, lane)] - vw;
      const bool hit = rel >= 0 && rel < kWaveM && ((rel >> 2) & 3) == (lane >> 4);
      if (__builtin_amdgcn_ballot_w64(hit)) {
        const int rel_l = rel - lane_row;
        float ut = 0.0f;
#pragma unroll
        for (int mi = 0; mi < kMI; mi++)
#pragma unroll
          for (int r = 0; r < 4; r++)
            if (16 * mi + r == rel_l) ut = acc[mi][ni][r];
        if (hit) st_zt[wave][ni][lane] = SOFTCAP ? fmaf(-a.two_cap, fast_rcp(fast_exp2(ut) + 1.0f), a.cap) : ut;
      }
      const float m_old = st_m[ni];
      if (mx > m_old) {   // a new running max: its lowest row in this tile (rows past V come last)
        int ix = 0;
#pragma unroll
        for (int mi = kMI - 1; mi >= 0; mi--)
#pragma unroll
          for (int r = 3; r >= 0; r--)
            if (acc[mi][ni][r] == mu) ix = 16 * mi + r;
        st_idx[wave][ni][lane] = vw + lane_row + ix;
      }
      const float m_new = fmaxf(m_old, mx);
      const float mL = m_new * kLog2e;
      const float alpha = fast_exp2(fmaf(m_old, kLog2e, -mL));
      float se0 = 0.f, se1 = 0.f, sz0 = 0.f, sz1 = 0.f;
      // with the cap, sz accumulates sum e r
      const float k0 = fmaf(a.cap, kLog2e, -mL);
#pragma unroll
      for (int mi = 0; mi < kMI; mi++) {
        float z4[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float u = acc[mi][ni][r];
          const bool keep = !ragged || 16 * mi + r < lim;
          float e, w;
          if constexpr (SOFTCAP) {
            const float rr = fast_rcp(fast_exp2(u) + 1.0f);
            z4[r] = fmaf(-a.two_cap, rr, a.cap);
            w = keep ? rr : 1e30f;   // e = 2^(-huge) = 0, and e r = 0
            e = fast_exp2(fmaf(w, k1, k0));
          } else {
            z4[r] = u;
            w = keep ? u : kMasked;
            e = fast_exp2(fmaf(w, kLog2e, -mL));
          }
          if (r & 1) {
            se1 += e;
            sz1 = fmaf(e, w, sz1);
          } else {
            se0 += e;
            sz0 = fmaf(e, w, sz0);
          }
        }
        if constexpr (STORE_Z) {
          if constexpr (sizeof(T) == 2) {
            // into this wave's 16 KiB of LDS: 64 token rows x 128 logits (256 B);
            // 16-byte chunk q of row t sits at chunk q ^ (t & 15); the lane's
            // 4 logits are half of chunk 2 mi + lane/32
            const int tl = acc_col(ni, lane);
            // (opaque, so that the swizzled offsets are formed here and not
            // kept in registers across the main loop)
            int key = (tl & 15) << 4;
            asm volatile("" : "+v"(key));
            char* zst = g_lds + wave * 16384 + tl * 256 + 8 * ((lane >> 4) & 1);
            const int q = mi * 2 + (lane >> 5);
            store_z4(reinterpret_cast<T*>(zst + ((q << 4) ^ key)), z4);
          } else {
            const int t = wn * kWaveN + acc_col(ni, lane);   // within this token tile
            T* zrow = reinterpret_cast<T*>(a.z) + (size_t)(t0 + t) * a.ldz + vw + acc_row(mi, 0, lane);
            store_z4(zrow, z4);
          }
        }
      }
      const float se = se0 + se1;
      const float sz = SOFTCAP ? fmaf(-a.two_cap, sz0 + sz1, a.cap * se) : sz0 + sz1;
      st_l[ni] = fmaf(st_l[ni], alpha, se);
      st_T[wave][ni][lane] = fmaf(st_T[wave][ni][lane], alpha, sz);
      st_m[ni] = m_new;
    }
    if constexpr (STORE_Z && sizeof(T) == 2) {
      // the staged logits leave as whole rows, four 256-byte rows per store
      // instruction (each lane reads rows other lanes wrote); then every wave
      // has read its region back before the next tile's first stage is loaded
      // over it
      wave_lds_sync();
      const char* zst = g_lds + wave * 16384;
      const int q = lane & 15;
      T* zbase = reinterpret_cast<T*>(a.z) + (size_t)(t0 + wn * kWaveN + (lane >> 4)) * a.ldz + vw + 8 * q;
#pragma unroll 2
      for (int k = 0; k < 16; k++) {
        const int r = 4 * k + (lane >> 4);
        const i32x4 v = *reinterpret_cast<const i32x4*>(zst + r * 256 + ((q ^ (r & 15)) << 4));
        *reinterpret_cast<i32x4*>(zbase + (size_t)(4 * k) * a.ldz) = v;
      }
      __syncthreads();
    }
  }

  RowState st[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
    st[ni].m = st_m[ni];
    st[ni].l = st_l[ni];
    st[ni].T = st_T[wave][ni][lane];
    st[ni].zt = st_zt[wave][ni][lane];
    st[ni].idx = st_idx[wave][ni][lane];
  }
  // ---- merge the four lanes of a token column (lanes l, l^16, l^32, l^48: the
  // same token, rows in disjoint groups of 4)
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) {
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      RowState o;
      o.m = __shfl_xor(st[ni].m, x);
      o.l = __shfl_xor(st[ni].l, x);
      o.T = __shfl_xor(st[ni].T, x);
      o.zt = __shfl_xor(st[ni].zt, x);
      o.idx = __shfl_xor(st[ni].idx, x);
      merge_state(st[ni], o);
    }
  }
  // ---- merge the two M waves through LDS, then write the split's partials
  static_assert(kWavesM == 2, "the merge below pairs two waves along M");
  float* xs = reinterpret_cast<float*>(g_stage0);   // [wn][field][kWaveN]
  if (wm == 1 && lane < 16) {
#pragma unroll
    for (int ni = 0; ni < kNI; ni++) {
      const int c = acc_col(ni, lane);
      float* p = xs + wn * 5 * kWaveN;
      p[0 * kWaveN + c] = st[ni].m;
      p[1 * kWaveN + c] = st[ni].l;
      p[2 * kWaveN + c] = st[ni].T;
      p[3 * kWaveN + c] = st[ni].zt;
      p[4 * kWaveN + c] = __int_as_float(st[ni].idx);
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
#pragma unroll
    for (int ni = 0; ni < kNI; ni++) {
      const int c = acc_col(ni, lane);
      const float* p = xs + wn * 5 * kWaveN;
      RowState o;
      o.m = p[0 * kWaveN + c];
      o.l = p[1 * kWaveN + c];
      o.T = p[2 * kWaveN + c];
      o.zt = p[3 * kWaveN + c];
      o.idx = __float_as_int(p[4 * kWaveN + c]);
      merge_state(st[ni], o);
      const int t = t0 + wn * kWaveN + c;
      const size_t o_ = (size_t)s * a.N_pad + t;
      a.part_m[o_] = st[ni].m;
      a.part_l[o_] = st[ni].l;
      a.part_T[o_] = st[ni].T;
      a.part_zt[o_] = st[ni].zt;
      a.part_idx[o_] = st[ni].idx;
    }
  }
}

// ---------------------------------------------------------------------------
// Finalize: merge the S splits of each row in order, then per-block sums.
// ---------------------------------------------------------------------------
struct FinArgs {
  const void* targets;
  int tgt_i32;
  int N, V, S, N_pad, reduction;
  int64_t ignore_index;
  float z_loss;
  const float* part_m;
  const float* part_l;
  const float* part_T;
  const int* part_idx;
  const float* part_zt;
  float* loss;
  float* lse;
  BlockPart* blk;
};

__global__ __launch_bounds__(256) void fwd_finalize_rows(FinArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  double lsum = 0.0, esum = 0.0;
  int nv = 0, nc = 0, bad = 0;
  if (i < a.N) {
    RowState r;
    r.m = a.part_m[i];
    r.l = a.part_l[i];
    r.T = a.part_T[i];
    r.zt = a.part_zt[i];
    r.idx = a.part_idx[i];
    // splits merged in index order; their partials are loaded 8 at a time so
    // that the loads do not wait on each other
    for (int s0 = 1; s0 < a.S; s0 += 8) {
      RowState q[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {   // past the last split: reload the last one (not merged)
        const size_t o = (size_t)min(s0 + j, a.S - 1) * a.N_pad + i;
        q[j].m = a.part_m[o];
        q[j].l = a.part_l[o];
        q[j].T = a.part_T[o];
        q[j].zt = a.part_zt[o];
        q[j].idx = a.part_idx[o];
      }
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (s0 + j < a.S) merge_state(r, q[j]);
    }
    const float lse = r.m + fast_log2(r.l) * kLn2;
    const float ent = lse - r.T / r.l;
    const int64_t t = load_target(a.targets, i, a.tgt_i32);
    const bool in_range = t >= 0 && t < a.V;
    const bool valid = t != a.ignore_index && in_range;
    bad = (t != a.ignore_index && !in_range) ? 1 : 0;
    const float row_loss = valid ? (lse - r.zt + a.z_loss * lse * lse) : 0.0f;
    a.lse[i] = lse;
    if (a.reduction == FLCE_REDUCTION_NONE) a.loss[i] = row_loss;
    lsum = row_loss;
    esum = valid ? (double)ent : 0.0;
    nv = valid ? 1 : 0;
    nc = (valid && r.idx == (int)t) ? 1 : 0;
  }
  __shared__ double sl[256], se[256];
  __shared__ int sv[256], sc[256], sb[256];
  const int tid = threadIdx.x;
  sl[tid] = lsum;
  se[tid] = esum;
  sv[tid] = nv;
  sc[tid] = nc;
  sb[tid] = bad;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      sl[tid] += sl[tid + w];
      se[tid] += se[tid + w];
      sv[tid] += sv[tid + w];
      sc[tid] += sc[tid + w];
      sb[tid] |= sb[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    BlockPart b;
    b.loss = sl[0];
    b.entropy = se[0];
    b.n_valid = sv[0];
    b.n_correct = sc[0];
    b.bad_target = sb[0];
    b.pad = 0;
    a.blk[blockIdx.x] = b;
  }
}

struct ScalarArgs {
  const BlockPart* blk;
  int nblk, reduction;
  float* loss;
  int64_t* num_correct;
  float* entropy_sum;
  int* status;
};

__global__ __launch_bounds__(256) void fwd_finalize_scalars(ScalarArgs a) {
  __shared__ double sl[256], se[256];
  __shared__ long long sv[256], sc[256];
  __shared__ int sb[256];
  const int tid = threadIdx.x;
  double l = 0.0, e = 0.0;
  long long v = 0, c = 0;
  int b = 0;
  for (int j = tid; j < a.nblk; j += 256) {
    const BlockPart p = a.blk[j];
    l += p.loss;
    e += p.entropy;
    v += p.n_valid;
    c += p.n_correct;
    b |= p.bad_target;
  }
  sl[tid] = l;
  se[tid] = e;
  sv[tid] = v;
  sc[tid] = c;
  sb[tid] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      sl[tid] += sl[tid + w];
      se[tid] += se[tid + w];
      sv[tid] += sv[tid + w];
      sc[tid] += sc[tid + w];
      sb[tid] |= sb[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (a.reduction == FLCE_REDUCTION_SUM) a.loss[0] = (float)sl[0];
    else if (a.reduction == FLCE_REDUCTION_MEAN)
      a.loss[0] = sv[0] > 0 ? (float)(sl[0] / (double)sv[0]) : __builtin_nanf("");
    if (a.num_correct) a.num_correct[0] = (int64_t)sc[0];
    if (a.entropy_sum) a.entropy_sum[0] = (float)se[0];
    a.status[0] = sb[0] ? FLCE_ERR_TARGET_OUT_OF_RANGE : FLCE_OK;
  }
}

template <typename T, bool STORE_Z>
static void launch_fwd_tiles_z(const Plan& pl, const FwdTileArgs& args, int nwg, hipStream_t st) {
  if (pl.has_bias) {
    if (pl.cap > 0) fwd_tiles_kernel<T, true, true, STORE_Z><<<nwg, kThreads, 0, st>>>(args);
    else fwd_tiles_kernel<T, true, false, STORE_Z><<<nwg, kThreads, 0, st>>>(args);
  } else {
    if (pl.cap > 0) fwd_tiles_kernel<T, false, true, STORE_Z><<<nwg, kThreads, 0, st>>>(args);
    else fwd_tiles_kernel<T, false, false, STORE_Z><<<nwg, kThreads, 0, st>>>(args);
  }
}

template <typename T>
static void launch_fwd_tiles(const Plan& pl, const FwdTileArgs& args, int nwg, hipStream_t st) {
  if (args.z) launch_fwd_tiles_z<T, true>(pl, args, nwg, st);
  else launch_fwd_tiles_z<T, false>(pl, args, nwg, st);
}

// The tile kernel and the per-row merge for rows [r0, r0 + rows) of the batch:
// S vocabulary splits, partials in part (5 arrays of S x rows_pad), one
// BlockPart per 256 rows at blk[r0 / 256 ...], LSE (and the per-row loss for
// "none") at row r0 onwards; z: optional logits buffer (row stride ldz).
void launch_forward_rows(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                         const void* targets, int64_t r0, int rows, int S, float* part, float* loss, float* lse,
                         BlockPart* blk, void* z, int ldz, hipStream_t st) {
  const int n_tt = (rows + 255) / 256;
  const int rows_pad = n_tt * 256;
  const size_t NP = (size_t)rows_pad * S;
  float* part_m = part;
  float* part_l = part_m + NP;
  float* part_T = part_l + NP;
  float* part_zt = part_T + NP;
  int* part_idx = reinterpret_cast<int*>(part_zt + NP);
  const void* tg = static_cast<const char*>(targets) + (size_t)r0 * (pl.tgt_i32 ? 4 : 8);
  if (rows > 0) {
    FwdTileArgs a;
    a.hidden = static_cast<const char*>(hidden) + (size_t)r0 * pl.H * pl.esize;
    a.weight = static_cast<const char*>(weight);
    a.bias = bias;
    a.targets = tg;
    a.tgt_i32 = pl.tgt_i32 ? 1 : 0;
    a.N = rows;
    a.H = (int)pl.H;
    a.V = (int)pl.V;
    a.ignore_index = pl.ignore_index;
    a.scale = pl.scale;
    a.cap = pl.cap;
    a.two_log2e_over_cap = pl.cap > 0 ? 2.0f * kLog2e / pl.cap : 0.0f;
    a.two_cap = 2.0f * pl.cap;
    a.n_vt = (int)pl.n_vt;
    a.S = S;
    a.N_pad = rows_pad;
    a.part_m = part_m;
    a.part_l = part_l;
    a.part_T = part_T;
    a.part_idx = part_idx;
    a.part_zt = part_zt;
    a.z = z;
    a.ldz = ldz;
    const int nwg = n_tt * S;
    time_begin(pl, st);
    if (pl.dtype == FLCE_BF16) launch_fwd_tiles<bf16>(pl, a, nwg, st);
    else if (pl.dtype == FLCE_F16) launch_fwd_tiles<f16>(pl, a, nwg, st);
    else launch_fwd_tiles<float>(pl, a, nwg, st);
    time_end(pl, FLCE_KERNEL_FORWARD_TILES, st);
  }
  const int nblk = n_tt > 0 ? n_tt : 1;
  FinArgs f;
  f.targets = tg;
  f.tgt_i32 = pl.tgt_i32 ? 1 : 0;
  f.N = rows;
  f.V = (int)pl.V;
  f.S = S;
  f.N_pad = rows_pad;
  f.reduction = pl.reduction;
  f.ignore_index = pl.ignore_index;
  f.z_loss = pl.z_loss;
  f.part_m = part_m;
  f.part_l = part_l;
  f.part_T = part_T;
  f.part_idx = part_idx;
  f.part_zt = part_zt;
  f.loss = loss ? loss + r0 : nullptr;
  f.lse = lse ? lse + r0 : nullptr;
  f.blk = blk + r0 / 256;
  fwd_finalize_rows<<<nblk, 256, 0, st>>>(f);
}

// Fixed-order sums of the nblk BlockParts: the reduced loss, the metrics and the status word.
void launch_forward_scalars(const Plan& pl, const BlockPart* blk, int nblk, float* loss, int64_t* num_correct,
                            float* entropy_sum, int* status, hipStream_t st) {
  ScalarArgs sa;
  sa.blk = blk;
  sa.nblk = nblk;
  sa.reduction = pl.reduction;
  sa.loss = loss;
  sa.num_correct = num_correct;
  sa.entropy_sum = entropy_sum;
  sa.status = status;
  fwd_finalize_scalars<<<1, 256, 0, st>>>(sa);
}

hipError_t launch_forward(const Plan& pl, const void* hidden, const void* weight, const void* bias,
                          const void* targets, float* loss, float* lse, int64_t* num_correct,
                          float* entropy_sum, char* ws, hipStream_t st) {
  BlockPart* blk = reinterpret_cast<BlockPart*>(ws + pl.f_blk);
  launch_forward_rows(pl, hidden, weight, bias, targets, 0, (int)pl.N, pl.S, reinterpret_cast<float*>(ws + pl.f_part),
                      loss, lse, blk, nullptr, 0, st);
  const int nblk = pl.N > 0 ? (int)pl.n_tt : 1;
  launch_forward_scalars(pl, blk, nblk, loss, num_correct, entropy_sum, reinterpret_cast<int*>(ws), st);
  return hipGetLastError();
}

}  // namespace flce
