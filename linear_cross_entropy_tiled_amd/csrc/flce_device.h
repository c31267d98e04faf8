// Device-side building blocks for the fused linear cross-entropy kernels
// (gfx950 / CDNA4): vector types, buffer loads, fast transcendentals and the
// shared 256x256 MFMA tile main loop.
//
// Tile main loop: C[256 x 256] += A[256 x K] . B[256 x K]^T with fp32
// accumulation, 4 waves (2 x 2), each wave owning a 128 x 128 block as 4 x 4
// tiles of v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x2_f32 for fp32 inputs).
// Each operand lives in global memory either
//   KMAJOR  -- rows are the M (or N) index, K contiguous   (weight, hidden as
//              read by the logit GEMM), or
//   MNMAJOR -- rows are the K index, M (or N) contiguous   (hidden, weight and
//              the dlogits scratch as read by the two gradient contractions).
// Both are staged through LDS as they lie in memory; MNMAJOR fragments are
// read with ds_read_b64_tr_b16, which transposes 16-bit elements across each
// group of 16 lanes, so no operand is ever transposed in global memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Logit value given to vocabulary rows past V.  Finite, so that e * z stays
// finite when e underflows to 0; any real row outweighs it in every merge.
// A power of two, so that kMasked * log2(e) is exact in fp32: exponents are
// formed as fma(z, log2e, -m*log2e), and for z = m = kMasked that must give
// exactly 0 (a rounding residual of a 1e30-sized product would not).
constexpr float kMasked = -0x1p100f;

constexpr int kBM = 256;            // tile rows (A operand)
constexpr int kBN = 256;            // tile cols (B operand)
constexpr int kBKB = 128;           // bytes of K per pipeline stage per row
constexpr int kThreads = 256;       // 4 waves
constexpr int kOperandStage = kBM * kBKB;           // 32 KiB
constexpr int kStageBytes = 2 * kOperandStage;      // A + B, 64 KiB
constexpr int kMainLds = 2 * kStageBytes;           // double buffer, 128 KiB
constexpr uint32_t kOob = 0x80000000u;              // buffer offset that reads 0

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// cap * tanh(v / cap) written as cap - 2 cap / (exp(2 v / cap) + 1); saturates
// to +-cap when the exponential over- or underflows.
__device__ __forceinline__ float softcap_apply(float v, float two_log2e_over_cap, float cap,
                                               float two_cap) {
  float e = fast_exp2(v * two_log2e_over_cap);
  return fmaf(-two_cap, fast_rcp(e + 1.0f), cap);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<bf16> {
  static constexpr int kSize = 2;
  static constexpr int kPerChunk = 8;     // elements per 16-byte chunk
};
template <> struct ElemTraits<float> {
  static constexpr int kSize = 4;
  static constexpr int kPerChunk = 4;
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Row (within a 128-row wave block) held by accumulator register r of MFMA
// tile mi for this lane:  mi*32 + 8*(r/4) + 4*(lane/32) + r%4.
__device__ __forceinline__ int acc_row(int mi, int r, int lane) {
  return mi * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

// ---------------------------------------------------------------------------
// Operand descriptors and loaders.  Loads go straight from global memory into
// LDS (buffer_load_dwordx4 ... lds): one wave instruction fills 1 KiB of LDS,
// lane l writing bytes [16 l, 16 l + 16).  The LDS layouts are swizzled, so
// each lane fetches the global chunk that belongs at its LDS position.
// Anything past `nrec` (rows past the end, masked columns, the K tail) reads
// as zero through the buffer's range check.
// ---------------------------------------------------------------------------
struct OperandDesc {
  const char* base;      // KMAJOR: row 0 of the tile; MNMAJOR: element (k=0, col 0 of tile)
  uint32_t ld_bytes;     // bytes between consecutive rows in global memory
  uint32_t nrec;         // bytes readable from base; beyond reads as 0
  int cols_valid;        // MNMAJOR: valid tile columns (M side); unused for KMAJOR
  int k_bytes;           // KMAJOR: valid K extent in bytes
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor as four scalar words: base address, stride 0, byte range,
// raw 32-bit format.  Loads at offsets >= nbytes return 0.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = 0x00020000;
  return r;
}

// 16-byte direct-to-LDS load: lane l's 16 bytes land at LDS byte address
// lds_addr + 16 l.  Issued through inline assembly so that the compiler does
// not treat every later LDS read as dependent on it; the caller waits for
// vmcnt(0) and synchronises before the data is read.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const LDS_AS char*)p);
}

template <typename T, bool KMAJOR>
struct OperandLoader {
  i32x4 rsrc;
  uint32_t voff0, voff1;  // lane offsets (even / odd 1 KiB block for bf16 MNMAJOR)
  int kc_bytes;           // KMAJOR: this lane's logical chunk column in bytes
  int k_bytes;
  uint32_t ld_bytes;
  int wave;

  __device__ __forceinline__ void init(const OperandDesc& d, int tid) {
    rsrc = make_rsrc_words(d.base, d.nrec);
    k_bytes = d.k_bytes;
    ld_bytes = d.ld_bytes;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    if constexpr (KMAJOR) {
      // block b holds rows 8b..8b+7; lane l -> row 8b + l/8, LDS slot l%8
      const int row = l >> 3;
      const int kc = (l & 7) ^ (row & 7);
      kc_bytes = kc * 16;
      voff0 = voff1 = (uint32_t)row * d.ld_bytes + kc * 16;
    } else if constexpr (sizeof(T) == 2) {
      // block b holds rows 2b, 2b+1 (512 B each); lane l -> row 2b + l/32, slot l%32
      kc_bytes = 0;
      const int half = l >> 5, slot = l & 31;
      const int c_even = slot ^ (4 * (half & 3));          // row & 3 = half      (b even)
      const int c_odd = slot ^ (4 * ((2 + half) & 3));     // row & 3 = 2 + half  (b odd)
      voff0 = c_even * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c_even * 16 : kOob;
      voff1 = c_odd * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c_odd * 16 : kOob;
    } else {
      // fp32: block b is row b (1 KiB); lane l -> chunk l
      kc_bytes = 0;
      voff0 = voff1 = l * 4 < d.cols_valid ? (uint32_t)l * 16 : kOob;
    }
  }

  // Issue the 8 direct-to-LDS loads of stage kt (this wave's 8 KiB).
  __device__ __forceinline__ void load(int kt, char* stage) const {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int b = wave * 8 + i;            // 1 KiB block of the 32 KiB operand stage
      uint32_t voff, soff;
      if constexpr (KMAJOR) {
        const uint32_t k0 = (uint32_t)kt * kBKB;
        voff = (int)k0 + kc_bytes < k_bytes ? voff0 : kOob;
        soff = k0 + (uint32_t)(8 * b) * ld_bytes;
      } else if constexpr (sizeof(T) == 2) {
        voff = (i & 1) ? voff1 : voff0;
        soff = ((uint32_t)kt * 64 + 2 * b) * ld_bytes;
      } else {
        voff = voff0;
        soff = ((uint32_t)kt * 32 + b) * ld_bytes;
      }
      dma16(rsrc, __builtin_amdgcn_readfirstlane(lds_addr_of(stage) + b * 1024), voff, soff);
    }
  }
};

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// ---------------------------------------------------------------------------
// Fragment reads from LDS.  Sub-step s covers K elements [16s, 16s+16) (bf16)
// or [8s, 8s+8) (fp32) of the stage.  `c0` is the first tile row/column of the
// 32-wide MFMA fragment.  Lane l gets row/column c0 + l%32 and K values
// 16s + 8(l/32) + 0..7 (bf16) -- the same K order for both layouts, so any
// pairing of a KMAJOR and an MNMAJOR operand contracts consistently.
// ---------------------------------------------------------------------------
template <typename T, bool KMAJOR> struct Frag;

template <> struct Frag<bf16, true> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int row = c0 + (lane & 31);
    const int kc = 2 * s + (lane >> 5);
    const int off = row * kBKB + ((kc ^ (row & 7)) << 4);
    return *reinterpret_cast<const bf16x8*>(op + off);
  }
};

template <> struct Frag<bf16, false> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int g = lane >> 4, kk = lane & 15, j = kk >> 2, q = kk & 3;
    const int row = 16 * s + 8 * (g >> 1) + j;
    const int u = (c0 >> 2) + 4 * (g & 1) + q;
    const int off = row * 512 + ((u ^ (j << 3)) << 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(op + off));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(op + off + 4 * 512));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

// fp32: lane half h reads K chunk (2s + h), i.e. K = (2s+h)*4 + j for j = 0..3.
template <> struct Frag<float, true> {
  typedef f32x4 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int row = c0 + (lane & 31);
    const int kc = 2 * s + (lane >> 5);
    const int off = row * kBKB + ((kc ^ (row & 7)) << 4);
    return *reinterpret_cast<const f32x4*>(op + off);
  }
};

template <> struct Frag<float, false> {
  typedef f32x4 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int col = c0 + (lane & 31);
    const int k0 = (2 * s + (lane >> 5)) * 4;
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = *reinterpret_cast<const float*>(op + (k0 + j) * 1024 + col * 4);
    return v;
  }
};

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int j = 0; j < 4; j++) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS: two pipeline stages of 64 KiB; kernels also use stage 0 as epilogue
// scratch after the main loop.
// ---------------------------------------------------------------------------
static __shared__ __attribute__((aligned(1024))) char g_lds[kMainLds];
#define g_stage0 (g_lds)

template <typename T, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void compute_stage(const char* stage, int wm, int wn, int lane,
                                              f32x16 (&acc)[4][4]) {
  const char* opA = stage;
  const char* opB = stage + kOperandStage;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    typename Frag<T, A_KMAJOR>::type fa[4];
    typename Frag<T, B_KMAJOR>::type fb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) fa[i] = Frag<T, A_KMAJOR>::read(opA, wm * 128 + i * 32, s, lane);
#pragma unroll
    for (int i = 0; i < 4; i++) fb[i] = Frag<T, B_KMAJOR>::read(opB, wn * 128 + i * 32, s, lane);
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
      for (int ni = 0; ni < 4; ni++) mma(acc[mi][ni], fa[mi], fb[ni]);
  }
}

// ---------------------------------------------------------------------------
// The main loop: stage kt+1 streams into one buffer while stage kt is
// multiplied out of the other.  acc must be zeroed by the caller.  Ends with
// a barrier, so the caller may reuse LDS afterwards.
// ---------------------------------------------------------------------------
template <typename T, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void tile_mainloop(const OperandDesc& da, const OperandDesc& db, int KT,
                                              f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  OperandLoader<T, A_KMAJOR> la;
  OperandLoader<T, B_KMAJOR> lb;
  la.init(da, tid);
  lb.init(db, tid);

  if (KT > 0) {
    la.load(0, g_lds);
    lb.load(0, g_lds + kOperandStage);
  }
  wait_loads();
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      char* nxt = g_lds + ((kt + 1) & 1) * kStageBytes;
      la.load(kt + 1, nxt);
      lb.load(kt + 1, nxt + kOperandStage);
    }
    compute_stage<T, A_KMAJOR, B_KMAJOR>(g_lds + (kt & 1) * kStageBytes, wm, wn, lane, acc);
    wait_loads();
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mi = 0; mi < 4; mi++)
#pragma unroll
    for (int ni = 0; ni < 4; ni++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;
}

// Workgroups are dispatched to the 8 XCDs round-robin (b -> b % 8).  Renumber
// so that each XCD receives one contiguous range of logical ids.
__device__ __forceinline__ int xcd_logical_id(int b, int nwg) {
  const int q = nwg >> 3, r = nwg & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Grouped tile order: consecutive ids walk `gm` M-tiles, then the next N-tile,
// so that the ~32 tiles one XCD runs at once share A and B tiles in its L2.
__device__ __forceinline__ void grouped_tile(int id, int n_m, int n_n, int gm, int& tm, int& tn) {
  const int per_group = gm * n_n;
  const int group = id / per_group;
  const int first = group * gm;
  const int size = min(n_m - first, gm);
  const int in = id - group * per_group;
  tm = first + in % size;
  tn = in / size;
}

template <typename T> __device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<bf16>(const bf16* p, int64_t i) { return (float)p[i]; }

}  // namespace flce
