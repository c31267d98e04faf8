// Device-side building blocks for the fused linear cross-entropy kernels
// (gfx950 / CDNA4): vector types, buffer loads, fast transcendentals and the
// shared 256x256 MFMA tile main loop.
//
// Tile main loop: C[256 x 256] += A[256 x K] . B[256 x K]^T with fp32
// accumulation, 8 waves (2 along M x 4 along N, two per SIMD), each wave
// owning a 128 x 64 block as 8 x 4 tiles of v_mfma_f32_16x16x32_bf16
// (v_mfma_f32_16x16x32_f16 for fp16, v_mfma_f32_16x16x4_f32 for fp32 inputs).
// The 16x16 tiles move fewer register-file bytes per flop than 32x32x16 ones
// (under the board's power cap that is clock); in these kernels they measured
// within 1% of the 32x32 tiles, a little ahead.  Two waves per SIMD keep
// enough LDS reads in flight to feed the matrix cores (one wave per SIMD with
// 128 x 128 wave tiles measured 9% slower).
//
// Both operands are staged through LDS.  Each lives in global memory either
//   KMAJOR  -- rows are the M (or N) index, K contiguous   (weight and hidden
//              as read by the logit GEMM, hidden^T, the dlogits scratch as
//              read by the grad_hidden contraction), or
//   MNMAJOR -- rows are the K index, M (or N) contiguous   (the weight and
//              the dlogits scratch as read by the gradient contractions);
// MNMAJOR fragments are read with ds_read_b64_tr_b16, which transposes
// 16-bit elements across each group of 16 lanes.
//
// K order: a stage is 128 bytes of K per row (64 bf16 or fp16 / 32 fp32), eight
// 16-byte chunks.  In sub-step s (0..1) the lanes of 16-lane group g (lane / 16)
// contract chunk 4s + g.  Any order is correct as long as both operands use the
// same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

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
constexpr int kBKB = 128;           // bytes of K per pipeline stage per row (64 16-bit / 32 fp32)
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kWaves = kWavesM * kWavesN;        // 8 waves
constexpr int kThreads = 64 * kWaves;            // 512 threads
constexpr int kMI = 8, kNI = 4;                  // 16 x 16 MFMA tiles per wave (M x N)
constexpr int kWaveM = 16 * kMI, kWaveN = 16 * kNI;   // 128 x 64
constexpr int kOperandStage = kBM * kBKB;           // one operand's stage: 32 KiB
constexpr int kStageBytes = 2 * kOperandStage;      // A + B: 64 KiB
constexpr int kMainLds = 2 * kStageBytes;           // double buffer, 128 KiB
constexpr int kLoadWaves = kWaves / 2;                          // waves that issue the stage loads
constexpr int kLoadBlocks = kOperandStage / 1024 / kLoadWaves;  // 1 KiB DMA blocks per loading wave per operand
constexpr int kSubsteps = 2;
constexpr uint32_t kOob = 0x80000000u;              // buffer offset that reads 0

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Accumulator layout: acc[mi][ni] (4 fp32) holds, for this lane, rows
// acc_row(mi, r, lane) = mi*16 + 4*(lane/16) + r (r = 0..3, within the wave's
// 128-row block) of column acc_col(ni, lane) = ni*16 + lane%16 (within its 64).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef f32x4 Acc;
__device__ __forceinline__ int acc_row(int mi, int r, int lane) { return mi * 16 + ((lane >> 4) << 2) + r; }
__device__ __forceinline__ int acc_col(int ni, int lane) { return ni * 16 + (lane & 15); }

// ---------------------------------------------------------------------------
// Operand descriptor and loader.  Loads go straight from global memory
// into LDS (buffer_load_dwordx4 ... lds): one wave instruction fills 1 KiB of
// LDS, lane l writing bytes [16 l, 16 l + 16).  The LDS layouts are swizzled,
// so each lane fetches the global chunk that belongs at its LDS position.
// Anything past `nrec` (rows past the end, masked columns) reads as zero
// through the buffer's range check.
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
// vmcnt(0) and synchronises before the data is read.  The statement sets M0
// (the LDS address of a direct-to-LDS load) itself.  M0 is a reserved register
// that a clobber list cannot protect, so correctness rests on the compiler
// keeping no value of its own in M0 in these kernels; a CPU test compiles the
// device code and checks that every M0 access is one of these pairs.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

// 4-byte direct-to-LDS load used only to pull a line into L2: every lane's
// word lands in a small sink that is never read.  Offsets >= the descriptor's
// range (kOob) fetch nothing.
__device__ __forceinline__ void dma4_sink(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

// Orders the LDS accesses of one wave whose lanes exchange data through LDS:
// every access before it, by any lane of the wave, takes effect before any
// access after it.  A wave's LDS instructions execute in issue order, so this
// only stops the compiler from moving reads above another lane's writes (or
// writes above another lane's reads); it emits no wait of its own.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const LDS_AS char*)p);
}

// One wave copies `nbytes` (a multiple of 256) from global `src` to LDS `dst`
// by direct-to-LDS loads, 4 bytes per lane per 256-byte block; bytes at or
// past `valid_bytes` arrive as 0.  The caller waits for vmcnt and
// synchronises before reading (the main loop's first stage wait does both).
__device__ __forceinline__ void dma_vector(const void* src, uint32_t valid_bytes, char* dst, int nbytes,
                                           int lane) {
  const i32x4 r = make_rsrc_words(src, valid_bytes);
  const uint32_t base = lds_addr_of(dst);
  for (int b = 0; b < nbytes; b += 256) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(base + b)), "v"((uint32_t)(b + 4 * lane)), "s"(r)
                 : "memory");
  }
}

// Four consecutive entries of a vector staged in LDS, widened to fp32.
template <typename T> __device__ __forceinline__ void lds_vec4(const char* v, int i, float* out);
template <> __device__ __forceinline__ void lds_vec4<float>(const char* v, int i, float* out) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(v + 4 * i);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = x[j];
}
template <> __device__ __forceinline__ void lds_vec4<bf16>(const char* v, int i, float* out) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(v + 2 * i);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = (float)x[j];
}
template <> __device__ __forceinline__ void lds_vec4<f16>(const char* v, int i, float* out) {
  const f16x4 x = *reinterpret_cast<const f16x4*>(v + 2 * i);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = (float)x[j];
}

template <typename T, bool KMAJOR>
struct OperandLoader {
  i32x4 rsrc;
  uint32_t voff0, voff1;  // lane offsets for even / odd 1 KiB blocks
  uint32_t voff2, voff3;  // M/N-major 16-bit: the same for blocks with bit 2 of the block index set
  int kc_bytes0, kc_bytes1;   // KMAJOR: the lane's logical chunk column (even / odd blocks)
  int k_bytes;
  uint32_t ld_bytes;
  int wave;

  __device__ __forceinline__ void init(const OperandDesc& d, int tid) {
    rsrc = make_rsrc_words(d.base, d.nrec);
    // (uniform by construction; said so, for descriptors the compiler cannot see through)
    k_bytes = __builtin_amdgcn_readfirstlane(d.k_bytes);
    ld_bytes = __builtin_amdgcn_readfirstlane(d.ld_bytes);
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    if constexpr (KMAJOR) {
      // block b holds rows 8b..8b+7 (128 B each); lane l -> row 8b + l/8,
      // LDS slot l%8, which holds logical chunk slot ^ ((row >> 1) & 7)
      // = slot ^ ((4b + l/16) & 7): the pattern depends on the parity of b
      const int row = l >> 3, slot = l & 7;
      const int kc0 = slot ^ ((l >> 4) & 7);
      const int kc1 = slot ^ ((4 + (l >> 4)) & 7);
      kc_bytes0 = kc0 * 16;
      kc_bytes1 = kc1 * 16;
      voff0 = (uint32_t)row * d.ld_bytes + kc0 * 16;
      voff1 = (uint32_t)row * d.ld_bytes + kc1 * 16;
    } else if constexpr (sizeof(T) == 2) {
      // block b holds rows 2b, 2b+1 (512 B each); lane l -> row 2b + l/32,
      // LDS slot l%32, which holds the row's 16-byte column chunk
      // slot ^ (4 (row & 3)) ^ (2 ((row >> 3) & 1)); row & 3 follows the parity
      // of b, and (row >> 3) & 1 = (b >> 2) & 1
      kc_bytes0 = kc_bytes1 = 0;
      const int half = l >> 5, slot = l & 31;
      const int c0 = slot ^ (4 * half);                 // b even, (b >> 2) even: row & 3 = half
      const int c1 = slot ^ (4 * (2 + half));           // b odd: row & 3 = 2 + half
      const int c2 = c0 ^ 2, c3 = c1 ^ 2;               // the same with (row >> 3) odd
      voff0 = c0 * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c0 * 16 : kOob;
      voff1 = c1 * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c1 * 16 : kOob;
      voff2 = c2 * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c2 * 16 : kOob;
      voff3 = c3 * 8 < d.cols_valid ? (uint32_t)half * d.ld_bytes + c3 * 16 : kOob;
    } else {
      // fp32: block b is row b (1 KiB); lane l -> chunk l
      kc_bytes0 = kc_bytes1 = 0;
      voff0 = voff1 = l * 4 < d.cols_valid ? (uint32_t)l * 16 : kOob;
    }
  }

  // L2 prefetch of 128-byte line j (0..255) of stage kt: K-major row j;
  // M/N-major 16-bit row 64 kt + j/4, column block j%4.  Inactive lanes fetch
  // nothing.
  __device__ __forceinline__ void prefetch_line(int kt, int j, bool active, uint32_t sink) const {
    uint32_t voff;
    if constexpr (KMAJOR) voff = (uint32_t)j * ld_bytes + (uint32_t)kt * kBKB;
    else voff = (uint32_t)(kt * (kBKB / 2) + (j >> 2)) * ld_bytes + (uint32_t)(j & 3) * 128;
    dma4_sink(rsrc, sink, active ? voff : kOob);
  }

  // Issue this wave's direct-to-LDS loads of stage kt.  Only the first half
  // of the waves load (kLoadBlocks blocks each): the two waves that share a
  // SIMD are not issued evenly (the older one, wm = 0, runs ahead and then
  // waits at the stage barrier), so the loads go to the waves with slack.
  __device__ __forceinline__ void load(int kt, char* stage) const {
    if (wave >= kLoadWaves) return;
#pragma unroll
    for (int i = 0; i < kLoadBlocks; i++) {
      const int b = wave * kLoadBlocks + i;   // 1 KiB block of the stage; parity = parity of i
      uint32_t voff, soff;
      if constexpr (KMAJOR) {
        const uint32_t k0 = (uint32_t)kt * kBKB;
        voff = (i & 1) ? ((int)k0 + kc_bytes1 < k_bytes ? voff1 : kOob)
                       : ((int)k0 + kc_bytes0 < k_bytes ? voff0 : kOob);
        soff = k0 + (uint32_t)(8 * b) * ld_bytes;
      } else if constexpr (sizeof(T) == 2) {
        static_assert(kLoadBlocks % 8 == 0, "bit 2 of the block index must be that of i");
        voff = (i & 4) ? ((i & 1) ? voff3 : voff2) : ((i & 1) ? voff1 : voff0);
        soff = ((uint32_t)kt * (kBKB / 2) + 2 * b) * ld_bytes;
      } else {
        voff = voff0;
        soff = ((uint32_t)kt * (kBKB / 4) + b) * ld_bytes;
      }
      dma16(rsrc, __builtin_amdgcn_readfirstlane(lds_addr_of(stage) + b * 1024), voff, soff);
    }
  }
};

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// vmcnt(1): all but the most recent vector-memory load have completed (loads
// complete in issue order)
__device__ __forceinline__ void wait_vmcnt_1() { __builtin_amdgcn_s_waitcnt(0x0F71); }

// ---------------------------------------------------------------------------
// LDS fragment reads.  `c0` is the first tile row/column of the 16-wide MFMA
// fragment; lane l gets row/column c0 + l%16 and the 16 bytes of K chunk
// 4s + l/16 (sub-step s).
// ---------------------------------------------------------------------------
template <typename T, bool KMAJOR> struct Frag;

// KMAJOR rows are 128 B; the 16-byte chunk kc of row r sits at slot
// kc ^ ((r >> 1) & 7).  A ds_read_b128 is served 16 lanes (16 consecutive
// rows, two per 256-byte bank line, one chunk) at a time, and this spreads them
// over all 64 banks.
// (The same reads serve both 16-bit types; only the register type differs.)
template <typename V8> struct Frag16K {
  typedef V8 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int row = c0 + (lane & 15);
    const int kc = 4 * s + (lane >> 4);
    const int off = row * kBKB + ((kc ^ ((row >> 1) & 7)) << 4);
    return *reinterpret_cast<const V8*>(op + off);
  }
};
template <> struct Frag<bf16, true> : Frag16K<bf16x8> {};
template <> struct Frag<f16, true> : Frag16K<f16x8> {};

// MNMAJOR 16-bit rows are 512 B (256 elements); 8-byte unit u of row r sits at
// unit u ^ ((r & 3) << 3) ^ (((r >> 3) & 1) << 2).  ds_read_b64_tr_b16 gives
// lane i of each 16-lane group element i%4 of the 8-byte pieces that lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of the group addressed.  So lane a of
// group g addresses row 32s + 8g + a/4 (+ 4 for the second read) at columns
// c0 + 4(a%4) .. + 3, and lane i receives column c0 + i of K rows
// 32s + 8g .. + 7: its K chunk 4s + g.  The 32 lanes of two groups served
// together read 4 rows each, one of each row & 3, and the two groups' rows
// differ in bit 3: all 32 pieces fall in distinct banks.
template <typename V8> struct Frag16MN {
  typedef V8 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int g = lane >> 4, a = lane & 15;
    const int row = 32 * s + 8 * g + (a >> 2);
    const int u = (c0 >> 2) + (a & 3);
    const int off = row * 512 + ((u ^ ((row & 3) << 3) ^ ((g & 1) << 2)) << 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(op + off));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(op + off + 4 * 512));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(V8, v);
  }
};
template <> struct Frag<bf16, false> : Frag16MN<bf16x8> {};
template <> struct Frag<f16, false> : Frag16MN<f16x8> {};

// fp32: a stage row is eight 16-byte chunks of 4 floats; lane group g holds
// chunk 4s + g, and v_mfma_f32_16x16x4_f32 number j of the sub-step contracts
// element j of every group's chunk (K = 4(4s + g) + j over the four groups).
template <> struct Frag<float, true> {
  typedef f32x4 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int row = c0 + (lane & 15);
    const int kc = 4 * s + (lane >> 4);
    const int off = row * kBKB + ((kc ^ ((row >> 1) & 7)) << 4);
    return *reinterpret_cast<const f32x4*>(op + off);
  }
};

// fp32 MNMAJOR rows are 1 KiB (256 floats), unswizzled.
template <> struct Frag<float, false> {
  typedef f32x4 type;
  __device__ __forceinline__ static type read(const char* op, int c0, int s, int lane) {
    const int col = c0 + (lane & 15);
    const int k0 = (4 * s + (lane >> 4)) * 4;
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = *reinterpret_cast<const float*>(op + (k0 + j) * 1024 + col * 4);
    return v;
  }
};

__device__ __forceinline__ void mma(Acc& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(Acc& c, const f16x8& a, const f16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(Acc& c, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int j = 0; j < 4; j++) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS: two pipeline stages of 64 KiB (A then B); kernels also use stage 0 as
// epilogue scratch after the main loop.
// ---------------------------------------------------------------------------
static __shared__ __attribute__((aligned(1024))) char g_lds[kMainLds];
#define g_stage0 (g_lds)

// Fragments in registers: the A fragments of one sub-step (32 deep in K, 16
// for fp32) plus one spare, and the B fragments of two sub-steps, the current
// and the next.  Row tile mi < kMI - 1 keeps its A fragment in a[mi], which is
// overwritten with the next sub-step's as soon as the MFMAs of that row have
// issued.  The last row tile alternates between a[kMI - 1] (sub-step 0) and
// the spare a[kMI] (sub-step 1), so that its next fragment is read while the
// MFMAs still run rather than after them.  In all kMI + 1 + 2 kNI fragments
// of 4 VGPRs (68) next to the accumulator's 128.
template <typename T, bool A_KMAJOR, bool B_KMAJOR>
struct MainFrags {
  typename Frag<T, A_KMAJOR>::type a[kMI + 1];
  typename Frag<T, B_KMAJOR>::type b[2][kNI];

  __device__ __forceinline__ void read_a(const char* stage, int s, int mi, int slot, int wm, int lane) {
    a[slot] = Frag<T, A_KMAJOR>::read(stage, wm * kWaveM + mi * 16, s, lane);
  }
  template <int BUF>
  __device__ __forceinline__ void read_b(const char* stage, int s, int wn, int lane) {
#pragma unroll
    for (int i = 0; i < kNI; i++)
      b[BUF][i] = Frag<T, B_KMAJOR>::read(stage + kOperandStage, wn * kWaveN + i * 16, s, lane);
  }
};

// Shared-tile L2 prefetch.  The 32 workgroups that one XCD runs at once
// cover a few A tiles and a few B tiles, each read by several of them in step.
// Workgroup `a_rank` of the `a_n` that read the same A tile fetches its
// 1/a_n of the tile's lines kPrefetchAhead stages ahead, one iteration before
// the stage's loads are issued (likewise for B), so that the others' loads
// hit in L2 instead of all waiting on the same misses.
// a_n = 0 (or b_n = 0) turns it off for that operand.
struct L2Share {
  int a_rank, a_n, b_rank, b_n;
};
constexpr int kPrefetchAhead = 3;
static __shared__ __attribute__((aligned(256))) char g_prefetch_sink[256];

// Issues this wave's share of the prefetch of stage kt (16-bit types only); returns
// whether the wave issued a load (wave-uniform).
template <typename T, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ bool prefetch_stage(const OperandLoader<T, A_KMAJOR>& la,
                                               const OperandLoader<T, B_KMAJOR>& lb, const L2Share& sh,
                                               int kt, int wave, int lane) {
  if constexpr (sizeof(T) != 2) {
    return false;
  } else {
    // the loading waves prefetch too: waves 0-1 take A's lines, waves 2-3
    // B's, 64 each (a share of at most 128 lines: n >= 2)
    if (wave >= kLoadWaves) return false;
    const bool is_a = wave < kLoadWaves / 2;
    const int n = is_a ? sh.a_n : sh.b_n;
    if (n < 2) return false;
    const int rank = is_a ? sh.a_rank : sh.b_rank;
    const int first = rank * 256 / n, count = (rank + 1) * 256 / n - first;
    const int off = (wave % (kLoadWaves / 2)) * 64;
    if (off >= count) return false;
    const uint32_t sink = __builtin_amdgcn_readfirstlane(lds_addr_of(g_prefetch_sink));
    const bool active = off + lane < count;
    if (is_a) la.prefetch_line(kt, first + off + lane, active, sink);
    else lb.prefetch_line(kt, first + off + lane, active, sink);
    return true;
  }
}

// One sub-step: the MFMAs of the fragments in registers (B buffer CUR, the
// last row tile's A in slot kMI - 1 + CUR) while the next sub-step's are read
// (sub-step s of `stage`): B into the other buffer during row tile 0, A row
// tile mi - 1 during row tile mi, and the last row tile's into the slot this
// sub-step does not use, halfway through.  Scheduling barriers fence the row
// tiles, so that no read is hoisted above the MFMAs whose registers it
// overwrites (which would need more registers) and none is sunk to right
// before its first use (where the wave would wait on it).
template <int CUR, typename T, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void substep(MainFrags<T, A_KMAJOR, B_KMAJOR>& f, const char* stage, int s, int wm,
                                        int wn, int lane, Acc (&acc)[kMI][kNI]) {
  constexpr int kLastCur = kMI - 1 + CUR, kLastNext = kMI - CUR;
  __builtin_amdgcn_sched_barrier(0);
  f.template read_b<1 - CUR>(stage, s, wn, lane);
#pragma unroll
  for (int ni = 0; ni < kNI; ni++) mma(acc[0][ni], f.a[0], f.b[CUR][ni]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 1; mi < kMI; mi++) {
    f.read_a(stage, s, mi - 1, mi - 1, wm, lane);
    if (mi == kMI / 2) f.read_a(stage, s, kMI - 1, kLastNext, wm, lane);
    const int slot = mi == kMI - 1 ? kLastCur : mi;
    // odd row tiles walk the columns backwards, so that the MFMAs on either side
    // of a row boundary share their B fragment (fewer operand bits switch: the
    // step is power-bound, and this measured 1% faster)
#pragma unroll
    for (int nj = 0; nj < kNI; nj++) {
      const int ni = (mi & 1) ? kNI - 1 - nj : nj;
      mma(acc[mi][ni], f.a[slot], f.b[CUR][ni]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// The main loop.  Global -> LDS: two stage buffers.  Stage kt + 2 is loaded
// into stage kt's buffer as soon as the barrier in the middle of iteration kt
// has passed (no wave reads that buffer after it), so each stage's loads have
// a whole iteration, two sub-steps of MFMAs, to land before the barrier that
// waits for them.  LDS -> registers: the fragments of sub-step 1 are read
// while the 32 MFMAs of sub-step 0 run, and those of the first sub-step of the
// next stage right after the barrier, under the MFMAs of sub-step 1 of the
// current one.  acc must be zeroed by the caller.  Every LDS read whose value
// is used completes before the last barrier (the reads after it fill
// fragments that are discarded), and no load is in flight when the loop
// returns, so the caller may write LDS at once.
// ---------------------------------------------------------------------------
template <typename T, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void tile_mainloop(const OperandDesc& da, const OperandDesc& db, int KT,
                                              const L2Share& sh, Acc (&acc)[kMI][kNI]) {
  // (opaque, so that a kernel calling this in a loop forms the per-thread
  // offsets afresh each time instead of keeping them in registers around it)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;

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
  if (KT <= 0) return;
  if (KT > 1) {
    la.load(1, g_lds + kStageBytes);
    lb.load(1, g_lds + kStageBytes + kOperandStage);
  }

  MainFrags<T, A_KMAJOR, B_KMAJOR> f;
  f.template read_b<0>(g_lds, 0, wn, lane);
#pragma unroll
  for (int mi = 0; mi < kMI; mi++) f.read_a(g_lds, 0, mi, mi, wm, lane);
  bool pf = false;   // this wave's most recent vector-memory instruction is an L2 prefetch
  for (int kt = 0; kt < KT; ++kt) {
    char* cur = g_lds + (kt & 1) * kStageBytes;
    const char* nxt = g_lds + ((kt + 1) & 1) * kStageBytes;
    substep<0>(f, cur, 1, wm, wn, lane, acc);
    // stage kt+1 (loaded during the previous iteration) must be in LDS; a
    // prefetch issued after it may still be in flight
    if (pf) wait_vmcnt_1();
    else wait_loads();
    __syncthreads();
    if (kt + 2 < KT) {
      la.load(kt + 2, cur);
      lb.load(kt + 2, cur + kOperandStage);
    }
    pf = kt + kPrefetchAhead < KT &&
         prefetch_stage<T, A_KMAJOR, B_KMAJOR>(la, lb, sh, kt + kPrefetchAhead, wave, lane);
    // after the last stage this reads stale (in-bounds) LDS that is never used
    substep<1>(f, nxt, 0, wm, wn, lane, acc);
  }
}

__device__ __forceinline__ void zero_acc(Acc (&acc)[kMI][kNI]) {
#pragma unroll
  for (int mi = 0; mi < kMI; mi++)
#pragma unroll
    for (int ni = 0; ni < kNI; ni++) acc[mi][ni] = Acc{0.0f, 0.0f, 0.0f, 0.0f};
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

// No L2 prefetch (the logit-gradient and grad_weight kernels measured faster
// without it: their stage loads, issued a full iteration ahead, already find
// their lines in L2 often enough, and the prefetch costs issue slots).
__device__ __forceinline__ L2Share no_share() {
  L2Share s;
  s.a_rank = s.a_n = s.b_rank = s.b_n = 0;
  return s;
}

// Prefetch shares under grouped_tile(..., 4, ...) when one XCD runs 32
// consecutive ids at a time: 4 M-tiles x 8 N-tiles, so each A tile is read by
// the 8 workgroups of distinct tn and each B tile by the 4 of distinct tm.
__device__ __forceinline__ L2Share grouped_share(int tm, int tn) {
  L2Share s;
  s.a_rank = tn & 7;
  s.a_n = 8;
  s.b_rank = tm & 3;
  s.b_n = 4;
  return s;
}

template <typename T> __device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<bf16>(const bf16* p, int64_t i) { return (float)p[i]; }
template <> __device__ __forceinline__ float load_elem<f16>(const f16* p, int64_t i) { return (float)p[i]; }

// Target i of an int64 or int32 target array.
__device__ __forceinline__ int64_t load_target(const void* p, int64_t i, int int32) {
  return int32 ? (int64_t) reinterpret_cast<const int32_t*>(p)[i] : reinterpret_cast<const int64_t*>(p)[i];
}

}  // namespace flce
