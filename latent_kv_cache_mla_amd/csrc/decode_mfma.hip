// decode_mfma.hip — split-KV absorbed-MLA decode on the gfx950 matrix cores
// for the DeepSeek attention shape (d_c = 512, d_R = 64, bf16 cache).
//
// What it computes (per query row r = (query token m, head i) and cached
// token j of one sequence):
//   s_j = scale * (q_abs[r] . c_j + q_rope[r] . k^R_j)      ([LLMsBlog]
//        "Multi-Head Latent Attention: How Low-Rank KV Compression Scales LLM
//        Serving", "Query Key Absorption"; [Mishra] "Multi-head Latent
//        Attention", "Step 4: decoupled RoPE": content and rope dot products
//        add over the concatenated 576-lane entry)
//   o[r] = sum_j softmax(s)_j c_j                              ([Zhang]
//        "Multi-head latent attention", "Value absorption: weight and sum
//        first, project after": the cached latent is the value)
// The 128 query rows of a workgroup form the dense dimension of both
// products, so the cached page is read from HBM once and shared by all rows.
//
// Work decomposition:
//   * workgroup = (page range g, row group of 128 rows); 4 wavefronts, each
//     owns 32 rows; one workgroup per CU (LDS and registers are sized for
//     it: O^T fills the 256 accumulation registers, Q^T and the scores live
//     in the 256 vector registers).
//   * block ids are mapped so that each XCD (ids congruent mod 8) receives a
//     contiguous run of ranges: the ranges of one sequence, and the row
//     groups of one range, then share that XCD's L2 for the queries and the
//     pages.
//   * the cache streams through LDS in 32-token chunks (half a page) held in
//     a ring of four stages. Chunks are copied HBM -> LDS with direct
//     global-to-LDS loads (no register round trip); two chunks are always in
//     flight while one is being multiplied against the queries and the one
//     before it against the probabilities.
//   * scores: S^T[32 tok x 32 rows] = K[32 x 576] Q^T[576 x 32] with
//     v_mfma_f32_32x32x16_bf16, tokens as the M dimension: the A operand is
//     read from LDS (16 bytes per lane), Q^T stays in registers all along.
//     In this orientation each lane holds 16 tokens of one row, so the row
//     max and sum are in-lane but for one exchange between the wave halves.
//     The score MFMAs are issued as single asm instructions with
//     vector-register constraints: that keeps the score accumulator out of
//     the accumulation registers, which O^T fills.
//   * software pipeline per chunk k: the score MFMAs of chunk k are
//     interleaved with the vector-ALU softmax of chunk k - 1 (scale, mask,
//     row max, exponentials, bf16 packing), then the weighted sum of chunk
//     k - 1 runs on the matrix unit. The matrix unit is thus never idle
//     while the softmax is computed.
//   * online softmax in base 2 with a lazy reference: probabilities are taken
//     relative to a running max m that only moves when a chunk's max exceeds
//     it by more than 2^8. Instead of rescaling O then (which would make the
//     compiler keep the 128 accumulator registers on the VALU side of the
//     register file), the workgroup restarts the piece from its first chunk
//     with the raised m: rare, and exact (O and l are rebuilt against one
//     reference).
//   * weighted sum: O^T[512 x 32] += V^T[512 x 32] P^T[32 x 32]; P^T comes
//     straight from the score registers (converted to bf16), and V^T is the
//     same LDS chunk read with the LDS transpose load (ds_read_b64_tr_b16):
//     keys and values are never materialised.
//   * the LDS chunk layout is XOR-swizzled in 16-byte units so that both the
//     row-wise score reads and the transposed value reads are free of bank
//     conflicts.
//   * fp8 cache (e4m3 codes, bf16 rope lanes, one fp32 scale per token), two
//     modes: by default each chunk is dequantised into bf16 stages laid out as
//     above, and the rest is the bf16 code; with MLA_DECODE_FP8_MATH the scores
//     run on the fp8 matrix cores from the codes as stored, against queries
//     rounded to e4m3 with a power-of-two scale per 32 lanes, and the weighted
//     sum is split by columns across the wavefronts (codes widened to bf16 in
//     registers once per workgroup, weights exchanged through LDS).
#include <type_traits>

#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kChunk = 32;                           // tokens per pipeline stage
constexpr int kChunkContent = kChunk * 2 * kDc;      // 32 tokens x 512 bf16
constexpr int kChunkBytes = kChunkContent + kChunk * 2 * kDr;
constexpr int kStages = 4;                           // LDS ring of chunks (bf16 cache)
// fp8 cache: rows of 512 e4m3 codes and 64 bf16 rope lanes, plus one fp32
// scale per token. Chunks land in one of two staging buffers and are then
// dequantised into a ring of three bf16 stages laid out exactly like the bf16
// cache's, so scores, softmax and weighted sum are shared.
constexpr int kF8Row = kDc + 2 * kDr;                // 640 bytes per cached token
constexpr int kF8Codes = kChunk * kDc;               // 16 KB of codes per chunk
constexpr int kF8Rope = kChunk * 2 * kDr;            // 4 KB of rope lanes per chunk
constexpr int kF8Stage = kF8Codes + kF8Rope + kChunk * 4;
constexpr int kF8Stages = 3;
constexpr int kF8CopiesPerChunk = 6;
// fp8 cache on the fp8 matrix cores: chunks land in a ring of four stages
// that hold the codes as stored (32 rows of 512 bytes, XOR-swizzled in
// 16-byte units), the 32 bf16 rope rows and the 32 token scales. Nothing is
// dequantised in LDS: the scores multiply the codes as they are, and the
// weighted sum converts them to bf16 in registers.
constexpr int kF8MRope = kChunk * kDc;                    // rope rows at 16 KB
constexpr int kF8MScales = kF8MRope + kChunk * 2 * kDr;   // token scales at 20 KB
constexpr int kF8MStage = 20992;   // 20608 bytes used; a multiple of 512 (fragment XORs)
constexpr int kF8MStages = 4;
constexpr int kF8MCopies = 6;      // copy instructions per wave and chunk
constexpr int kRowBytes = 2 * (kDc + kDr);           // one cached token, bf16
constexpr float kRescaleLog2 = 8.0f;                 // lazy-rescale threshold (2^8)

struct MfmaParams {   // the scalar arguments of the kernel
  int part_bf16;  // partials stored as bf16, else fp32
  float c_log2;   // |softmax scale| * log2(e), at least FLT_MIN
  int neg_q;      // the scale is negative: the kernel negates the queries (exact)
  int B, q_len, n_h, max_blocks, rows, row_groups;
  int64_t G;
};

// XOR swizzle of the 16-byte chunk index within a content row: a map of the
// token's low 4 bits chosen so that 8 or 16 consecutive tokens at one chunk
// (score reads), and 4 consecutive tokens x 4 consecutive chunks
// (transposed value reads), fall in distinct bank groups (32- and 64-bank
// models).
__device__ __forceinline__ int swz(int t) {
  const int v = t & 3, u = (t >> 2) & 3;
  return ((v >> 1) << 3) | ((v & 1) << 2) | (((v >> 1) ^ (u >> 1)) << 1) | (u & 1);
}

// Score MFMA S += A B with S in vector registers (see the file comment).
// The first of a chain starts from zero; the last one of a chain is followed
// by 16 wait states so that vector ALU reads of S see the final value.
__device__ __forceinline__ void mfma_s_first(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7"
               : "+v"(s) : "v"(a), "v"(b));
}
// the same for the 8 chunks of a rope row (128-byte rows)
__device__ __forceinline__ int swz_rope(int t) { return (t & 7) ^ ((t >> 3) & 1); }

// 16-byte unit swizzle of an fp8 code row (512 bytes), a function of the
// token's low 4 bits: bijective over 16 consecutive tokens (score reads, one
// unit per lane), and over each 8-token set of a transposed value read
// ({0-3, 8-11} or {4-7, 12-15} plus two adjacent units), for the 32-bank and
// the 64-bank model alike (checked by enumeration).
__device__ __forceinline__ int swz8(int t) {
  return (((t & 3) << 1) | ((t >> 2) & 1)) ^ (((t >> 3) & 1) * 9);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Score MFMA on the fp8 matrix cores, S += A B with S in vector registers:
// A = 32 tokens x 64 lanes of e4m3 codes (scale 1: `one` holds the E8M0 byte
// 127), B = 64 lanes x 32 query rows of e4m3 queries whose two 32-lane
// blocks carry E8M0 scales in byte `sel` of `qs` (lane i gives the first
// block's scale of row i, lane 32 + i the second's). Each lane's bytes 0..15
// belong to the first block and 16..31 to the second.
__device__ __forceinline__ void mfma8_s(bool first, int sel, f32x16& s, const i32x8& a,
                                        const i32x8& b, int one, int qs) {
#define MLA_F8(SEL)                                                                        \
  if (first)                                                                               \
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 " SEL             \
                 : "=&v"(s) : "v"(a), "v"(b), "v"(one), "v"(qs));                           \
  else                                                                                     \
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 " SEL            \
                 : "+v"(s) : "v"(a), "v"(b), "v"(one), "v"(qs));
  switch (sel) {
    case 0: MLA_F8("op_sel_hi:[0,0,0]") break;
    case 1: MLA_F8("op_sel:[0,1,0] op_sel_hi:[0,0,0]") break;
    case 2: MLA_F8("op_sel_hi:[0,1,0]") break;
    default: MLA_F8("op_sel:[0,1,0] op_sel_hi:[0,1,0]") break;
  }
#undef MLA_F8
}

// One 16-byte-per-lane global -> LDS copy: lane i's 16 bytes from
// sbase + voff land at LDS address lds + 16 i. Issued as a single instruction
// so that it is not counted as an LDS access by the compiler's wait-count
// logic (which would otherwise drain every LDS read while a copy is in
// flight); its completion is waited for explicitly (vmcnt) before the
// barrier that publishes the page.
__device__ __forceinline__ void lds_dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// The same copy with a full 64-bit source address per lane.
__device__ __forceinline__ void lds_dma16_va(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ s16x4 lds_tr16a(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(static_cast<uintptr_t>(a)));
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Per-lane source offsets of a chunk copy, precomputed once:
//   content rows t = 16 j + 4 w + i (j in 0..1, i in 0..3) need logical
//   16-byte unit lane ^ swz(t) of the row, and swz depends on t only through
//   4 w + i, so four patterns serve all 8 rows of the wave;
//   rope rows are one per 8 lanes: row 8 w + lane / 8 of the chunk.
struct CopyPlan {
  uint32_t content[4];   // lane byte offset within a content row, per i
  uint32_t rope;         // lane byte offset within the chunk source, all rows valid
};

__device__ __forceinline__ uint32_t rope_src(int w, int lane, int n_valid) {
  const int t = 8 * w + (lane >> 3);
  const int ts = t < n_valid ? t : 0;
  return ts * kRowBytes + 2 * kDc + (((lane & 7) ^ swz_rope(t)) << 4);
}

// Copy instruction i (0..8) of the 32-token chunk whose first cached row is
// at `src` (tokens [0, n_valid) valid) into the LDS stage at `buf`:
// instructions 0..7 copy content rows 16 (i / 4) + 4 w + i % 4, instruction 8
// the wave's 8 rope rows. Rows past n_valid are read from row 0 so that every
// LDS value is finite. `w` and `n_valid` are wave-uniform: all row
// arithmetic is scalar.
constexpr int kCopiesPerChunk = 9;
__device__ __forceinline__ void copy_part(int i, const uint8_t* src, int n_valid, uint32_t buf,
                                          int w, int lane, const CopyPlan& cp) {
  if (i < 8) {
    const int t = 16 * (i >> 2) + 4 * w + (i & 3);
    const int ts = t < n_valid ? t : 0;
    lds_dma16(src + ts * kRowBytes, cp.content[i & 3], buf + t * 1024);
  } else {
    lds_dma16(src, n_valid == kChunk ? cp.rope : rope_src(w, lane, n_valid),
              buf + kChunkContent + w * 1024);
  }
}

// Copy instruction i (0..5) of an fp8 chunk: the 32 code rows (two tokens per
// instruction, instructions 0..3), the wave's 8 rope rows (4) and the wave's 8
// scales (5, two lanes). `src` is the chunk's first cached row, `ssrc` its
// first scale; rows past n_valid are read from row 0.
__device__ __forceinline__ void copy_part_f8(int i, const uint8_t* src, const uint8_t* ssrc,
                                             int n_valid, uint32_t stg, int w, int lane) {
  if (i < 4) {
    const int j = 4 * w + i;                  // token pair
    const int t = 2 * j + (lane >> 5);
    const int ts = t < n_valid ? t : 0;
    lds_dma16(src, ts * kF8Row + (lane & 31) * 16, stg + j * 1024);
  } else if (i == 4) {
    const int t = 8 * w + (lane >> 3);
    const int ts = t < n_valid ? t : 0;
    lds_dma16(src, ts * kF8Row + kDc + (lane & 7) * 16, stg + kF8Codes + w * 1024);
  } else if (lane < 2) {
    lds_dma16(ssrc, (8 * w + 4 * lane) * 4, stg + kF8Codes + kF8Rope + w * 32);
  }
}

// Copy instruction i (0..5) of an fp8 chunk into its matrix-core stage at
// `stg`: instructions 0..3 copy the code rows of tokens 8 w + 2 i and
// 8 w + 2 i + 1 (each 16-byte unit to its swizzled place), 4 the wave's 8
// rope rows, 5 the wave's 8 scales (two lanes). `src` is the chunk's first
// cached row, `ssrc` its first scale; rows past n_valid are read from row 0
// (their scales are never used).
__device__ __forceinline__ void copy_part_f8m(int i, const uint8_t* src, const uint8_t* ssrc,
                                              int n_valid, uint32_t stg, int w, int lane) {
  if (i < 4) {
    const int t = 8 * w + 2 * i + (lane >> 5);
    const int ts = t < n_valid ? t : 0;
    lds_dma16(src, ts * kF8Row + (((lane & 31) ^ swz8(t)) << 4), stg + (4 * w + i) * 1024);
  } else if (i == 4) {
    const int t = 8 * w + (lane >> 3);
    const int ts = t < n_valid ? t : 0;
    lds_dma16(src, ts * kF8Row + kDc + (((lane & 7) ^ swz_rope(t)) << 4), stg + kF8MRope + w * 1024);
  } else if (lane < 2) {
    lds_dma16(ssrc, (8 * w + 4 * lane) * 4, stg + kF8MScales + w * 32);
  }
}

// Per-lane source offsets of a full fp8 chunk's copies into a matrix-core
// stage (copy_part_f8m with every row valid), precomputed once.
struct F8MCopyPlan {
  uint32_t code[4];   // instruction i, from the row of token 8 w + 2 i
  uint32_t rope;      // the rope copy, from the row of token 8 w
};

__device__ __forceinline__ F8MCopyPlan f8m_copy_plan(int w, int lane) {
  F8MCopyPlan c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 8 * w + 2 * i + (lane >> 5);
    c.code[i] = (lane >> 5) * kF8Row + (((lane & 31) ^ swz8(t)) << 4);
  }
  const int t = 8 * w + (lane >> 3);
  c.rope = (lane >> 3) * kF8Row + kDc + (((lane & 7) ^ swz_rope(t)) << 4);
  return c;
}

// s_waitcnt with vmcnt(n), expcnt and lgkmcnt left free (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define MLA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// The lane index, formed afresh where it is used: the empty asm statement
// keeps the compiler from reusing (and so keeping alive or spilling) an
// earlier copy. A value reloaded from scratch memory would cost a wait on
// every vector memory operation in flight, including the cache copies.
__device__ __forceinline__ uint32_t lane_now() {
  uint32_t l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}


// Pointer arguments are separate restrict-qualified parameters, so that the
// compiler reads the read-only tables with scalar loads.
//
// kLdsPlan: every workgroup forms the page prefix sums itself in LDS (batch
// up to kMaxLdsBatch, or kF8MMaxLdsBatch for the fp8 matrix-core mode, whose
// query staging leaves less LDS), and workgroup 0 also stores them for the
// combine; otherwise they come from the plan kernel through page_start.
//
// kMode: 0 = bf16 cache; 1 = fp8 cache dequantised to bf16 in LDS (bf16
// matrix cores throughout); 2 = fp8 cache on the fp8 matrix cores (scores
// from the codes as stored against e4m3-rounded queries; weighted sum in bf16).
constexpr int kMaxLdsBatch = 1024;
constexpr int kF8MMaxLdsBatch = 256;
template <bool kLdsPlan, int kMode>
__global__ __launch_bounds__(256, 1) void decode_mfma_bf16(
    const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
    const uint8_t* __restrict__ cache, const float* __restrict__ cache_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ page_start, void* __restrict__ o_part, float* __restrict__ lse_part,
    float* __restrict__ l_part, void* __restrict__ o_out, float* __restrict__ lse_out,
    MfmaParams p) {
  constexpr bool kFp8 = kMode == 1;   // fp8 cache, dequantised in LDS
  constexpr bool kF8M = kMode == 2;   // fp8 cache on the fp8 matrix cores
  // ring of chunk stages: chunk k lives in stage k % kS (fp8 dequantised: plus
  // two staging buffers after the ring; fp8 matrix cores: plus a query
  // staging region of 18 KB per wave)
  constexpr int kS = kF8M ? kF8MStages : (kFp8 ? kF8Stages : kStages);
  constexpr int kStageBytes = kF8M ? kF8MStage : kChunkBytes;
  constexpr int kSmem = kF8M ? kS * kF8MStage + 4 * (32 * 36 * 16)
                             : kS * kChunkBytes + (kFp8 ? 2 * kF8Stage : 0);
  constexpr int kMaxB = kF8M ? kF8MMaxLdsBatch : kMaxLdsBatch;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  __shared__ int restart_flag[4];   // per wave: some row raised its reference in this pass
  __shared__ int ps_lds[kLdsPlan ? kMaxB + 1 : 1];   // page prefix sums
  __shared__ int lens_lds[kLdsPlan ? kMaxB : 1];     // clamped sequence lengths
  __shared__ int wtot_lds[4];                               // per-wave page totals
  __shared__ float inv_lds[kMfmaRows];                      // 1 / row sum, whole-sequence pieces

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int half = lane >> 5, l32 = lane & 31;   // k-group and column of the 32x32 layouts
  CopyPlan cp;
#pragma unroll
  for (int i = 0; i < 4; ++i) cp.content[i] = (lane ^ swz(4 * w + i)) << 4;
  cp.rope = rope_src(w, lane, kChunk);

  // block id -> (range, row group): ids congruent mod 8 run on one XCD; XCD x
  // gets ranges [x G8, (x + 1) G8) with all their row groups
  const int64_t id = blockIdx.x;
  const int64_t G8 = (p.G + 7) / 8;
  const int64_t jx = id >> 3;
  const int64_t g = (id & 7) * G8 + jx / p.row_groups;
  const int rg = static_cast<int>(jx % p.row_groups);
  if (g >= p.G) return;
  // rows of this group that exist (the last group of a row count that is
  // not a multiple of 128 is padded: its missing rows load the group's first
  // query row, are computed like the others, and are never stored)
  const int rv = min(kMfmaRows, p.rows - rg * kMfmaRows);
  if constexpr (kLdsPlan) {
    // page_start[b] = sum_{b' < b} ceil(S_b' / 64): four sequences per thread,
    // a scan across the wavefront, then the totals of the waves before
    const int t = threadIdx.x;
    int cnt[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = 4 * t + i;
      const int len = bb < p.B ? clamp_len(seq_lens[bb], p.max_blocks) : 0;
      if (bb < p.B) lens_lds[bb] = len;
      cnt[i] = static_cast<int>(pages_of(len));
      local += cnt[i];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wtot_lds[w] = incl;
    __syncthreads();
    int run = incl - local;
    for (int ww = 0; ww < w; ++ww) run += wtot_lds[ww];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = 4 * t + i;
      if (bb <= p.B) ps_lds[bb] = run;
      run += cnt[i];
    }
    // with B = 4 * 256 no thread's sequences reach index B: the last thread
    // stores the total
    if constexpr (kMaxB == 4 * 256) {
      if (t == 255 && p.B == kMaxB) ps_lds[p.B] = run;
    }
    __syncthreads();
    if (blockIdx.x == 0)
      for (int bb = t; bb <= p.B; bb += 256) page_start[bb] = ps_lds[bb];
  }
  auto PS = [&](int i) -> int64_t {
    if constexpr (kLdsPlan) return ps_lds[i];
    else return page_start[i];
  };
  const int64_t P = PS(p.B);
  const int64_t pb = range_begin_dev(g, P, p.G), pe = range_begin_dev(g + 1, P, p.G);
  if (pb >= pe) return;

  // first sequence of the range: the number of sequences that end at or
  // before page pb (the prefix sums are non-decreasing), 64 per ballot
  int b = 0;
  for (int j0 = 0; j0 < p.B; j0 += 64) {
    const int j = j0 + lane;
    const uint64_t before = __ballot(j < p.B && PS(j + 1) <= pb);
    b += __popcll(before);
    if (before != ~0ull) break;
  }

  const float c = p.c_log2;
  const bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // LDS byte offsets of this lane's fragments within a stage. The swizzle
  // only changes offset bits that the unrolled loop constants reach through
  // an XOR, so one base register per pattern suffices: offset = (base ^ k) + imm.
  const int hx = swz(l32);
  // score A-fragment, token l32, content unit 2 kc + half:
  //   bits 5..7 = (kc & 7) ^ (hx >> 1), + 256 * (kc >> 3)
  const uint32_t qk_base = l32 * 1024 + ((half ^ (hx & 1)) << 4) + ((hx >> 1) << 5);
  // rope unit 2 kk + half of a 128-byte rope row: bits 5..6 = kk ^ (hr >> 1)
  const int hr = swz_rope(l32);
  const uint32_t rope_base = kChunkContent + l32 * 128 + ((half ^ (hr & 1)) << 4) + ((hr >> 1) << 5);
  // transposed value reads: 16-lane group g16, source lane s16 reads
  // row 4 (g16 >> 1) + (s16 >> 2) (+8 for the second read) of a 16-token
  // step, columns 32 mb + 16 (g16 & 1) + 4 (s16 & 3):
  //   bits 6..7 = (mb & 3) ^ (swz >> 2), + 256 * (mb >> 2) + 16384 * step
  const int g16 = lane >> 4, s16 = lane & 15;
  uint32_t pv_base[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int t = 4 * (g16 >> 1) + (s16 >> 2) + 8 * sec;
    const int ht = swz(t);
    const int qlow = 2 * (g16 & 1) + ((s16 & 3) >> 1);
    pv_base[sec] = t * 1024 + ((qlow ^ (ht & 3)) << 4) + (s16 & 1) * 8 + ((ht >> 2) << 6);
  }
  // fp8 matrix-core mode: score A fragment e (0, 1) of k-block kb is the
  // 16-byte unit 4 kb + 2 e + half of token l32's code row, at
  // f8_qb[e] ^ (64 kb); rope fragments as above but at kF8MRope; transposed
  // value reads (ds_read_b64_tr_b8): in 16-lane group g16, source lane s16
  // reads row p = s16 / 2, bytes 8 (s16 % 2) of unit 2 mb + (g16 & 1), where
  // row p is token (p & 3) + 8 (p >> 2) + 4 (g16 >> 1) of a 16-token step;
  // destination lane j then holds column j of the 8 rows
  uint32_t f8_qb[2], f8_pv = 0;
  {
    const int s8 = swz8(l32);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      f8_qb[e] = l32 * kDc + 64 * (s8 >> 2) + 16 * ((2 * e + half) ^ (s8 & 3));
    const int pr = s16 >> 1;
    const int tau = (pr & 3) + 8 * (pr >> 2) + 4 * (g16 >> 1);
    const int st8 = swz8(tau);
    f8_pv = tau * kDc + 32 * (st8 >> 1) + 16 * ((g16 & 1) ^ (st8 & 1)) + 8 * (s16 & 1);
  }
  const uint32_t rope_base8 = kF8MRope + l32 * 128 + ((half ^ (hr & 1)) << 4) + ((hr >> 1) << 5);
  const uint32_t lds0 = lds_addr(smem);

  for (; b < p.B && PS(b) < pe; ++b) {
    const int64_t s0 = PS(b), s1 = PS(b + 1);
    if (s1 == s0) continue;
    const int64_t a0 = s0 > pb ? s0 : pb, a1 = s1 < pe ? s1 : pe;
    // a piece that holds every page of its sequence writes the final output
    // itself (normalised, in the output dtype, with its log-sum-exp) when the
    // caller passed it; the combine then skips that sequence
    const bool whole = o_out != nullptr && a0 == s0 && a1 == s1;
    const int n_pages = static_cast<int>(a1 - a0);
    int S;
    if constexpr (kLdsPlan) S = lens_lds[b];
    else S = clamp_len(seq_lens[b], p.max_blocks);
    // query token of this lane's row (row / heads), formed per piece from the
    // lane index
    const int m = (rg * kMfmaRows + w * 32 + static_cast<int>(lane_now() & 31)) / p.n_h;
    const int pidx0 = static_cast<int>(a0 - s0);
    const int tok0 = pidx0 * 64;
    const int tok1 = min(S, static_cast<int>((a1 - s0) * 64));
    const int n = (tok1 - tok0 + kChunk - 1) / kChunk;   // chunks of this piece (>= 1)
    const int tend = min(tok1, S - p.q_len + m + 1);      // this row's visible end
    // tokens below tend_all are visible to every row of the wave (its first
    // row has the smallest query index)
    const int tend_all = min(tok1, S - p.q_len + (rg * kMfmaRows + w * 32) / p.n_h + 1);
    const int32_t* bt = block_table + static_cast<int64_t>(b) * p.max_blocks;
    // Q^T fragments: fragment kc of lane (half, l32) holds the 16-byte unit
    // 2 kc + half of the wave's row l32, where units 0..63 are q_abs and
    // 64..71 q_rope. The wave's 32 rows are consecutive (rows b * rows +
    // rg * 128 + 32 w + l32). Loaded straight into that layout, every load
    // instruction would touch 32 rows; instead each half of the units (36 per
    // row) is copied HBM -> LDS with whole rows per instruction into a region
    // of the wave's own, then read in fragment layout. Within a half, row n's
    // unit v sits at 16-byte slot 36 n + (v ^ ((n >> 2) & 3)): the swizzle
    // keeps 16 consecutive rows of a fragment read in distinct bank groups.
    bf16x8 qf[36];
    constexpr int kQHalf = 32 * 36 * 16;      // one wave's half: 18 KB
    auto q_region = [&]() {
      if constexpr (kF8M) return lds0 + kS * kF8MStage + w * kQHalf;
      else return lds0 + (kS - 2) * kChunkBytes + w * kQHalf;
    };
    auto q_copy = [&](int H) {
      const int64_t qrow0 = static_cast<int64_t>(b) * p.rows + rg * kMfmaRows + w * 32;
      const uint8_t* qa = reinterpret_cast<const uint8_t*>(q_abs + qrow0 * kDc);
      const uint8_t* qr = reinterpret_cast<const uint8_t*>(q_rope + qrow0 * kDr);
      const uint32_t li = lane_now();
      const uint32_t reg = q_region();
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const uint32_t sl = 64 * i + li, n = sl / 36, x = sl % 36;
        uint32_t u = 36 * H + (x ^ ((n >> 2) & 3));
        if constexpr (kF8M) {   // see q_read8
          const uint32_t y = x ^ ((n >> 2) & 3);
          u = y < 32 ? 32 * H + y : 64 + 4 * H + (y - 32);
        }
        // a padded row reads the group's first row (32 w rows back)
        const int64_t nr = static_cast<int>(32 * w + n) < rv ? static_cast<int64_t>(n) : -32LL * w;
        const uint8_t* src = u < 64 ? qa + nr * (2 * kDc) + 16 * u : qr + nr * (2 * kDr) + 16 * (u - 64);
        lds_dma16_va(src, reg + 1024 * i);
      }
    };
    auto q_read = [&](int H) {
      const uint32_t li = lane_now();
      const uint32_t n = li & 31, hl = li >> 5, sw = (n >> 2) & 3;
      const uint32_t r0 = q_region() + 576 * n + 16 * (hl ^ sw);          // even fragments
      const uint32_t r1 = q_region() + 576 * n + 16 * ((2 + hl) ^ sw);    // odd fragments
#pragma unroll
      for (int kc = 0; kc < 18; ++kc)
        qf[18 * H + kc] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            static_cast<uintptr_t>(((kc & 1) ? r1 : r0) + 64 * (kc >> 1)));
    };
    // fp8 matrix-core mode: the queries as B fragments of the fp8 score
    // MFMA. Half H of a row is q_abs units [32 H, 32 H + 32) and rope units
    // 64 + [4 H, 4 H + 4) (units of 8 bf16): slot x of the half holds unit
    // 32 H + x below 32, 64 + 4 H + x - 32 above. Fragment kb of lane
    // (half, l32) holds lanes 64 kb + 16 half + (0..15) of row l32 in bytes
    // 0..15 (the k-block's first 32-lane block) and lanes 64 kb + 32 +
    // 16 half + (0..15) in bytes 16..31 (its second block), the same order as
    // the code fragments. Each block is scaled by a power of two that puts its
    // largest magnitude in [128, 256) and rounded to e4m3 (to nearest even);
    // byte kb % 4 of qs8[kb / 4] holds the E8M0 scale of the lane's block
    // (its half), which the MFMA applies.
    i32x8 qf8[8];
    int qs8[2] = {0, 0};
    bf16x8 qr8[4];
    auto q_read8 = [&](int H) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const uint32_t li = lane_now();
      const uint32_t nn = li & 31, hl = li >> 5, sw = (nn >> 2) & 3;
      const uint32_t reg = q_region() + 576 * nn;
      const uint32_t neg = p.neg_q ? 0x80808080u : 0u;
      auto rd = [&](uint32_t y) {
        return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            static_cast<uintptr_t>(reg + 16 * (y ^ sw)));
      };
#pragma unroll
      for (int kbl = 0; kbl < 4; ++kbl) {
        const u32x4 v0 = rd(8 * kbl + 2 * hl), v1 = rd(8 * kbl + 2 * hl + 1);
        const u32x4 v2 = rd(8 * kbl + 4 + 2 * hl), v3 = rd(8 * kbl + 5 + 2 * hl);
        const uint32_t wv[16] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3],
                                 v2[0], v2[1], v2[2], v2[3], v3[0], v3[1], v3[2], v3[3]};
        // block maxima of |q| on the bf16 patterns (sign cleared, the integer
        // order is the magnitude order), then across the wave halves
        uint32_t a0 = 0, a1 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a0 = max(a0, max(wv[i] & 0x7FFFu, (wv[i] >> 16) & 0x7FFFu));
          a1 = max(a1, max(wv[8 + i] & 0x7FFFu, (wv[8 + i] >> 16) & 0x7FFFu));
        }
        const uint32_t pk = a0 | (a1 << 16);
        const auto xs = __builtin_amdgcn_permlane32_swap(pk, pk, false, false);
        const uint32_t b0 = max(xs[0] & 0xFFFFu, xs[1] & 0xFFFFu);
        const uint32_t b1 = max(xs[0] >> 16, xs[1] >> 16);
        // E8M0 byte e = E - 7 for a block maximum with biased exponent E (at
        // least 1): the block divided by 2^(e - 127) has its maximum in
        // [128, 256), below the e4m3 maximum 448
        const int e0 = max(static_cast<int>(b0 >> 7) - 7, 1);
        const int e1 = max(static_cast<int>(b1 >> 7) - 7, 1);
        const float m0 = __uint_as_float(static_cast<uint32_t>(254 - e0) << 23);
        const float m1 = __uint_as_float(static_cast<uint32_t>(254 - e1) << 23);
        i32x8 f;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const float mult = d < 4 ? m0 : m1;
          const uint32_t lo = wv[2 * d], hi = wv[2 * d + 1];
          int r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(lo << 16) * mult,
                                                  __uint_as_float(lo & 0xFFFF0000u) * mult, 0, false);
          r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(hi << 16) * mult,
                                              __uint_as_float(hi & 0xFFFF0000u) * mult, r, true);
          f[d] = static_cast<int>(static_cast<uint32_t>(r) ^ neg);
        }
        qf8[4 * H + kbl] = f;
        qs8[H] |= (hl ? e1 : e0) << (8 * kbl);
      }
#pragma unroll
      for (int kkl = 0; kkl < 2; ++kkl) {
        const u32x4 r4 = rd(32 + 2 * kkl + hl) ^ (p.neg_q ? 0x80008000u : 0u);
        qr8[2 * H + kkl] = __builtin_bit_cast(bf16x8, r4);
      }
    };
    auto negate_q = [&]() {   // c s with c < 0 equals |c| (-s), and negating bf16 is exact
#pragma unroll
      for (int i = 0; i < 36; ++i) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        qf[i] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[i]) ^ 0x80008000u);
      }
    };

    f32x16 o[16];
    float m_run = -INFINITY, l_lane = 0.f;


    // zero O through the matrix unit: every definition of O is then an MFMA
    // result, and the compiler keeps O in the accumulation registers across
    // the chunk loop (a vector-ALU zero would make it carry O in the vector
    // registers and copy it in and out on every chunk)
    auto zero_o = [&]() {
      const bf16x8 z8 = {};
#pragma unroll
      for (int mb = 0; mb < 16; ++mb)
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z8, z8, f32x16{}, 0, 0, 0);
      l_lane = 0.f;
    };
    // first cached row of chunk q of the piece (the page id is a scalar load)
    constexpr int kRow = (kFp8 || kF8M) ? kF8Row : kRowBytes;   // bytes per cached row in HBM
    auto chunk_page = [&](int q) -> int { return bt[pidx0 + (q >> 1)]; };
    auto chunk_src = [&](int q) {
      return cache + chunk_page(q) * (64LL * kRow) + (q & 1) * (kChunk * kRow);
    };
    auto chunk_valid = [&](int q) { return min(kChunk, tok1 - tok0 - kChunk * q); };
    auto stage_of = [&](int q) { return lds0 + (static_cast<uint32_t>(q) % kS) * kStageBytes; };
    const uint32_t stg0 = lds0 + kS * kChunkBytes;   // fp8 staging buffers
    // copy all of chunk q at once (into its stage, or for fp8 its staging buffer)
    // (the per-lane offsets are formed afresh: see lane_now)
    auto issue = [&](int q) {
      const uint8_t* src = chunk_src(q);
      const int nv = chunk_valid(q);
      const int li = static_cast<int>(lane_now());
      if constexpr (kF8M) {
        const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(
            cache_scale + static_cast<int64_t>(chunk_page(q)) * 64 + (q & 1) * kChunk);
#pragma unroll
        for (int i = 0; i < kF8MCopies; ++i) copy_part_f8m(i, src, ssrc, nv, stage_of(q), w, li);
      } else if constexpr (kFp8) {
        const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(
            cache_scale + static_cast<int64_t>(chunk_page(q)) * 64 + (q & 1) * kChunk);
#pragma unroll
        for (int i = 0; i < kF8CopiesPerChunk; ++i)
          copy_part_f8(i, src, ssrc, nv, stg0 + (q & 1) * kF8Stage, w, li);
      } else {
        CopyPlan cpi;
#pragma unroll
        for (int i = 0; i < 4; ++i) cpi.content[i] = (li ^ swz(4 * w + i)) << 4;
        cpi.rope = rope_src(w, li, kChunk);
#pragma unroll
        for (int i = 0; i < kCopiesPerChunk; ++i)
          copy_part(i, src, nv, stage_of(q), w, li, cpi);
      }
    };
    // fp8: dequantise chunk q from its staging buffer into its bf16 stage:
    // thread (token t, group g) turns codes [64 g, 64 g + 64) of row t into
    // bf16 (e4m3 decoded exactly, times the token's scale, rounded to bf16)
    // and copies 16 bytes of the rope row; rows past the valid tokens get
    // scale 0. Every wave must have waited for the copies (and passed a
    // barrier) before, and a barrier must follow before the stage is read.
    auto dequant = [&](int q) {
      const int tid = w * 64 + static_cast<int>(lane_now());
      const int t = tid >> 3, gq = tid & 7;
      const uint32_t sb = stg0 + (q & 1) * kF8Stage;
      const uint32_t db = stage_of(q);
      const float sc = t < chunk_valid(q)
                           ? *reinterpret_cast<const __attribute__((address_space(3))) float*>(
                                 static_cast<uintptr_t>(sb + kF8Codes + kF8Rope + 4 * t))
                           : 0.f;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const int hs = swz(t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 c4 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            static_cast<uintptr_t>(sb + t * kDc + gq * 64 + i * 16));
#pragma unroll
        for (int h = 0; h < 2; ++h) {      // 8 codes -> one 16-byte bf16 unit
          u32x4 o4;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t wd = c4[2 * h + e];
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wd), false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wd), true);
            const bf16x2 b0 = {static_cast<__bf16>(lo[0] * sc), static_cast<__bf16>(lo[1] * sc)};
            const bf16x2 b1 = {static_cast<__bf16>(hi[0] * sc), static_cast<__bf16>(hi[1] * sc)};
            o4[2 * e] = __builtin_bit_cast(uint32_t, b0);
            o4[2 * e + 1] = __builtin_bit_cast(uint32_t, b1);
          }
          const int unit = 8 * gq + 2 * i + h;
          *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
              static_cast<uintptr_t>(db + t * 1024 + ((unit ^ hs) << 4))) = o4;
        }
      }
      const u32x4 r4 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          static_cast<uintptr_t>(sb + kF8Codes + t * 128 + gq * 16));
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(static_cast<uintptr_t>(
          db + kChunkContent + t * 128 + ((gq ^ swz_rope(t)) << 4))) = r4;
    };
    // The same dequantisation in pieces, for the pipeline step: dq_load
    // issues the LDS reads of the thread's first 16 codes and its scale and
    // copies the rope unit; dq_part(j), j = 0..15, converts 4 codes and stores
    // a 16-byte unit after every second part. Work split (free of LDS bank
    // conflicts for reads and writes): the 16 lanes of group g = tid / 16 take
    // tokens T = (g % 4) + 8 (g / 4) and T + 4 (lanes 8..15), and in
    // iteration i the 16-code units u = 8 ((i + sub) % 4) + lane % 8, sub =
    // lane / 8 % 2: the two tokens' reads fall in opposite halves of the
    // banks, and their stage swizzles differ in the lowest bit.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t dq_c[2], dq_o;   // codes of the current and the next 16-code group
    float dq_s = 0.f;
    auto dq_token = [](int tid) { return (((tid >> 4) & 3) + 8 * (tid >> 6)) + 4 * ((tid >> 3) & 1); };
    auto dq_unit = [](int tid, int i) { return 8 * ((i + ((tid >> 3) & 1)) & 3) + (tid & 7); };
    auto dq_codes = [&](int q, int i, int tid) {
      dq_c[i & 1] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
          static_cast<uintptr_t>(stg0 + (q & 1) * kF8Stage + dq_token(tid) * kDc + dq_unit(tid, i) * 16));
    };
    auto dq_load = [&](int q, int tid) {
      const int t = tid >> 3, gq = tid & 7;
      const uint32_t sb = stg0 + (q & 1) * kF8Stage;
      dq_codes(q, 0, tid);
      const int tt = dq_token(tid);
      dq_s = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
          static_cast<uintptr_t>(sb + kF8Codes + kF8Rope + 4 * tt));
      if (tt >= chunk_valid(q)) dq_s = 0.f;
      const u32x4_t r4 = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
          static_cast<uintptr_t>(sb + kF8Codes + t * 128 + gq * 16));
      *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(static_cast<uintptr_t>(
          stage_of(q) + kChunkContent + t * 128 + ((gq ^ swz_rope(t)) << 4))) = r4;
    };
    auto dq_part = [&](int q, int j, int tid) {
      const int t = dq_token(tid);
      const int i = j >> 2, h = (j >> 1) & 1, e = j & 1;
      if ((j & 3) == 0 && i < 3) dq_codes(q, i + 1, tid);   // one group ahead
      const uint32_t wd = dq_c[i & 1][2 * h + e];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wd), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wd), true);
      const bf16x2 b0 = {static_cast<__bf16>(lo[0] * dq_s), static_cast<__bf16>(lo[1] * dq_s)};
      const bf16x2 b1 = {static_cast<__bf16>(hi[0] * dq_s), static_cast<__bf16>(hi[1] * dq_s)};
      dq_o[2 * e] = __builtin_bit_cast(uint32_t, b0);
      dq_o[2 * e + 1] = __builtin_bit_cast(uint32_t, b1);
      asm volatile("" : "+v"(dq_o));
      if (e == 1) {
        const int unit = 2 * dq_unit(tid, i) + h;
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(static_cast<uintptr_t>(
            stage_of(q) + t * 1024 + ((unit ^ swz(t)) << 4))) = dq_o;
      }
    };
    // first two chunks in flight; wait for chunk 0 everywhere (fp8: and
    // dequantise it)
    auto start = [&]() {
      issue(0);
      if (n > 1) issue(1);
      if constexpr (kFp8) {
        if (n > 1) MLA_WAIT_VM(kF8CopiesPerChunk);
        else MLA_WAIT_VM(0);
        __syncthreads();
        dequant(0);
      } else {
        constexpr int kC = kF8M ? kF8MCopies : kCopiesPerChunk;
        if (n > 1) MLA_WAIT_VM(kC);
        else MLA_WAIT_VM(0);
      }
    };

    float m_prev = 0.f;      // reference of the previous chunk's probabilities
    f32x16 sp;               // raw (masked) scores of the previous chunk
    f32x16 scl_prev;         // (fp8 matrix cores) its token scales, zero past its valid rows
    auto clear_prev = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sp[r] = -INFINITY;
        scl_prev[r] = 0.f;
      }
      m_prev = 0.f;
    };
    bool raise = false;      // some row of this lane crossed the lazy threshold in this pass

    // One pipeline step k:
    //   phase 1: scores of chunk k on the matrix unit, interleaved with the
    //            exponentials of chunk k - 1 (p = 2^(c s - m)), their bf16
    //            packing and their row sums, and with the copy of chunk k + 2
    //            (one copy instruction every fourth MFMA);
    //   mask:    only for a chunk that reaches past a row's visible end;
    //   phase 2: weighted sum of chunk k - 1 on the matrix unit, interleaved
    //            with the row max of chunk k and the lazy reference update.
    // Every step runs the same code, so that one copy of the weighted sum
    // keeps O in the accumulation registers: step 0 weighs chunk 0 with the
    // zero probabilities of the empty chunk -1, and step n multiplies a stage
    // whose scores the mask removes entirely.
    // pg: page id of chunk k + 2, which the step copies. Its scalar load is
    // issued in the previous step's last weighted-sum MFMAs (whose LDS waits
    // are full waits anyway) and used at the top of the step, before any LDS
    // read: a scalar load still in flight elsewhere would make the compiler
    // wait for every LDS read in flight at its next LDS wait.
    int pg_next = 0;   // page id of the chunk the next step copies (chunk k + 3)
    auto step = [&](int k, int pg) {
      const uint32_t bq = stage_of(k);
      const uint32_t bv = k == 0 ? bq : stage_of(k + kS - 1);
      // stage (k + 2) % 4 last held chunk k - 2, whose weighted sum every
      // wave finished before the barrier that opened this step (the fp8 path
      // copies outside the step)
      const bool copy = k + 2 < n;
      const int cnv = copy ? chunk_valid(k + 2) : kChunk;
      // the copy sources of chunk k + 2, formed here at the top of the step,
      // where no LDS read is in flight
      const int64_t pgc = pg;
      const uint8_t* csrc = cache + pgc * (64LL * kRow) + ((k + 2) & 1) * (kChunk * kRow);
      const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(
          cache_scale + pgc * 64 + ((k + 2) & 1) * kChunk);
      asm volatile("" : "+s"(csrc));
      if constexpr (kFp8) asm volatile("" : "+s"(ssrc));
      const uint32_t cbuf = stage_of(k + 2);
      // full chunks are copied in nine pieces spread over the score MFMAs
      // (rows 4 w + j and 16 + 4 w + j, then the rope rows); a partial last
      // chunk is copied at once
      const bool cfast = copy && cnv == kChunk;
      const uint8_t* csw = csrc + 4 * w * kRowBytes;
      const uint32_t cbw = cbuf + 4 * w * 1024;
      auto copy_fast = [&](int i) {
        if (i < 8) {
          const int t = 16 * (i >> 2) + (i & 3);
          lds_dma16(csw + t * kRowBytes, cp.content[i & 3], cbw + t * 1024);
        } else {
          lds_dma16(csrc, cp.rope, cbuf + kChunkContent + w * 1024);
        }
      };
      if constexpr (!kFp8) {
        if (copy && !cfast) issue(k + 2);
      }
      // fp8: whether chunk k + 1 is to be dequantised in this step
      const bool dq = kFp8 && k + 1 < n;
      // the fragment bases pass through an empty asm statement, so that the
      // per-fragment XOR variants are formed here, step by step, instead of
      // being hoisted out of the loop (where they would pin 20 registers)
      uint32_t qb = qk_base, rb = rope_base, vb0 = pv_base[0], vb1 = pv_base[1];
      asm volatile("" : "+v"(qb), "+v"(rb), "+v"(vb0), "+v"(vb1));
      // (fp8) the thread id, re-derived per step for the same reason
      int tid_s = static_cast<int>(threadIdx.x);
      if constexpr (kFp8) asm volatile("" : "+v"(tid_s));
      const uint32_t qk_pg = bq + qb, rope_pg = bq + rb;
      auto kfrag = [&](int kc) {
        const uint32_t a = kc < 32 ? (qk_pg ^ ((kc & 7) << 5)) + (kc >> 3) * 256
                                   : rope_pg ^ ((kc - 32) << 5);
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            static_cast<uintptr_t>(a));
      };
      const uint32_t pv0 = bv + vb0, pv1 = bv + vb1;
      auto vfrag = [&](int st) {
        const int mb = st & 15, cc = st >> 4;   // all column blocks of one 16-token step, then the next
        const uint32_t off = (mb >> 2) * 256 + cc * 16384;
        const s16x4 lo = lds_tr16a((pv0 ^ ((mb & 3) << 6)) + off);
        const s16x4 hi = lds_tr16a((pv1 ^ ((mb & 3) << 6)) + off);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kD = kFp8 ? 3 : 4;   // score A-fragment read distance (MFMAs)
      constexpr int kV = kFp8 ? 3 : 4;   // value fragment read distance (MFMAs)
      bf16x8 kf[kD + 1];
      bf16x8 vf[kV + 1];
      bf16x8 pf[2];

      // exponentials of chunk k - 1: slot 2r computes p_r, the odd slots
      // pack pairs to bf16 and add them to the row sum (the sum is taken
      // over the bf16 weights the weighted sum uses). The empty asm
      // statements pin each result to its slot: without them the optimizer
      // sinks the whole softmax next to the weighted sum that consumes it,
      // and the matrix unit idles while it runs.
      auto smb_slot = [&](int s) {
        const int r = s >> 1;
        if (s < 32) {
          if ((s & 1) == 0) {
            sp[r] = __builtin_amdgcn_exp2f(fmaf(sp[r], c, -m_prev));
            asm volatile("" : "+v"(sp[r]));
          } else if (r & 1) {
            const bf16x2 two = {static_cast<__bf16>(sp[r - 1]), static_cast<__bf16>(sp[r])};
            pf[r >> 3][(r - 1) & 7] = two[0];
            pf[r >> 3][r & 7] = two[1];
            l_lane = __builtin_amdgcn_fdot2_f32_bf16(two, kOnes2, l_lane, false);
            asm volatile("" : "+v"(l_lane));
          }
        }
      };

      // ---- phase 1: S^T = K Q^T of chunk k ----
      f32x16 sn;
#pragma unroll
      for (int j = 0; j < kD; ++j) kf[j] = kfrag(j);
#pragma unroll
      for (int kc = 0; kc < 36; ++kc) {
        if (kc + kD < 36) kf[(kc + kD) % (kD + 1)] = kfrag(kc + kD);
        if (kc == 0) mfma_s_first(sn, kf[0], qf[0]);
        else if (kc == 35) mfma_s_last(sn, kf[kc % (kD + 1)], qf[kc]);
        else mfma_s(sn, kf[kc % (kD + 1)], qf[kc]);
        smb_slot(kc);
        // the weighted sum's first value fragments (its stage has been
        // complete since the previous step), so that its first MFMA does not
        // wait for an LDS read
        if (kc == 31) {
#pragma unroll
          for (int j = 0; j < kV; ++j) vf[j] = vfrag(j);
        }
        if constexpr (kFp8) {
          if ((kc & 3) == 2 && kc < 24 && copy)
            copy_part_f8(kc >> 2, csrc, ssrc, cnv, stg0 + ((k + 2) & 1) * kF8Stage, w, tid_s & 63);
        } else {
          if ((kc & 3) == 2 && cfast) copy_fast(kc >> 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- mask tokens at or past the row's visible end (wave-uniform test) ----
      if (tok0 + kChunk * k + kChunk > tend_all) {
        const int lim = tend - (tok0 + kChunk * k) - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[r] = (r & 3) + 8 * (r >> 2) < lim ? sn[r] : -INFINITY;
      }

      // ---- phase 2: row max of chunk k, reference update ----
      float mx = -INFINITY;
      auto sma_slot = [&](int s) {
        if (s < 8) {
          // max3 without the NaN canonicalisation that fmaxf adds (scores are
          // finite or -inf)
          asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(sn[2 * s]), "v"(sn[2 * s + 1]));
          asm volatile("" : "+v"(mx));
        } else if (s == 8) {   // the row's other 16 tokens sit in the other wave half
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
          asm volatile("" : "+v"(mx));
        } else if (s == 9) {
          // rows that already hold weight and see a max above the lazy
          // threshold force a restart; the others just move their reference
          const bool up = mx > m_run + kRescaleLog2;
          raise = raise || (up && m_run != -INFINITY);
          m_run = up ? mx : m_run;
        }
      };
      // ---- ... interleaved with O^T += V^T P^T over chunk k - 1 ----
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        if (st + kV < 32) vf[(st + kV) % (kV + 1)] = vfrag(st + kV);
        o[st & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % (kV + 1)], pf[st >> 4],
                                                               o[st & 15], 0, 0, 0);
        sma_slot(st);
        // next step's page id: a scalar load here only joins the full LDS
        // waits of the last MFMAs
        if (st == 27) pg_next = k + 3 < n ? chunk_page(k + 3) : 0;
        if constexpr (kFp8) {
          if (dq) {
            if (st == 0) dq_load(k + 1, tid_s);
            else if (st >= 10 && st < 26) dq_part(k + 1, st - 10, tid_s);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      sp = sn;
      m_prev = m_run == -INFINITY ? 0.f : m_run;
    };

    // ---- fp8 matrix-core mode: one pipeline step k ----
    // Scores and softmax are per row, as in the other modes: wave w owns rows
    // 32 w .. 32 w + 31 of the group. The weighted sum is split by columns
    // instead: wave w accumulates O^T for columns 128 w .. 128 w + 127 of all
    // 128 rows (the same 16 accumulator tiles), so each transposed code
    // fragment is read and widened once and multiplies the weights of all
    // four row blocks. The weights of chunk k are exchanged through LDS: each
    // wave stores its rows' bf16 weight fragments (in the B-operand layout)
    // into buffer k % 2 at the end of step k, and every wave reads all four in
    // step k + 1, after the barrier that opens it.
    //   phase 1: scores of chunk k: 8 fp8 MFMAs over the 512 code lanes
    //            (codes as stored, queries e4m3 with block scales) into one
    //            accumulator and 4 bf16 MFMAs over the 64 rope lanes into
    //            another, with the copy of chunk k + 2;
    //   phase 2: weighted sum of chunk k - 1 on the bf16 matrix cores (codes
    //            read transposed with ds_read_b64_tr_b8 and widened to bf16 in
    //            registers, exactly), interleaved with chunk k's scores
    //            (s_j times the code part plus the rope part), mask, row max,
    //            lazy reference update, weights w = 2^(c s - m) s_j (rounded
    //            to bf16; the row sum takes the unrounded 2^(c s - m)) and
    //            their store.
    // The token scale is applied once per score and once per weight:
    // c_j = s_j code_j, so s_j (q . code_j) is the content score and
    // sum_j p_j s_j code_j the weighted sum.
    F8MCopyPlan cp8 = f8m_copy_plan(w, static_cast<int>(lane_now()));
    const int one127 = 127;   // E8M0 1.0: the code operand is not scaled
    // weight buffers (2 x 8 KB, in the query staging region, which is idle
    // after the prologue): buffer q, row block rb, token step cc, lane l
    const uint32_t wbuf0 = lds0 + kS * kF8MStage;
    auto wslot = [&](int q, int rbk, int cc) {
      return wbuf0 + (q & 1) * 8192 + rbk * 2048 + cc * 1024 + lane_now() * 16;
    };
    // zero the weights of "chunk -1" (buffer 1), which step 0 multiplies
    auto clear_w = [&]() {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
            static_cast<uintptr_t>(wslot(1, w, cc))) = u32x4{0u, 0u, 0u, 0u};
    };
    auto step8 = [&](int k, int pg) {
      const uint32_t bq = stage_of(k);
      const uint32_t bv = k == 0 ? bq : stage_of(k + kS - 1);
      const bool copy = k + 2 < n;
      const int cnv = copy ? chunk_valid(k + 2) : kChunk;
      const int64_t pgc = pg;
      const uint8_t* csrc = cache + pgc * (64LL * kF8Row) + ((k + 2) & 1) * (kChunk * kF8Row);
      const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(
          cache_scale + pgc * 64 + ((k + 2) & 1) * kChunk);
      asm volatile("" : "+s"(csrc), "+s"(ssrc));
      const uint32_t cbuf = stage_of(k + 2);
      const bool cfast = copy && cnv == kChunk;
      if (copy && !cfast) issue(k + 2);
      const uint8_t* csw = csrc + 8 * w * kF8Row;
      uint32_t qb0 = f8_qb[0], qb1 = f8_qb[1], rb = rope_base8, vb = f8_pv;
      asm volatile("" : "+v"(qb0), "+v"(qb1), "+v"(rb), "+v"(vb));
      int tid_s = static_cast<int>(threadIdx.x);
      asm volatile("" : "+v"(tid_s));
      const uint32_t a0 = bq + qb0, a1 = bq + qb1, ar = bq + rb, av = bv + vb;
      auto copy_fast8 = [&](int i) {
        if (i < 4) lds_dma16(csw + 2 * i * kF8Row, cp8.code[i], cbuf + (4 * w + i) * 1024);
        else if (i == 4) lds_dma16(csw, cp8.rope, cbuf + kF8MRope + w * 1024);
        else if ((tid_s & 63) < 2)
          lds_dma16(ssrc, (8 * w + 4 * (tid_s & 63)) * 4, cbuf + kF8MScales + w * 32);
      };
      auto kfrag8 = [&](int kb) {
        const i32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
            static_cast<uintptr_t>(a0 ^ (64 * kb)));
        const i32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
            static_cast<uintptr_t>(a1 ^ (64 * kb)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      auto rfrag8 = [&](int kk) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            static_cast<uintptr_t>(ar ^ (kk << 5)));
      };
      // V^T fragment g = 4 cc + mb: columns 128 w + 32 mb, tokens 16 cc ..
      auto vraw8 = [&](int g) {
        const int mb = 4 * w + (g & 3), cc = g >> 2;
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(static_cast<uintptr_t>((av ^ (32 * mb)) + 8192 * cc)));
      };
      auto vcvt = [](i32x2 r) {
        const bf16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, false);
        const bf16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, true);
        const bf16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, false);
        const bf16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, true);
        return bf16x8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
      };
      // weight fragment (token step cc, row block rbk) of chunk k - 1
      auto wfrag = [&](int cc, int rbk) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            static_cast<uintptr_t>(wslot(k + 1, rbk, cc)));
      };
      i32x8 kf[3];
      bf16x8 rf[3];
      i32x2 vr[3];
      bf16x8 va[2];
      bf16x8 pb[8];            // weights of chunk k - 1: [cc][row block]
      bf16x8 pw[2];            // this wave's weights of chunk k: [cc]
      f32x4 scl4[4];           // token scales of chunk k (tokens 8 a + 4 half + 0..3)
      f32x16 sc, sr;           // code and rope parts of chunk k's scores

      // ---- phase 1 ----
      kf[0] = kfrag8(0);
      kf[1] = kfrag8(1);
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        if (j < 8) {
          if (j + 2 < 8) kf[(j + 2) % 3] = kfrag8(j + 2);
          else rf[(j - 6) % 3] = rfrag8(j - 6);
          mfma8_s(j == 0, j & 3, sc, kf[j % 3], qf8[j], one127, qs8[j >> 2]);
        } else {
          const int kk = j - 8;
          if (kk + 2 < 4) rf[(kk + 2) % 3] = rfrag8(kk + 2);
          if (kk == 0) mfma_s_first(sr, rf[0], qr8[0]);
          else if (kk == 3) mfma_s_last(sr, rf[kk % 3], qr8[kk]);
          else mfma_s(sr, rf[kk % 3], qr8[kk]);
        }
        if (j == 0) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
            scl4[a] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                static_cast<uintptr_t>(bq + kF8MScales + 32 * a + 16 * half));
        }
        if (j < kF8MCopies && cfast) copy_fast8(j);
        // the weighted sum's first operands
        if (j == 6) {
#pragma unroll
          for (int q = 0; q < 4; ++q) pb[q] = wfrag(0, q);
        }
        if (j == 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) pb[4 + q] = wfrag(1, q);
        }
        if (j == 9) vr[0] = vraw8(0);
        if (j == 10) vr[1] = vraw8(1);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- phase 2 ----
      const bool part = tok0 + kChunk * k + kChunk > tend_all;   // wave-uniform
      f32x16 sn;
      float mx = -INFINITY;
      auto sma8 = [&](int s) {
        if (s == 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sn[r] = fmaf(sc[r], scl4[r >> 2][r & 3], sr[r]);
          if (part) {
            // tokens at or past the row's visible end get -inf; scales of
            // rows past the chunk's valid rows (copied from row 0) get 0, so
            // that their zero weights stay zero
            const int base = tok0 + kChunk * k + 4 * half;
            const int lim = tend - base, nvr = tok1 - base;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int idx = (r & 3) + 8 * (r >> 2);
              sn[r] = idx < lim ? sn[r] : -INFINITY;
              scl4[r >> 2][r & 3] = idx < nvr ? scl4[r >> 2][r & 3] : 0.f;
            }
          }
        } else if (s >= 2 && s < 10) {
          const int q = s - 2;
          asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(sn[2 * q]), "v"(sn[2 * q + 1]));
          asm volatile("" : "+v"(mx));
        } else if (s == 10) {
          const auto xs = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(xs[0]), __uint_as_float(xs[1])) * c;
          asm volatile("" : "+v"(mx));
        } else if (s == 11) {
          const bool up = mx > m_run + kRescaleLog2;
          raise = raise || (up && m_run != -INFINITY);
          m_run = up ? mx : m_run;
        } else if (s >= 12 && s < 20) {
          // weights of chunk k, two tokens per slot
          const int r = 2 * (s - 12);
          const float mref = m_run == -INFINITY ? 0.f : m_run;
          float p0 = __builtin_amdgcn_exp2f(fmaf(sn[r], c, -mref));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sn[r + 1], c, -mref));
          const bf16x2 two = {static_cast<__bf16>(p0 * scl4[r >> 2][r & 3]),
                              static_cast<__bf16>(p1 * scl4[r >> 2][(r & 3) + 1])};
          pw[r >> 3][r & 7] = two[0];
          pw[r >> 3][(r & 7) + 1] = two[1];
          l_lane += p0 + p1;
          asm volatile("" : "+v"(l_lane));
        } else if (s == 20 || s == 21) {
          const int cc = s - 20;
          *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(
              static_cast<uintptr_t>(wslot(k, w, cc))) = pw[cc];
        }
      };
      va[0] = vcvt(vr[0]);
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const int g = st >> 2, rbk = st & 3;   // code fragment, row block
        if (rbk == 0 && g + 2 < 8) vr[(g + 2) % 3] = vraw8(g + 2);
        o[4 * rbk + (g & 3)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            va[g & 1], pb[4 * (g >> 2) + rbk], o[4 * rbk + (g & 3)], 0, 0, 0);
        if (rbk == 2 && g + 1 < 8) va[(g + 1) & 1] = vcvt(vr[(g + 1) % 3]);
        sma8(st);
        if (st == 27) pg_next = k + 3 < n ? chunk_page(k + 3) : 0;
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    zero_o();
    clear_prev();
    __syncthreads();   // earlier reads of every stage are done
    // nothing of this piece is in flight yet: a full wait here also completes
    // any reload of a spilled value the compiler placed before this point,
    // so that no wait for it lands among the copies below
    MLA_WAIT_VM(0);
    // Prologue: the first half of the queries and chunk 0 in flight; the
    // half read into registers; the second half and chunk 1 in flight; wait
    // for all but chunk 1 (copies complete in order). The query regions are
    // the ring's last two stages, which chunks 0 and 1 do not use.
    constexpr int kCopies = kF8M ? kF8MCopies : (kFp8 ? kF8CopiesPerChunk : kCopiesPerChunk);
    q_copy(0);
    issue(0);
    MLA_WAIT_VM(kCopies);          // this wave's first query half
    if constexpr (kF8M) q_read8(0);
    else q_read(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): read before it is overwritten
    q_copy(1);
    if (n > 1) {
      issue(1);
      MLA_WAIT_VM(kCopies);        // the second half and chunk 0
    } else {
      MLA_WAIT_VM(0);
    }
    if constexpr (kF8M) {
      q_read8(1);                  // (negates the queries itself)
      __syncthreads();             // every wave has read its queries: the region
      clear_w();                   // now holds the weight buffers
    } else {
      q_read(1);
    }
    if constexpr (kFp8) {
      __syncthreads();             // every wave's copies of chunk 0 have landed
      dequant(0);
    }
    if constexpr (!kF8M) {
      if (p.neg_q) negate_q();
    }
    // Chunk loop. A row whose max rose past the lazy threshold makes its wave
    // raise a flag at the end of the pass; then the piece restarts in place
    // from its first chunk with the raised maxima (every wave sees the same
    // flags, so all restart together).
    pg_next = n > 2 ? chunk_page(2) : 0;
    for (int k = 0; k <= n; ++k) {
      const int pg = pg_next;
      if constexpr (kFp8) {
        // chunk k was dequantised in the previous step (or the prologue);
        // chunk k + 1 must have landed in its staging buffer
        if (k + 1 < n) MLA_WAIT_VM(0);
        __syncthreads();
        // the step dequantises chunk k + 1 into stage (k + 1) % 3 (which last
        // held chunk k - 2) and copies chunk k + 2 into staging buffer k % 2
        // (which held chunk k): both were done with before the barrier
      } else {
        if (k > 0 && k < n) {
          if (k + 1 < n) MLA_WAIT_VM(kCopies);   // this wave's copies of chunk k
          else MLA_WAIT_VM(0);
        }
        __syncthreads();     // ... and every other wave's
      }
      if constexpr (kF8M) step8(k, pg);
      else step(k, pg);
      if (k == n) {        // end of the pass: no copy is in flight
        const bool any_raise = __any(raise);
        if (lane == 0) restart_flag[w] = any_raise ? 1 : 0;
        __syncthreads();
        if (restart_flag[0] | restart_flag[1] | restart_flag[2] | restart_flag[3]) {
          __syncthreads();   // every wave has read the flags
          zero_o();
          clear_prev();
          raise = false;
          if constexpr (kF8M) clear_w();
          start();
          pg_next = n > 2 ? chunk_page(2) : 0;
          k = -1;
        }
      }
    }

    // ---- epilogue: the unnormalised partial, its row sum and log-sum-exp ----
    // O^T sits in the MFMA layout (lane = row, registers = columns). Four
    // passes of 128 columns each: the wave stores its 32 x 128 fp32 block
    // into LDS straight from the accumulation registers (no vector-ALU work),
    // then reads it back two rows per instruction and writes coalesced rows.
    // The combine divides by the row sum (l_part), which saves the 256
    // per-lane multiplications a normalisation here would cost. The partial
    // is written with non-temporal stores: it is read once, by the combine.
    // LDS rows are 528 bytes (128 fp32 + 16): the 16 rows of a write
    // instruction's lane group then fall in distinct bank groups.
    const float l_row = l_lane + __shfl_xor(l_lane, 32, 64);
    const int64_t slot = slot_of(g, b);
    constexpr int kEpiRow = 528;
    const uint32_t li = lane_now();
    const uint32_t ewave = lds0 + w * 32 * kEpiRow;
    const uint32_t ewr = ewave + (li & 31) * kEpiRow + (li >> 5) * 16;   // row l32, unit half
    const uint32_t erd = ewave + (li >> 5) * kEpiRow + (li & 31) * 16;   // row li / 32, unit li % 32
    // rows of pass qq: the wave's own 32 rows (columns 128 qq ..), or in the
    // fp8 matrix-core mode row block qq (the wave's columns 128 w ..)
    // (a whole-sequence piece: output rows b * rows + ..., each divided by its
    // row sum, whose inverses the row owners publish in LDS first)
    const int64_t rowg = (whole ? static_cast<int64_t>(b) : slot) * p.rows + rg * kMfmaRows;
    if (whole && (li >> 5) == 0) inv_lds[w * 32 + (li & 31)] = l_row > 0.f ? 1.f / l_row : 0.f;
    __syncthreads();                           // every wave is done with the stages
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      // columns 32 mb + 8 j + 4 half + (0..3) of tile mb = 4 qq + t sit in
      // registers 4 j .. 4 j + 3: LDS bytes 128 t + 32 j of the row's unit half
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x16& ot = o[4 * qq + t];
        const f32x4 q0 = ot.s0123, q1 = ot.s4567, q2 = ot.s89ab, q3 = ot.scdef;
        asm volatile("ds_write_b128 %0, %1 offset:%2" :: "v"(ewr), "a"(q0), "i"(128 * t) : "memory");
        asm volatile("ds_write_b128 %0, %1 offset:%2" :: "v"(ewr), "a"(q1), "i"(128 * t + 32) : "memory");
        asm volatile("ds_write_b128 %0, %1 offset:%2" :: "v"(ewr), "a"(q2), "i"(128 * t + 64) : "memory");
        asm volatile("ds_write_b128 %0, %1 offset:%2" :: "v"(ewr), "a"(q3), "i"(128 * t + 96) : "memory");
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the block is in LDS
      __builtin_amdgcn_wave_barrier();
      // rows 2 s2 and 2 s2 + 1 per instruction: a scalar row base plus the
      // lane's offset (row li / 32, columns 128 qq + 4 (li % 32) ...)
      // (all 16 reads of the pass are issued before the first conversion)
      const uint32_t eoff = (li >> 5) * kDc + 4 * (li & 31);
      f32x4 ev[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2)
        ev[s2] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
            static_cast<uintptr_t>(erd + 2 * s2 * kEpiRow));
      const int64_t row0 = rowg + 32 * (kF8M ? qq : w);
      const int col0 = 128 * (kF8M ? w : qq);
      if (whole) {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
          ev[s2] *= inv_lds[32 * (kF8M ? qq : w) + 2 * s2 + static_cast<int>(li >> 5)];
      }
      void* const obase = whole ? o_out : o_part;
      // rows 2 s2 + li / 32 of the block exist below `lim` (all of them but
      // in a padded group)
      const int lim = rv - 32 * (kF8M ? qq : w) - static_cast<int>(li >> 5);
      auto store_rows = [&](auto pred) {
        if (p.part_bf16) {
          uint16_t* ob = static_cast<uint16_t*>(obase) + row0 * kDc + col0;
#pragma unroll
          for (int s2 = 0; s2 < 16; ++s2) {
            const bf16x2 lo = {static_cast<__bf16>(ev[s2][0]), static_cast<__bf16>(ev[s2][1])};
            const bf16x2 hi = {static_cast<__bf16>(ev[s2][2]), static_cast<__bf16>(ev[s2][3])};
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 u = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            if (!decltype(pred)::value || 2 * s2 < lim)
              __builtin_nontemporal_store(u, reinterpret_cast<u32x2*>(ob + 2 * s2 * kDc + eoff));
          }
        } else {
          float* ob = static_cast<float*>(obase) + row0 * kDc + col0;
#pragma unroll
          for (int s2 = 0; s2 < 16; ++s2)
            if (!decltype(pred)::value || 2 * s2 < lim)
              __builtin_nontemporal_store(ev[s2], reinterpret_cast<f32x4*>(ob + 2 * s2 * kDc + eoff));
        }
      };
      if (rv == kMfmaRows) store_rows(bool_c<false>{});
      else store_rows(bool_c<true>{});
      __builtin_amdgcn_s_waitcnt(0xC07F);      // the reads are done before the next pass
      __builtin_amdgcn_wave_barrier();
    }
    if ((li >> 5) == 0 && w * 32 + static_cast<int>(li & 31) < rv) {
      const float lse = l_row > 0.f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
      const int64_t r = rowg + w * 32 + static_cast<int>(li & 31);
      if (whole) {
        if (lse_out != nullptr) lse_out[r] = lse;
      } else {
        lse_part[r] = lse;
        l_part[r] = l_row;
      }
    }
  }
}

}  // namespace

bool mfma_fp8_math(const mla_decode_desc* d) {
  return d->cache_dtype == MLA_FP8_E4M3 && (d->flags & MLA_DECODE_FP8_MATH) != 0;
}

bool mfma_lds_plan(const mla_decode_desc* d) {
  return d->batch <= (mfma_fp8_math(d) ? kF8MMaxLdsBatch : kMaxLdsBatch);
}

bool mfma_supports(const mla_decode_desc* d) {
  return d->d_c == kDc && d->d_rope == kDr &&
         (d->cache_dtype == MLA_BF16 || d->cache_dtype == MLA_FP8_E4M3) &&
         d->q_dtype == MLA_BF16;
}

mla_status launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  const mla_decode_desc* d = a.d;
  MfmaParams p;
  p.part_bf16 = a.p->part_bf16;
  // the kernel scales scores by a positive factor (masked scores are -inf,
  // and -inf * 0 would be NaN); a zero scale becomes FLT_MIN, which leaves
  // every finite score's exponential at exactly 1
  p.c_log2 = fmaxf(fabsf(a.scale) * 1.4426950408889634f, 1.17549435e-38f);
  p.neg_q = a.scale < 0.f ? 1 : 0;
  p.B = d->batch;
  p.q_len = d->q_len;
  p.n_h = d->n_heads;
  p.max_blocks = d->max_blocks_per_seq;
  p.rows = a.p->rows;
  p.row_groups = a.p->row_groups;
  p.G = a.p->G;
  const int64_t g_pad = (a.p->G + 7) / 8 * 8;
  const dim3 grid(static_cast<unsigned>(g_pad * a.p->row_groups)), block(256);
  const bool lds_plan = mfma_lds_plan(d), fp8 = d->cache_dtype == MLA_FP8_E4M3;
  const int mode = fp8 ? (mfma_fp8_math(d) ? 2 : 1) : 0;
  auto kernel = lds_plan ? (mode == 2 ? decode_mfma_bf16<true, 2>
                            : mode == 1 ? decode_mfma_bf16<true, 1> : decode_mfma_bf16<true, 0>)
                         : (mode == 2 ? decode_mfma_bf16<false, 2>
                            : mode == 1 ? decode_mfma_bf16<false, 1> : decode_mfma_bf16<false, 0>);
  hipLaunchKernelGGL(kernel, grid, block, 0, st, static_cast<const uint16_t*>(a.q_abs),
                     static_cast<const uint16_t*>(a.q_rope), static_cast<const uint8_t*>(a.cache),
                     a.cache_scale, a.block_table, a.seq_lens, const_cast<int32_t*>(a.page_start),
                     a.o_part, a.lse_part, a.l_part, a.o_latent, a.lse_out, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode_mfma launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
