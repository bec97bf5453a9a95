// gemm_mfma.hip — bf16 matrix-core GEMM for the dense projections of the
// unabsorbed (prefill) form of MLA: the down-projection to the cached latent
// ([Mishra] "Multi-head Latent Attention", "Step 1: a low-rank latent"), the
// up-projections of the latent to per-head keys and values and of the query
// ([Zhang] "Multi-head latent attention", "The definitions: project down,
// then up"), and the output projection W^O.
//
//   C[m, n] = sum_k A[m, k] B[n, k]      A [M, K], B [N, K]: bf16, row-major
//
// (activations times the transpose of a weight stored [out, in]), fp32
// accumulation, C in fp32 or bf16 (round to nearest even).
//
// Workgroup = 128 x 128 output tile, 4 wavefronts in 2 x 2, each 64 x 64 as
// 2 x 2 v_mfma_f32_32x32x16_bf16 tiles. K advances 64 at a time through a
// double-buffered LDS tile whose rows are padded to 144 bytes: the 16-byte
// fragment reads of 8 or 16 consecutive rows then fall in distinct bank
// groups. Global loads go through three register sets: a K step's loads
// are issued three steps before its chunks are stored to LDS, so two steps of
// matrix work besides the current one cover their latency. Rows past M or N
// read the last row (their outputs are not stored), and A chunks past the end
// of a split's k range are zeroed in LDS.
// Split-K (for skinny M, where the output tiles alone do not fill the chip)
// writes fp32 partial tiles that a second kernel sums in split order.
#include <type_traits>

#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// Epilogue stores of the large tile. Its MFMAs take the B fragment as their
// first operand, so accumulator tile (i, j) holds C^T: register 4 q + e of
// lane (half, l32) is C[l32][8 q + 4 half + e] of the 32 x 32 tile, and each
// lane stores runs of four consecutive outputs of one row with one 16-byte
// (fp32) or 8-byte (bf16) store (measured on the prefill projections: 0.242
// -> 0.230 ms at 4096 x 16384 x 1536 with a bf16 output, 0.122 -> 0.113 ms at
// 4096 x 8192 x 1536 with an fp32 one; on the 128 x 128 tile the same stores
// were 4% slower than one output per store). wide_ok: the row stride is a
// multiple of 4 and the base is aligned for those stores; otherwise, and in
// tiles at the edge of C, the four outputs go one by one, each within bounds.
__device__ __forceinline__ void put4(float* q, f32x4v_t v) { *reinterpret_cast<f32x4v_t*>(q) = v; }
__device__ __forceinline__ void put4(uint16_t* q, f32x4v_t v) {
  u32x2v_t u;
  u[0] = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u[1] = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<u32x2v_t*>(q) = u;
}
__device__ __forceinline__ void put1(float* q, float v) { *q = v; }
__device__ __forceinline__ void put1(uint16_t* q, float v) { *q = f32_to_bf16(v); }
template <class T>
__device__ __forceinline__ bool wide_ok(const T* base, int64_t ld) {
  return (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(base) & (4 * sizeof(T) - 1)) == 0;
}
// four outputs v of row m, columns n .. n + 3
template <class T>
__device__ __forceinline__ void store_run(T* base, int64_t ld, int64_t m, int64_t n, f32x4v_t v,
                                          bool fast, int64_t M, int64_t N) {
  if (fast) {
    put4(base + m * ld + n, v);
  } else if (m < M) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) put1(base + m * ld + n + e, v[e]);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;   // elements per LDS row (144 bytes)

__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(MfmaGemmArgs g, int k_per_split) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kPitch];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  const int kz = blockIdx.z;
  const int kb = kz * k_per_split;
  const int ke = min(g.K, kb + k_per_split);

  // thread tid loads 16-byte chunks c = tid + 256 j (j < 4) of each tile:
  // row c / 8 = tid / 8 + 32 j, elements 8 (tid % 8) .. + 7. The row
  // pointers are formed once; rows past M or N read the last row (their
  // outputs are not stored). Every stage runs the same loads: a chunk at or
  // past the split's end reads the split's last chunk of the row instead
  // (finite values, already cached), and A chunks at or past the split's end
  // are zeroed when the stage is stored to LDS, which zeroes their products.
  const int r8 = tid >> 3, kc = (tid & 7) * 8;
  const uint16_t* pa[4];
  const uint16_t* pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pa[j] = g.A + min(m0 + r8 + 32 * j, static_cast<int64_t>(g.M) - 1) * g.lda + kc;
    pb[j] = g.B + min(n0 + r8 + 32 * j, static_cast<int64_t>(g.N) - 1) * g.ldb + kc;
  }
  const int klim = ke - 8 - kc;   // the split's last chunk start in a row, minus kc
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  // kPF register sets of staged chunks: the loads of step s + kPF are issued
  // at the start of step s, so a load has kPF - 1 whole steps of matrix work
  // and the step it is issued in to arrive before its chunks go to LDS.
  constexpr int kPF = 3;
  u32x4_t ra[kPF][4], rb[kPF][4];
  auto gload = [&](auto SET, int k0) {
    constexpr int st = decltype(SET)::value;
    const int kk = min(k0, klim);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[st][j] = *reinterpret_cast<const u32x4_t*>(pa[j] + kk);
      rb[st][j] = *reinterpret_cast<const u32x4_t*>(pb[j] + kk);
    }
  };
  auto swrite = [&](auto SET, int buf, int k0) {
    constexpr int st = decltype(SET)::value;
    // 0 for A chunks at or past the split's end (the first test is uniform)
    const uint32_t keep = k0 + kBK > ke && k0 + kc >= ke ? 0u : ~0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = r8 + 32 * j;
      *reinterpret_cast<u32x4_t*>(&As[buf][row * kPitch + kc]) = ra[st][j] & keep;
      *reinterpret_cast<u32x4_t*>(&Bs[buf][row * kPitch + kc]) = rb[st][j];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  auto mfmas = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int col = kk * 16 + half * 8;
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][(wm * 64 + i * 32 + l32) * kPitch + col]);
        b[i] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][(wn * 64 + i * 32 + l32) * kPitch + col]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  typedef std::integral_constant<int, 2> S2;
  static_assert(kPF == 3, "the step sequence below names three sets");
  // step s: its chunks are in LDS buffer s % 2 and came from set s % kPF,
  // which is free again; the next step's chunks wait in set (s + 1) % kPF.
  auto step = [&](auto SET, int s) {
    constexpr int st = decltype(SET)::value;
    const int k0 = kb + s * kBK;
    gload(SET, k0 + kPF * kBK);
    mfmas(s & 1);
    swrite(std::integral_constant<int, (st + 1) % kPF>{}, (s + 1) & 1, k0 + kBK);
    __syncthreads();
  };
  const int n = kb < ke ? (ke - kb + kBK - 1) / kBK : 0;   // K steps of this split
  gload(S0{}, kb);
  gload(S1{}, kb + kBK);
  gload(S2{}, kb + 2 * kBK);
  swrite(S0{}, 0, kb);
  __syncthreads();
  int s = 0;
  for (; s + kPF <= n; s += kPF) {
    step(S0{}, s);
    step(S1{}, s + 1);
    step(S2{}, s + 2);
  }
  if (s < n) step(S0{}, s);
  if (s + 1 < n) step(S1{}, s + 1);

  // acc[i][j] register r holds C[m][n] with m = 8 (r / 4) + 4 half + r % 4 and
  // n = l32 within the 32 x 32 tile (i, j). One pass per output form; the
  // row offsets are uniform multiples of the row stride, and only a tile at
  // the edge of C tests bounds.
  const bool edge = m0 + kBM > g.M || n0 + kBN > g.N;
  const int64_t mw = m0 + wm * 64 + 4 * half, nw = n0 + wn * 64 + l32;
  auto store_all = [&](auto* base, int64_t ld, auto put) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        auto* t = base + (mw + i * 32) * ld + nw + j * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dm = 8 * (r >> 2) + (r & 3);
          if (edge && (mw + i * 32 + dm >= g.M || nw + j * 32 >= g.N)) continue;
          put(t + dm * ld, acc[i][j][r]);
        }
      }
  };
  if (g.splits > 1)
    store_all(g.partial + static_cast<int64_t>(kz) * g.M * g.N, static_cast<int64_t>(g.N),
              [](float* q, float v) { *q = v; });
  else if (g.c_bf16)
    store_all(static_cast<uint16_t*>(g.C), g.ldc, [](uint16_t* q, float v) { *q = f32_to_bf16(v); });
  else
    store_all(static_cast<float*>(g.C), g.ldc, [](float* q, float v) { *q = v; });
}

// ---- large-tile variant: 256 x 256 output tile, one wavefront per SIMD ----
// Workgroup = 4 wavefronts in 2 x 2, each 128 x 128 as 4 x 4
// v_mfma_f32_32x32x16_bf16 tiles (its 256 accumulation registers): every
// 16-byte fragment read from LDS feeds four MFMAs, against two in the 128 x 128
// tile. K advances 32 at a time through a ring of five 32 KB LDS stages (the
// whole LDS; A 256 x 32 and B 256 x 32 bf16) filled straight from memory with
// global_load_lds_dwordx4 (no register round trip), four stages ahead; each
// stage's fragments are read during the previous stage's MFMAs, so about
// three stages of matrix work cover the memory latency and one the LDS
// latency. A stage
// row is 64 bytes; 16-byte unit u of row r sits at position u ^ ((r >> 2) & 3),
// which puts the fragment reads of 16 consecutive rows in distinct bank
// groups. Rows past M or N are read from row M - 1 or N - 1 and their outputs
// are not stored; the k range of a split must be a multiple of 32.
constexpr int kLM = 256, kLN = 256, kLK = 32, kLS = 5;
#ifndef MLA_GEMM_BIG_MIN_TILES
#define MLA_GEMM_BIG_MIN_TILES 240   // smallest grid (tiles x splits) the large tile takes
#endif
#ifndef MLA_GEMM_BIG_MIN_K
#define MLA_GEMM_BIG_MIN_K 1024      // smallest k range per split it takes
#endif
constexpr int kLStage = (kLM + kLN) * kLK * 2;   // 32 KB
constexpr int kLCopies = 8;                      // copy instructions per wavefront and stage

__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// s_waitcnt vmcnt(n), expcnt and lgkmcnt left free (gfx9 encoding)
#define GEMM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// f(integral_constant<int, I>) for I = 0 .. 3, unrolled at compile time
template <class F>
__device__ __forceinline__ void static_for4(F&& f) {
  f(std::integral_constant<int, 0>{});
  f(std::integral_constant<int, 1>{});
  f(std::integral_constant<int, 2>{});
  f(std::integral_constant<int, 3>{});
}

// Tile order: workgroup ids congruent mod 8 run on one XCD (the dispatcher
// deals them out in turn), so XCD x is given the x-th contiguous eighth of the
// tiles in a grouped order: groups of kLGroup tile rows, each walked column by
// column. The tiles one XCD runs at a time then share a few A row blocks and
// B column blocks, which its L2 serves after the first read, instead of every
// tile fetching its own from memory.
#ifndef MLA_GEMM_GROUP
#define MLA_GEMM_GROUP 4
#endif
constexpr int kLGroup = MLA_GEMM_GROUP;

__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(MfmaGemmArgs g, int k_per_split,
                                                               int tiles_m, int tiles_n, int tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLS * kLStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int per = (tiles + 7) / 8;
  const int t = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  if (t >= tiles) return;
  const int mn = tiles_m * tiles_n;
  // (the divisions run on the vector unit: readfirstlane keeps the results
  // scalar, as the copy addresses need)
  const int kz = __builtin_amdgcn_readfirstlane(t / mn), rt = t % mn;
  const int grp = rt / (kLGroup * tiles_n), rr = rt % (kLGroup * tiles_n);
  const int gsz = min(kLGroup, tiles_m - grp * kLGroup);
  const int64_t m0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(grp * kLGroup + rr % gsz)) * kLM;
  const int64_t n0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(rr / gsz)) * kLN;
  const int kb = kz * k_per_split;
  const int ke = min(g.K, kb + k_per_split);
  const int nst = ke > kb ? (ke - kb) / kLK : 0;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)smem));

  // copies: wavefronts 0 and 1 fill rows 128 w .. of the A tile, 2 and 3 rows
  // 128 (w - 2) .. of the B tile; instruction j covers 16 rows: lane i reads
  // row 16 j + i / 4, logical unit (i & 3) ^ ((i >> 4) & 3), and lands at
  // byte 1024 j + 16 i of the wavefront's 8 KB
  const bool isA = w < 2;
  const uint8_t* mat = reinterpret_cast<const uint8_t*>(isA ? g.A : g.B);
  const int64_t ld = isA ? g.lda : g.ldb;
  const int64_t lim = (isA ? g.M : g.N) - 1;
  const int64_t r0 = (isA ? m0 : n0) + 128 * (w & 1);
  const uint32_t dst0 = (isA ? 0u : static_cast<uint32_t>(kLM * kLK * 2)) + 8192u * (w & 1);
  uint32_t voff[kLCopies];
#pragma unroll
  for (int j = 0; j < kLCopies; ++j) {
    int64_t row = r0 + 16 * j + (lane >> 2);
    row = row < lim ? row : lim;
    voff[j] = static_cast<uint32_t>(row * ld * 2) + 16u * ((lane & 3) ^ ((lane >> 4) & 3));
  }
  auto issue = [&](int st) {
    const uint8_t* src = mat + 2LL * (kb + kLK * st);
    asm volatile("" : "+s"(src));
    const uint32_t dst = lds0 + (st % kLS) * kLStage + dst0;
#pragma unroll
    for (int j = 0; j < kLCopies; ++j) dma16(src, voff[j], dst + 1024 * j);
  };

  // fragment reads: row r of a tile, unit 2 kk + half, at r * 64 +
  // 16 ((2 kk + half) ^ ((r >> 2) & 3)); (r >> 2) & 3 = (l32 >> 2) & 3
  const uint32_t sw = (l32 >> 2) & 3;
  const uint32_t fa = l32 * 64u + 16u * (static_cast<uint32_t>(half) ^ sw);          // kk = 0
  const uint32_t fb = l32 * 64u + 16u * (static_cast<uint32_t>(2 + half) ^ sw);      // kk = 1
  auto frag = [&](uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(static_cast<uintptr_t>(a));
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  // Software pipeline over a five-slot ring: the 16 fragments of stage st + 1
  // are read from LDS while the 32 MFMAs of stage st run (two fragment sets,
  // alternating at compile time through pairs of steps), so the LDS latency
  // is hidden behind matrix work. The copies of stage st + 4 go out during
  // step st's MFMAs into the slot of stage st - 1, whose fragments every
  // wavefront read during step st - 2, before the barrier of step st - 1.
  // At the top of step st, stage st + 1 must have landed (issued three steps
  // earlier): the copies of stages st + 2 and st + 3 may still be in flight.
  typedef bf16x8_t Frags[2][4];
  auto read_frags = [&](int st, Frags& a, Frags& b) {
    const uint32_t sb = lds0 + (st % kLS) * kLStage;
    const uint32_t sa = sb + wm * 128 * 64, sbb = sb + kLM * kLK * 2 + wn * 128 * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[kk][i] = frag(sa + i * 32 * 64 + (kk ? fb : fa));
        b[kk][i] = frag(sbb + i * 32 * 64 + (kk ? fb : fa));
      }
  };
  auto wait_for = [&](int st) {   // stage st has landed; later issued stages may be in flight
    const int later = min(nst - 1 - st, kLS - 3);
    if (later >= 2) GEMM_WAIT_VM(2 * kLCopies);
    else if (later == 1) GEMM_WAIT_VM(kLCopies);
    else GEMM_WAIT_VM(0);
  };
  auto step = [&](int st, Frags& a, Frags& b, Frags& na, Frags& nb) {
    if (st + 1 < nst) {
      wait_for(st + 1);
      __syncthreads();
      read_frags(st + 1, na, nb);
    }
    // (the copies of stage st + 4 go out one per four MFMAs: issued all at
    // once they would stall the wavefront on the memory queue)
    const bool cp = st + kLS - 1 < nst;
    const uint8_t* csrc = mat + 2LL * (kb + kLK * (st + kLS - 1));
    asm volatile("" : "+s"(csrc));
    const uint32_t cdst = lds0 + ((st + kLS - 1) % kLS) * kLStage + dst0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[kk][j], a[kk][i], acc[i][j], 0, 0, 0);
        if (cp) dma16(csrc, voff[4 * kk + i], cdst + 1024 * (4 * kk + i));
      }
  };
  const int pre = nst < kLS - 1 ? nst : kLS - 1;
  for (int st = 0; st < pre; ++st) issue(st);
  Frags a0, b0, a1, b1;
  if (nst > 0) {
    // stage 0 has landed when at most the copies of stages 1 .. 3 are in flight
    const int later = min(nst - 1, kLS - 2);
    if (later >= 3) GEMM_WAIT_VM(3 * kLCopies);
    else if (later == 2) GEMM_WAIT_VM(2 * kLCopies);
    else if (later == 1) GEMM_WAIT_VM(kLCopies);
    else GEMM_WAIT_VM(0);
    __syncthreads();
    read_frags(0, a0, b0);
  }
  // (pairs of steps with no test between them, then the odd last step: a
  // test inside the pair made the compiler copy the accumulators between
  // register files every pair)
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    step(st, a0, b0, a1, b1);
    step(st + 1, a1, b1, a0, b0);
  }
  if (st < nst) step(st, a0, b0, a1, b1);

  // acc[i][j] holds C^T of the 32 x 32 tile (i, j) of the wavefront's
  // 128 x 128 block (see store_run); one pass per output form, the bounds
  // tests only on edge tiles
  const bool edge = m0 + kLM > g.M || n0 + kLN > g.N;
  const int64_t mw = m0 + wm * 128 + l32, nw = n0 + wn * 128 + 4 * half;
  auto store_all = [&](auto* base, int64_t ld) {
    const bool fast = !edge && wide_ok(base, ld);
    static_for4([&](auto I) {
      static_for4([&](auto J) {
        constexpr int i = decltype(I)::value, j = decltype(J)::value;
        // (the empty asm keeps each tile's reads of the accumulation
        // registers next to its stores: hoisted ahead of the three output
        // forms, they would need more vector registers than there are)
        asm volatile("" : "+a"(acc[i][j]));
        static_for4([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          store_run(base, ld, mw + i * 32, nw + j * 32 + 8 * q,
                    __builtin_shufflevector(acc[i][j], acc[i][j], 4 * q, 4 * q + 1, 4 * q + 2, 4 * q + 3),
                    fast, g.M, g.N);
        });
        // one tile's stores at a time (the addresses of all 64 would not
        // fit the registers)
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };
  // the same stores with the run's two pairs rotated first (a run of four
  // outputs starts at a multiple of 4, so it holds whole pairs of one block)
  auto store_all_rope = [&](uint16_t* base, int64_t ld) {
    const bool fast = !edge && wide_ok(base, ld);
    const int dr = g.rope_dr;
    static_for4([&](auto I) {
      static_for4([&](auto J) {
        constexpr int i = decltype(I)::value, j = decltype(J)::value;
        asm volatile("" : "+a"(acc[i][j]));
        const int64_t m = mw + i * 32;
        const float* cs = g.rope_cs + min(m, static_cast<int64_t>(g.M) - 1) * dr;
        static_for4([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int64_t n = nw + j * 32 + 8 * q;
          f32x4v_t v = __builtin_shufflevector(acc[i][j], acc[i][j], 4 * q, 4 * q + 1, 4 * q + 2, 4 * q + 3);
          const f32x4v_t t = *reinterpret_cast<const f32x4v_t*>(cs + n % dr);
          const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
          v[0] = a0 * t[0] - b0 * t[1];
          v[1] = a0 * t[1] + b0 * t[0];
          v[2] = a1 * t[2] - b1 * t[3];
          v[3] = a1 * t[3] + b1 * t[2];
          store_run(base, ld, m, n, v, fast, g.M, g.N);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };
  if (g.splits > 1)
    store_all(g.partial + static_cast<int64_t>(kz) * g.M * g.N, static_cast<int64_t>(g.N));
  else if (g.rope_cs != nullptr)
    store_all_rope(static_cast<uint16_t*>(g.C), g.ldc);
  else if (g.c_bf16)
    store_all(static_cast<uint16_t*>(g.C), g.ldc);
  else
    store_all(static_cast<float*>(g.C), g.ldc);
}

// C = sum over the splits of the fp32 partial tiles, in split order.
__global__ __launch_bounds__(256) void gemm_split_reduce(MfmaGemmArgs g) {
  const int64_t total = static_cast<int64_t>(g.M) * g.N;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < total; e += static_cast<int64_t>(gridDim.x) * 256) {
    float s = 0.f;
    for (int z = 0; z < g.splits; ++z) s += g.partial[z * total + e];
    const int64_t m = e / g.N, n = e % g.N;
    if (g.c_bf16) static_cast<uint16_t*>(g.C)[m * g.ldc + n] = f32_to_bf16(s);
    else static_cast<float*>(g.C)[m * g.ldc + n] = s;
  }
}

// The split sums for C rows of a multiple of 4 outputs with 16-byte (fp32)
// or 8-byte (bf16) aligned rows: workgroup (x, row) sums 4 consecutive
// outputs per thread, every split's loads issued before the sums, added in
// split order (the same order as above).
__global__ __launch_bounds__(256) void gemm_split_reduce4(MfmaGemmArgs g) {
  typedef float f32x4s __attribute__((ext_vector_type(4)));
  const int64_t m = blockIdx.y;
  const int64_t n = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (n >= g.N) return;
  const int64_t total = static_cast<int64_t>(g.M) * g.N;
  const float* p = g.partial + m * g.N + n;
  f32x4s s = *reinterpret_cast<const f32x4s*>(p);
  for (int z0 = 1; z0 < g.splits; z0 += 4) {
    f32x4s v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (z0 + u < g.splits) v[u] = *reinterpret_cast<const f32x4s*>(p + (z0 + u) * total);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (z0 + u < g.splits) s += v[u];
  }
  if (g.c_bf16) {
    const uint32_t lo = f32_to_bf16(s[0]) | (static_cast<uint32_t>(f32_to_bf16(s[1])) << 16);
    const uint32_t hi = f32_to_bf16(s[2]) | (static_cast<uint32_t>(f32_to_bf16(s[3])) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + m * g.ldc + n) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<f32x4s*>(static_cast<float*>(g.C) + m * g.ldc + n) = s;
  }
}

}  // namespace

int gemm_bf16_k_per_split(int K, int splits) {
  const int per = (K + splits - 1) / splits;
  return (per + kBK - 1) / kBK * kBK;
}

mla_status launch_gemm_bf16(const MfmaGemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return MLA_OK;
  if (g.K % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 || !aligned16(g.A) || !aligned16(g.B))
    return fail(MLA_ERR_MISALIGNED, "bf16 GEMM: K, lda and ldb must be multiples of 8 and A, B "
                "16-byte aligned");
  const int splits = g.splits < 1 ? 1 : g.splits;
  const int kps = splits > 1 ? gemm_bf16_k_per_split(g.K, splits) : (g.K + kBK - 1) / kBK * kBK;
  const int gz = splits > 1 ? (g.K + kps - 1) / kps : 1;
  MfmaGemmArgs a = g;
  a.splits = gz;
  if (gz > 1 && a.partial == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bf16 GEMM: split-K needs a partial buffer");
  // the large tile where its grid still covers the chip, each split runs
  // long enough (at least 1024 k) to repay its deeper pipeline, K is a
  // multiple of its k step and the per-lane 32-bit copy offsets reach every
  // row (measured on the prefill projections: 0.54 -> 0.38 ms at 4096 x 24576
  // x 1536, 0.97 -> 0.92 ms at 4096 x 5120 x 16384; shorter k ranges and
  // grids below the chip run faster on the 128 x 128 tile)
  const int64_t big_tiles = static_cast<int64_t>((g.N + kLN - 1) / kLN) * ((g.M + kLM - 1) / kLM) * gz;
  const bool big = g.K % kLK == 0 && big_tiles >= MLA_GEMM_BIG_MIN_TILES && kps >= MLA_GEMM_BIG_MIN_K &&
                   static_cast<int64_t>(g.M) * g.lda * 2 < (1LL << 32) &&
                   static_cast<int64_t>(g.N) * g.ldb * 2 < (1LL << 32);
  if (g.rope_cs != nullptr &&
      (!big || gz > 1 || !g.c_bf16 || g.rope_dr < 4 || g.rope_dr % 4 != 0 || g.N % g.rope_dr != 0 ||
       (reinterpret_cast<uintptr_t>(g.rope_cs) & 15) != 0))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 GEMM: RoPE in the epilogue needs the large tile, no split, "
                                     "a bf16 output and whole 4-aligned rope blocks");
  if (big) {
    const int tm = (g.M + kLM - 1) / kLM, tn = (g.N + kLN - 1) / kLN;
    const int tiles = tm * tn * gz;
    const unsigned blocks = static_cast<unsigned>((tiles + 7) / 8 * 8);
    hipLaunchKernelGGL(gemm_bf16_big_kernel, dim3(blocks), dim3(256), 0, st, a, kps, tm, tn, tiles);
  } else {
    const dim3 grid(static_cast<unsigned>((g.N + kBN - 1) / kBN), static_cast<unsigned>((g.M + kBM - 1) / kBM),
                    static_cast<unsigned>(gz));
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, a, kps);
  }
  if (gz > 1) {
    const uintptr_t al = g.c_bf16 ? 7u : 15u;
    if (g.N % 4 == 0 && g.ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(g.C) & al) == 0 &&
        aligned16(g.partial) && g.M <= 65535) {
      const dim3 grid4(static_cast<unsigned>((g.N / 4 + 255) / 256), static_cast<unsigned>(g.M));
      hipLaunchKernelGGL(gemm_split_reduce4, grid4, dim3(256), 0, st, a);
    } else {
      const int64_t total = static_cast<int64_t>(g.M) * g.N;
      const unsigned blocks = static_cast<unsigned>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
      hipLaunchKernelGGL(gemm_split_reduce, dim3(blocks), dim3(256), 0, st, a);
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "bf16 GEMM launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
