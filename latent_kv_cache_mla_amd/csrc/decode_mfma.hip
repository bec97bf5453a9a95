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
//     Workgroups of one range but different row groups get block ids that
//     differ by a multiple of 8, so they land on the same XCD and the second
//     read of a page hits that XCD's L2.
//   * a 64-token page is one tile. It is copied HBM -> LDS with direct
//     global-to-LDS loads (no register round trip), double buffered, so the
//     next page streams in while this one is computed.
//   * scores: S^T[32 tok x 32 rows] = K[32 x 576] Q^T[576 x 32] with
//     v_mfma_f32_32x32x16_bf16, tokens as the M dimension: the A operand is
//     read from LDS (16 bytes per lane), Q^T stays in registers all along.
//     In this orientation each lane holds 16 tokens of one row, so the row
//     max and sum are in-lane but for one exchange. The score MFMAs are
//     issued as single asm instructions with vector-register constraints:
//     that keeps the score accumulator out of the accumulation registers,
//     which O^T fills.
//   * online softmax in base 2 with a lazy reference: probabilities are taken
//     relative to a running max m that only moves when a tile's max exceeds it
//     by more than 2^8. Instead of rescaling O then (which would make the
//     compiler keep the 128 accumulator registers on the VALU side of the
//     register file), the workgroup restarts the piece from its first page
//     with the raised m: rare, and exact (O and l are rebuilt against one
//     reference).
//   * weighted sum: O^T[512 x 32] += V^T[512 x 32] P^T[32 x 32]; P^T comes
//     straight from the score accumulator registers (converted to bf16), and
//     V^T is the same LDS page read with the LDS transpose load
//     (ds_read_b64_tr_b16): keys and values are never materialised.
//   * the LDS page layout is XOR-swizzled in 16-byte chunks so that both the
//     row-wise score reads and the transposed value reads are free of bank
//     conflicts.
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kContentBytes = 64 * 1024;      // 64 tokens x 512 bf16
constexpr int kRopeBytes = 64 * 128;          // 64 tokens x 64 bf16
constexpr int kTileBytes = kContentBytes + kRopeBytes;
constexpr int kRowBytes = 2 * (kDc + kDr);    // one cached token, bf16
constexpr float kRescaleLog2 = 8.0f;          // lazy-rescale threshold (2^8)

struct MfmaParams {
  const uint16_t* q_abs;
  const uint16_t* q_rope;
  const uint8_t* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_start;
  float* o_part;
  float* lse_part;
  float c_log2;  // softmax scale * log2(e)
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

// One 16-byte-per-lane global -> LDS copy: lane i's 16 bytes from
// sbase + voff land at LDS address lds + 16 i. Issued as a single instruction
// so that it is not counted as an LDS access by the compiler's wait-count
// logic (which would otherwise drain every LDS read while a copy is in
// flight); its completion is waited for explicitly (vmcnt) before the
// barrier that publishes the page.
__device__ __forceinline__ void lds_dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
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

// Per-lane source offsets of a page copy, precomputed once:
//   content rows t = 16 j + 4 w + i (j, i in 0..3) need logical chunk
//   lane ^ swz(t) of the row, and swz depends on t only through 4 w + i, so
//   four patterns serve all 16 rows of the wave;
//   rope rows are one per 8 lanes: row 8 (2 w + k) + lane / 8 of the page.
struct CopyPlan {
  uint32_t content[4];   // lane byte offset within a content row, per i
  uint32_t rope[2];      // lane byte offset within the page, per rope group, all rows valid
};

__device__ __forceinline__ uint32_t rope_src(int w, int k, int lane, int n_valid) {
  const int t = 8 * (2 * w + k) + (lane >> 3);
  const int ts = t < n_valid ? t : 0;
  return ts * kRowBytes + 2 * kDc + (((lane & 7) ^ swz_rope(t)) << 4);
}

// Copy page `page` (tokens [0, n_valid) valid) into the LDS buffer at `buf`.
// Rows past n_valid are read from row 0 so that every LDS value is finite.
// `w` and `n_valid` are wave-uniform: all row arithmetic is scalar.
__device__ __forceinline__ void load_tile(const uint8_t* cache, int64_t page, int n_valid,
                                          uint32_t buf, int w, int lane, const CopyPlan& cp) {
  const uint8_t* pg = cache + page * (64LL * kRowBytes);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * j + 4 * w + i;
      const int ts = t < n_valid ? t : 0;
      lds_dma16(pg + ts * kRowBytes, cp.content[i], buf + t * 1024);
    }
  if (n_valid == 64) {
#pragma unroll
    for (int k = 0; k < 2; ++k) lds_dma16(pg, cp.rope[k], buf + kContentBytes + (2 * w + k) * 1024);
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      lds_dma16(pg, rope_src(w, k, lane, n_valid), buf + kContentBytes + (2 * w + k) * 1024);
  }
}

__global__ __launch_bounds__(256, 1) void decode_mfma_bf16(MfmaParams p) {
  // two page buffers: page `it` is computed from buffer it & 1 while page
  // it + 1 is copied into the other
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kTileBytes];
  __shared__ int restart_flag[2][4];   // per page parity, per wave

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int half = lane >> 5, l32 = lane & 31;   // k-group and column of the 32x32 layouts
  CopyPlan cp;
#pragma unroll
  for (int i = 0; i < 4; ++i) cp.content[i] = (lane ^ swz(4 * w + i)) << 4;
#pragma unroll
  for (int k = 0; k < 2; ++k) cp.rope[k] = rope_src(w, k, lane, 64);
  const int64_t id = blockIdx.x;
  const int rg = static_cast<int>((id >> 3) % p.row_groups);
  const int64_t g = (id / (8LL * p.row_groups)) * 8 + (id & 7);
  if (g >= p.G) return;
  const int64_t P = p.page_start[p.B];
  const int64_t pb = range_begin(g, P, p.G), pe = range_begin(g + 1, P, p.G);
  if (pb >= pe) return;

  int b = 0;
  {
    int hi = p.B - 1;
    while (b < hi) {
      const int mid = (b + hi) >> 1;
      if (p.page_start[mid + 1] > pb) hi = mid; else b = mid + 1;
    }
  }

  const int my_row = rg * kMfmaRows + w * 32 + l32;     // the row of this lane's columns
  const int m = my_row / p.n_h, hd = my_row % p.n_h;
  const float c = p.c_log2;

  // LDS byte offsets of this lane's fragments. The swizzle only changes
  // offset bits that the unrolled loop constants reach through an XOR, so one
  // base register per pattern suffices: offset = (base ^ (k << s)) + imm.
  const int hx = swz(l32);
  // score A-fragment, token 32 ch + l32, content chunk 2 kc + half:
  //   bits 5..7 = (kc & 7) ^ (hx >> 1), + 256 * (kc >> 3) + 32768 * ch
  const uint32_t qk_base = l32 * 1024 + ((half ^ (hx & 1)) << 4) + ((hx >> 1) << 5);
  // rope chunk 2 kk + half of a 128-byte rope row: bits 5..6 = kk ^ (hr >> 1), + 4096 * ch
  const int hr = swz_rope(l32);
  const uint32_t rope_base = kContentBytes + l32 * 128 + ((half ^ (hr & 1)) << 4) + ((hr >> 1) << 5);
  // transposed value reads: 16-lane group G16 = g16, source lane s16 reads
  // row 4 (g16 >> 1) + (s16 >> 2) (+8 for the second read) of a 16-token
  // chunk, columns 32 mb + 16 (g16 & 1) + 4 (s16 & 3):
  //   bits 6..7 = (mb & 3) ^ (swz >> 2), + 256 * (mb >> 2) + 16384 * chunk
  const int g16 = lane >> 4, s16 = lane & 15;
  uint32_t pv_base[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int t = 4 * (g16 >> 1) + (s16 >> 2) + 8 * sec;
    const int ht = swz(t);
    const int qlow = 2 * (g16 & 1) + ((s16 & 3) >> 1);
    pv_base[sec] = t * 1024 + ((qlow ^ (ht & 3)) << 4) + (s16 & 1) * 8 + ((ht >> 2) << 6);
  }

  for (; b < p.B && p.page_start[b] < pe; ++b) {
    const int64_t s0 = p.page_start[b], s1 = p.page_start[b + 1];
    if (s1 == s0) continue;
    const int64_t a0 = s0 > pb ? s0 : pb, a1 = s1 < pe ? s1 : pe;
    const int n_tiles = static_cast<int>(a1 - a0);
    const int S = clamp_len(p.seq_lens[b], p.max_blocks);
    const int pidx0 = static_cast<int>(a0 - s0);
    const int tok1 = min(S, static_cast<int>((a1 - s0) * 64));
    const int tend = min(tok1, S - p.q_len + m + 1);      // this row's visible end
    // tokens below tend_all are visible to every row of the wave
    int tend_all = tend;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) tend_all = min(tend_all, __shfl_xor(tend_all, off, 64));
    tend_all = __builtin_amdgcn_readfirstlane(tend_all);
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
    // page ids of this piece, 64 at a time: lane i holds page (base + i)
    auto ids_at = [&](int first) {
      const int k = pidx0 + first + lane;
      return (first + lane < n_tiles && k < p.max_blocks) ? bt[k] : 0;
    };
    int ids_cur, ids_nxt;

    // Q^T fragments: per 16-lane k chunk, the lane holds lanes [8 half, 8 half + 8) of its row
    bf16x8 qf[36];
    {
      const int64_t qrow = (static_cast<int64_t>(b) * p.q_len + m) * p.n_h + hd;
      const bf16x8* qa = reinterpret_cast<const bf16x8*>(p.q_abs + qrow * kDc);
      const bf16x8* qr = reinterpret_cast<const bf16x8*>(p.q_rope + qrow * kDr);
#pragma unroll
      for (int kc = 0; kc < 32; ++kc) qf[kc] = qa[2 * kc + half];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[32 + kk] = qr[2 * kk + half];
    }

    f32x16 o[16];
    float m_run = -INFINITY, l_lane = 0.f;
    const uint32_t lds0 = lds_addr(smem);

    // The outer loop runs again only when a row's max rose past the lazy
    // threshold: the piece restarts from its first page with the raised
    // maxima (every wave sees the same flags, so all restart together).
    for (bool again = true; again;) {
      // zero O through the matrix unit: every definition of O is then an
      // MFMA result, and the compiler keeps O in the accumulation registers
      // across the page loop (a vector-ALU zero would make it carry O in the
      // vector registers and copy it in and out on every page)
      {
        const bf16x8 z8 = {};
#pragma unroll
        for (int mb = 0; mb < 16; ++mb)
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z8, z8, f32x16{}, 0, 0, 0);
      }
      l_lane = 0.f;
      again = false;
      ids_cur = ids_at(0);
      ids_nxt = ids_at(64);
      __syncthreads();   // earlier reads of both buffers are done
      load_tile(p.cache, __builtin_amdgcn_readlane(ids_cur, 0), min(64, tok1 - pidx0 * 64), lds0, w,
                lane, cp);

      for (int it = 0;; ++it) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of page `it`
        __syncthreads();                      // ... and every other wave's, and their flags
        if (it > 0) {
          const int* f = restart_flag[(it - 1) & 1];
          if (f[0] | f[1] | f[2] | f[3]) {
            again = true;
            break;
          }
        }
        if (it == n_tiles) break;
        const uint32_t cur = (it & 1) * kTileBytes;
        const uint32_t next = lds0 + (kTileBytes - cur);
        // this page's fragment bases (cur only sets bits 13 and 16, which the
        // XOR constants below never touch)
        const uint32_t qk_pg = lds0 + cur + qk_base, rope_pg = lds0 + cur + rope_base;
        const uint32_t pv_pg0 = lds0 + cur + pv_base[0], pv_pg1 = lds0 + cur + pv_base[1];
        const int pidx = pidx0 + it;
        if (it + 1 < n_tiles) {
          if (((it + 1) & 63) == 0) {   // roll the page-id window
            ids_cur = ids_nxt;
            ids_nxt = ids_at(it + 65);
          }
          load_tile(p.cache, __builtin_amdgcn_readlane(ids_cur, (it + 1) & 63),
                    min(64, tok1 - (pidx + 1) * 64), next, w, lane, cp);
        }
        bool raise = false;   // some row of this wave crossed the lazy threshold

#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          // ---- scores S^T = K Q^T for tokens [32 ch, 32 ch + 32) ----
          // the per-half bases differ in the expression, so nothing is shared
          // (and kept live) across the halves
          const uint32_t qk_h = ch ? (qk_pg + 32768) : qk_pg;
          const uint32_t rope_h = ch ? (rope_pg + 4096) : rope_pg;
          auto kfrag = [&](int kc) {
            const uint32_t a = kc < 32 ? (qk_h ^ ((kc & 7) << 5)) + (kc >> 3) * 256
                                       : rope_h ^ ((kc - 32) << 5);
            return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                static_cast<uintptr_t>(a));
          };
          // A fragments are read kD steps ahead of their MFMAs; the
          // scheduling barriers pin that order
          constexpr int kD = 3;
          bf16x8 kf[kD + 1];
#pragma unroll
          for (int j = 0; j < kD; ++j) kf[j] = kfrag(j);
          f32x16 sc;
#pragma unroll
          for (int kc = 0; kc < 36; ++kc) {
            if (kc + kD < 36) kf[(kc + kD) % (kD + 1)] = kfrag(kc + kD);
            if (kc == 0) mfma_s_first(sc, kf[0], qf[0]);
            else if (kc == 35) mfma_s_last(sc, kf[kc % (kD + 1)], qf[kc]);
            else mfma_s(sc, kf[kc % (kD + 1)], qf[kc]);
            __builtin_amdgcn_sched_barrier(0);
          }

          // ---- scale to log2 units, mask tokens at or past this row's end ----
          float mx = -INFINITY;
          if (pidx * 64 + 32 * ch + 32 <= tend_all) {   // wave-uniform: nothing to mask
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sc[r] *= c;
              mx = fmaxf(mx, sc[r]);
            }
          } else {
            const int tk = pidx * 64 + 32 * ch + 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sc[r] = tk + (r & 3) + 8 * (r >> 2) < tend ? sc[r] * c : -INFINITY;
              mx = fmaxf(mx, sc[r]);
            }
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

          // ---- online softmax (base 2, lazy reference) ----
          // rows that already hold weight and see a max above the lazy
          // threshold force a restart; the others just move their reference
          if (mx > m_run + kRescaleLog2) {
            if (m_run != -INFINITY) raise = true;
            m_run = mx;
          }
          raise = __any(raise);
          const float msub = m_run == -INFINITY ? 0.f : m_run;
          bf16x8 pf[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(sc[r] - msub);
            l_lane += pr;
            pf[r >> 3][r & 7] = static_cast<__bf16>(pr);
          }

          // ---- weighted sum O^T += V^T P^T over these 32 tokens ----
          const uint32_t pv_h0 = ch ? (pv_pg0 + 32768) : pv_pg0;
          const uint32_t pv_h1 = ch ? (pv_pg1 + 32768) : pv_pg1;
          auto vfrag = [&](int st) {
            const int mb = st >> 1, cc = st & 1;
            const uint32_t off = (mb >> 2) * 256 + cc * 16384;
            const s16x4 lo = lds_tr16a((pv_h0 ^ ((mb & 3) << 6)) + off);
            const s16x4 hi = lds_tr16a((pv_h1 ^ ((mb & 3) << 6)) + off);
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          };
          constexpr int kV = 3;   // read distance in steps
          bf16x8 vf[kV + 1];
#pragma unroll
          for (int j = 0; j < kV; ++j) vf[j] = vfrag(j);
#pragma unroll
          for (int st = 0; st < 32; ++st) {
            if (st + kV < 32) vf[(st + kV) % (kV + 1)] = vfrag(st + kV);
            o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % (kV + 1)], pf[st & 1],
                                                                   o[st >> 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (lane == 0) restart_flag[it & 1][w] = raise ? 1 : 0;
      }
    }

    // ---- epilogue: normalised partial and its log-sum-exp ----
    const float l_row = l_lane + __shfl_xor(l_lane, 32, 64);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const int64_t slot = slot_of(g, b);
    float* orow = p.o_part + (slot * p.rows + my_row) * static_cast<int64_t>(kDc);
#pragma unroll
    for (int mb = 0; mb < 16; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = f32x4{o[mb][4 * j], o[mb][4 * j + 1], o[mb][4 * j + 2], o[mb][4 * j + 3]} * inv;
        *reinterpret_cast<f32x4*>(orow + mb * 32 + 4 * half + 8 * j) = v;
      }
    if (half == 0)
      p.lse_part[slot * p.rows + my_row] =
          l_row > 0.f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

bool mfma_supports(const mla_decode_desc* d) {
  return d->d_c == kDc && d->d_rope == kDr && d->cache_dtype == MLA_BF16 &&
         d->q_dtype == MLA_BF16 && (static_cast<int64_t>(d->q_len) * d->n_heads) % kMfmaRows == 0;
}

mla_status launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  const mla_decode_desc* d = a.d;
  MfmaParams p;
  p.q_abs = static_cast<const uint16_t*>(a.q_abs);
  p.q_rope = static_cast<const uint16_t*>(a.q_rope);
  p.cache = static_cast<const uint8_t*>(a.cache);
  p.block_table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.page_start = a.page_start;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.c_log2 = a.scale * 1.4426950408889634f;
  p.B = d->batch;
  p.q_len = d->q_len;
  p.n_h = d->n_heads;
  p.max_blocks = d->max_blocks_per_seq;
  p.rows = a.p->rows;
  p.row_groups = a.p->row_groups;
  p.G = a.p->G;
  const int64_t g_pad = (a.p->G + 7) / 8 * 8;
  const dim3 grid(static_cast<unsigned>(g_pad * a.p->row_groups)), block(256);
  hipLaunchKernelGGL(decode_mfma_bf16, grid, block, 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode_mfma launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
