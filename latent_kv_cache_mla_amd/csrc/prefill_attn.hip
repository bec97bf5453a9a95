// prefill_attn.hip — causal attention of the unabsorbed MLA form, on the
// gfx950 matrix cores: every head attends with its expanded content key
// k^C_{j,i} = W^UK_i c_j, the shared rotated rope key k^R_j, and its expanded
// value v_{j,i} = W^UV_i c_j ([Mishra] "Multi-head Latent Attention", "Step 1:
// a low-rank latent" and "Step 4: decoupled RoPE"; [Zhang] "Multi-head latent
// attention", "Value absorption: weight and sum first, project after": scores
// (q^C . k^C + q^R . k^R) / sqrt(d_h + d_R), softmax, weighted sum of values).
// Prefill processes every position of a prompt at once, where the pages note
// the work is bound by arithmetic rather than by the cache ([LLMsBlog]
// "Multi-Head Latent Attention: How Low-Rank KV Compression Scales LLM
// Serving", opening section and "Hardware Trade-offs and Tensor
// Parallelism"); query position t sees key positions 0..t of its sequence.
//
// Workgroup = (query tile of 128 positions, head, sequence); 4 wavefronts of
// 32 query rows. Keys and values stream through a double-buffered LDS tile of
// 32 positions, shared by the four wavefronts, copied straight from global
// memory (global_load_lds_dwordx4) one tile ahead of the one multiplied.
//   * scores S^T [32 keys x 32 queries] = K Q^T with v_mfma_f32_32x32x16_bf16,
//     keys as the M dimension: A = key rows from LDS, B = the wavefront's
//     queries, held in registers for the whole pass. Each lane then holds 16
//     keys of one query row: row max and sum are in-lane plus one exchange
//     between the wavefront halves.
//   * online softmax in base 2 with a lazy reference: the running max moves
//     only when a tile's max exceeds it by more than 2^8; then O and the row
//     sum are rescaled (rare).
//   * O^T [d_v x 32 queries] += V^T P^T: P^T straight from the score
//     registers (bf16), V^T read from the row-major value tile with the LDS
//     transpose load in the key order that matches the score registers.
// The LDS layout of a tile (TileRegion below) keeps the 16-byte key-fragment
// reads and the transposed value reads free of bank conflicts.
#include <algorithm>

#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQT = 128;   // query positions per workgroup
constexpr int kKT = 32;    // key positions per LDS tile

__device__ __forceinline__ s16x4_t tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(static_cast<uintptr_t>(a)));
}

// One part of a key/value tile in LDS (content keys, rope keys or values):
// 32 rows of CP 16-byte chunks, stored as 1 KB blocks of R = 64 / CP rows,
// each filled by one direct global-to-LDS copy instruction (lane L writes
// bytes 16 L .. 16 L + 15 of the block). Within a block the chunks are
// column-major: chunk x of the block's row rr is at 16 (R x + rr). Blocks
// are 1024 + 1024 / CP bytes apart (CP >= 8), which shifts each block by a
// quarter or half of the LDS banks: the key-fragment reads (16 rows, one
// chunk) and the transposed value reads (4 rows, 4 chunks) then touch
// every bank once.
template <int CP>
struct TileRegion {
  static constexpr int R = CP > 0 ? 64 / CP : 1;   // rows per block
  static constexpr int NB = CP > 0 ? 32 / R : 0;   // blocks
  static constexpr int kStride = 1024 + (CP >= 8 ? 1024 / CP : 0);
  static constexpr int kBytes = NB * kStride;
  // byte offset of row r, chunk x
  static __device__ __forceinline__ constexpr uint32_t at(int r, int x) {
    return static_cast<uint32_t>((r / R) * kStride + 16 * (R * x + r % R));
  }
};

__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// s_waitcnt vmcnt(n), expcnt and lgkmcnt left free (gfx9 encoding)
#define PA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

template <int DC, int DR, int DV>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int DQK = DC + DR;
  static_assert(DQK % 16 == 0 && DC % 8 == 0 && DR % 8 == 0 && DV % 32 == 0, "head dims");
  constexpr int CK = DC / 8, CR = DR / 8, CV = DV / 8;   // 16-byte chunks per row part
  static_assert(CK == 16 || CK == 8, "content key width");
  static_assert(CR == 0 || CR == 2 || CR == 4 || CR == 8, "rope key width");
  static_assert(CV == 16 || CV == 8, "value width");
  using RK = TileRegion<CK>;
  using RR = TileRegion<CR>;
  using RV = TileRegion<CV>;
  constexpr uint32_t kOffR = RK::kBytes, kOffV = RK::kBytes + RR::kBytes;
  constexpr uint32_t kTileBytes = RK::kBytes + RR::kBytes + RV::kBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[2 * kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5, l32 = lane & 31;
  // heads vary fastest, then the query tile from the last (the heaviest: it
  // sees the most keys) to the first: the dispatcher starts every head's
  // heaviest tile before any lighter one, which keeps the tail of the grid
  // short (longest work first)
  const int b = blockIdx.z, head = blockIdx.x;
  const int n_qt = (a.max_seq_len + kQT - 1) / kQT;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.y);
  const int s0 = a.cu_seqlens[b], S = a.cu_seqlens[b + 1] - s0;
  const int q0 = qt * kQT;
  if (q0 >= S) return;
  const int qrow = q0 + 32 * w + l32;          // this lane's query position
  const int q_last = min(q0 + kQT, S) - 1;     // last query of the workgroup
  const int n_kt = q_last / kKT + 1;           // key tiles the workgroup needs
  const int w_last = min(q0 + 32 * w + 31, S - 1);   // this wavefront's last query

  // ---- the wavefront's queries as B fragments: fragment kc holds dims
  // 16 kc + 8 half .. + 7 of query qrow (rope dims after the content dims)
  bf16x8_t qf[DQK / 16];
  {
    const int64_t t = s0 + min(qrow, S - 1);
    const uint16_t* qc = a.q + t * a.ldq + static_cast<int64_t>(head) * DC;
    const uint16_t* qr = a.qr + t * a.ldqr + static_cast<int64_t>(head) * DR;
#pragma unroll
    for (int kc = 0; kc < DQK / 16; ++kc) {
      const int d = 16 * kc + 8 * half;
      qf[kc] = d < DC ? *reinterpret_cast<const bf16x8_t*>(qc + d)
                      : *reinterpret_cast<const bf16x8_t*>(qr + (d - DC));
    }
  }

  const uint32_t lds0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)&kv_lds[0]));

  // ---- tile copies, straight from global memory into LDS. Wavefront w
  // fills blocks w, w + 4, ... of each part; lane L of block b copies row
  // b R + L % R, chunk L / R. A lane's byte offset from the block's first
  // row is the same for every block and tile; the row pointers are scalar.
  const uint32_t gk = static_cast<uint32_t>((lane % RK::R) * a.ldk * 2 + 16 * (lane / RK::R));
  const uint32_t gr = static_cast<uint32_t>((lane % RR::R) * a.ldkr * 2 + 16 * (lane / RR::R));
  const uint32_t gv = static_cast<uint32_t>((lane % RV::R) * a.ldv * 2 + 16 * (lane / RV::R));
  auto copy_part = [&](auto region, const uint16_t* rows, int64_t ld, uint32_t lane_off,
                       uint32_t dst, int lim) {
    using RG = decltype(region);
#pragma unroll
    for (int i = 0; i < (RG::NB + 3) / 4; ++i) {
      const int blk = w + 4 * i;
      if (blk >= RG::NB) break;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(rows);
      uint32_t off;
      if (lim >= kKT - 1) {   // every row of the tile is inside the sequence
        src += static_cast<int64_t>(blk) * RG::R * ld * 2;
        off = lane_off;
      } else {                // rows past the sequence end read its last row
        const int row = min(blk * RG::R + lane % RG::R, lim);
        off = static_cast<uint32_t>(row * ld * 2 + 16 * (lane / RG::R));
      }
      asm volatile("" : "+s"(src));
      dma16(src, off, dst + blk * RG::kStride);
    }
  };
  auto issue = [&](int kt, int buf) {
    const int64_t t0 = s0 + static_cast<int64_t>(kt) * kKT;
    const int lim = S - 1 - kt * kKT;   // the tile's last row inside the sequence
    const uint32_t tb = lds0 + static_cast<uint32_t>(buf) * kTileBytes;
    copy_part(RK{}, a.k + t0 * a.ldk + static_cast<int64_t>(head) * DC, a.ldk, gk, tb, lim);
    if constexpr (CR > 0) copy_part(RR{}, a.kr + t0 * a.ldkr, a.ldkr, gr, tb + kOffR, lim);
    copy_part(RV{}, a.v + t0 * a.ldv + static_cast<int64_t>(head) * DV, a.ldv, gv, tb + kOffV, lim);
  };

  f32x16_t o[DV / 32];
#pragma unroll
  for (int mb = 0; mb < DV / 32; ++mb) o[mb] = f32x16_t{};
  float m_run = -INFINITY, l_lane = 0.f;
  const float c = a.c_log2;

  // LDS byte offsets of this lane's fragments within a tile: key fragment
  // kc is row l32, chunk 2 kc + half of its part (the chunk term is an
  // immediate offset); the transposed value reads of 16-lane group g16 take
  // row 4 (g16 >> 1) + (s16 >> 2) (+8 for the upper four keys, +16 for the
  // second 16-key step) and dims 16 (g16 & 1) + 4 (s16 & 3) .. + 3 of the
  // 32-dim block mb
  const uint32_t kc_off = RK::at(l32, half);
  const uint32_t kr_off = kOffR + RR::at(l32, half);
  const int g16 = lane >> 4, s16 = lane & 15;
  const uint32_t v_off = kOffV + RV::at(4 * (g16 >> 1) + (s16 >> 2), 2 * (g16 & 1) + ((s16 & 3) >> 1)) + 8 * (s16 & 1);
  // offset of rows r0 + dr from row r0 (r0 < 8, dr a multiple of 8)
  auto vrow = [](int dr) { return static_cast<uint32_t>((dr / RV::R) * RV::kStride + 16 * (dr % RV::R)); };

  issue(0, 0);
  PA_WAIT_VM(0);
  __syncthreads();
  // tiles from n_vis on start after the wavefront's last query: fully
  // masked, the wavefront only takes part in their copies and barriers (two
  // loops rather than a test in one, so that O stays in the same registers);
  // a wavefront whose rows all lie past the sequence end computes none
  const int n_vis = q0 + 32 * w >= S ? 0 : min(n_kt, w_last / kKT + 1);
  int kt = 0;
  for (; kt < n_vis; ++kt) {
    const int buf = kt & 1;
    // tile kt + 1 goes into the other buffer, which every wavefront finished
    // reading before the barrier that ended the previous step
    if (kt + 1 < n_kt) issue(kt + 1, buf ^ 1);
    {
      const uint32_t tb = lds0 + static_cast<uint32_t>(buf) * kTileBytes;
      // every key fragment of the tile is read before the first product (the
      // scheduling barrier keeps the compiler from interleaving the reads
      // with the products, which would expose the LDS latency at each pair)
      bf16x8_t kf[DQK / 16];
#pragma unroll
      for (int kc = 0; kc < DQK / 16; ++kc) {
        const uint32_t ad = kc < DC / 16 ? tb + kc_off + 32 * RK::R * kc : tb + kr_off + 32 * RR::R * (kc - DC / 16);
        kf[kc] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(static_cast<uintptr_t>(ad));
      }
      __builtin_amdgcn_sched_barrier(0);
      // the score products at raised wavefront priority: the other wavefront
      // on the SIMD (another workgroup's) runs its softmax on the vector unit
      // meanwhile
      __builtin_amdgcn_s_setprio(1);
      f32x16_t s = f32x16_t{};
#pragma unroll
      for (int kc = 0; kc < DQK / 16; ++kc) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc], qf[kc], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // register r holds key kt * 32 + 8 (r / 4) + 4 half + r % 4 of query
      // qrow; only a tile that reaches past the wavefront's first query or the
      // sequence end needs the mask (a wave-uniform test)
      if (kt * kKT + kKT - 1 > q0 + 32 * w || kt * kKT + kKT > S) {
        const int kbase = kt * kKT + 4 * half;
        const int lim = min(qrow + 1, S);   // visible keys: key < lim
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[r] = kbase + 8 * (r >> 2) + (r & 3) < lim ? s[r] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2)   // scores are finite or -inf: no NaN handling needed
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(s[r]), "v"(s[r + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
      if (mx > m_run + 8.0f) {   // lazy reference: rescale only on a large rise
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
#pragma unroll
        for (int mb = 0; mb < DV / 32; ++mb) o[mb] *= alpha;
        l_lane *= alpha;
        m_run = mx;
      }
      // weights in bf16 pairs; the row sum is taken over the bf16 weights the
      // products use (a dot product of each pair with (1, 1))
      bf16x8_t pf[2];
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const bf16x2_t two = {static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[r], c, -m_run))),
                              static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -m_run)))};
        pf[r >> 3][r & 7] = two[0];
        pf[r >> 3][(r & 7) + 1] = two[1];
        l_lane = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_lane, false);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mb = 0; mb < DV / 32; ++mb) {
          const uint32_t va = tb + v_off + vrow(16 * kk) + 64 * RV::R * mb;
          const s16x4_t lo = tr16(va);
          const s16x4_t hi = tr16(va + vrow(8));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], o[mb], 0, 0, 0);
        }
      }
    }
    // this wavefront's copies of tile kt + 1 have landed; after the barrier
    // every wavefront's have
    PA_WAIT_VM(0);
    __syncthreads();
  }
  for (; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) issue(kt + 1, (kt & 1) ^ 1);
    PA_WAIT_VM(0);
    __syncthreads();
  }

  // ---- epilogue: O / l as bf16; register r of o[mb] is dim
  // 32 mb + 8 (r / 4) + 4 half + r % 4 of query qrow
  const float l_row = l_lane + __shfl_xor(l_lane, 32, 64);
  if (qrow < S) {
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    uint16_t* orow = a.o + (s0 + static_cast<int64_t>(qrow)) * a.ldo + static_cast<int64_t>(head) * DV;
#pragma unroll
    for (int mb = 0; mb < DV / 32; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u0 = f32_to_bf16(o[mb][4 * j] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[mb][4 * j + 1] * inv)) << 16);
        const uint32_t u1 = f32_to_bf16(o[mb][4 * j + 2] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[mb][4 * j + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * j + 4 * half) = make_uint2(u0, u1);
      }
    if (a.lse != nullptr && half == 0)
      a.lse[static_cast<int64_t>(head) * a.T + s0 + qrow] =
          l_row > 0.f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

bool prefill_attn_supported(int d_h, int d_rope, int d_v) {
  return (d_h == 128 && d_rope == 64 && d_v == 128) || (d_h == 64 && d_rope == 16 && d_v == 64) ||
         (d_h == 64 && d_rope == 32 && d_v == 64) || (d_h == 128 && d_rope == 0 && d_v == 128);
}

mla_status launch_prefill_attn(const PrefillAttnArgs& a, int d_h, int d_rope, int d_v, hipStream_t st) {
  // the per-lane byte offsets of a tile's rows are 32-bit
  const int64_t ld_max = std::max(a.ldk, std::max(a.ldkr, a.ldv));
  if (ld_max < 0 || ld_max * 2 * kKT >= (int64_t{1} << 31))
    return fail(MLA_ERR_UNSUPPORTED, "prefill attention: key/value row stride %lld too large",
                static_cast<long long>(ld_max));
  const dim3 grid(static_cast<unsigned>(a.n_heads), static_cast<unsigned>((a.max_seq_len + kQT - 1) / kQT),
                  static_cast<unsigned>(a.batch));
  if (d_h == 128 && d_rope == 64 && d_v == 128)
    hipLaunchKernelGGL((prefill_attn_kernel<128, 64, 128>), grid, dim3(256), 0, st, a);
  else if (d_h == 64 && d_rope == 16 && d_v == 64)
    hipLaunchKernelGGL((prefill_attn_kernel<64, 16, 64>), grid, dim3(256), 0, st, a);
  else if (d_h == 64 && d_rope == 32 && d_v == 64)
    hipLaunchKernelGGL((prefill_attn_kernel<64, 32, 64>), grid, dim3(256), 0, st, a);
  else if (d_h == 128 && d_rope == 0 && d_v == 128)
    hipLaunchKernelGGL((prefill_attn_kernel<128, 0, 128>), grid, dim3(256), 0, st, a);
  else
    return fail(MLA_ERR_UNSUPPORTED, "prefill attention is built for (d_h, d_R) in "
                "{(128, 64), (64, 16), (64, 32), (128, 0)}, got (%d, %d)", d_h, d_rope);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill attention launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
