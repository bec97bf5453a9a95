// combine.hip — the split planner and the log-sum-exp combine of split-KV
// partials.
//
// A sequence's tokens may be processed in several page ranges; each range r
// leaves the softmax-normalised partial o_r = sum_{j in r} a_j c_j / sum a_j
// and its log-sum-exp lse_r. The exact result over all tokens is
//   LSE = ln sum_r exp(lse_r),   o = sum_r exp(lse_r - LSE) o_r
// — the same softmax as one pass over the whole sequence ([Zhang]
// "Multi-head latent attention", "Value absorption: weight and sum first,
// project after": the weights come from one softmax over all cached tokens).
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

// page_start[b] = sum_{b' < b} ceil(S_b' / 64) for b = 0..B (one block).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                    int max_blocks, int32_t* __restrict__ page_start) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int chunk = (B + 1023) / 1024;
  const int b0 = min(B, t * chunk), b1 = min(B, b0 + chunk);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += static_cast<int>(pages_of(clamp_len(seq_lens[b], max_blocks)));
  part[t] = local;
  __syncthreads();
  // inclusive scan (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - local;  // exclusive prefix of this chunk
  for (int b = b0; b < b1; ++b) {
    page_start[b] = run;
    run += static_cast<int>(pages_of(clamp_len(seq_lens[b], max_blocks)));
  }
  if (t == 1023) page_start[B] = part[1023];
}

// Raw 8-element partial loads (bf16 or fp32) and their conversion to fp32:
// the loads of a batch are all issued before any value is used.
template <typename PT> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 x;
  __device__ __forceinline__ void load(const uint16_t* p) { x = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { x = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void get(float* v) const {
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 x, y;
  __device__ __forceinline__ void load(const float* p) {
    x = *reinterpret_cast<const float4*>(p);
    y = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { x = y = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
};

// kWR wavefronts per output row (sequence b, row r); a block of
// max(4, kWR) wavefronts holds max(4, kWR) / kWR
// rows. The row's ranges [glo, glo + n) follow from the page prefix sums by
// the partition arithmetic. Wavefront q takes ranges q, q + kWR, ...: it
// forms the max m_q and sum s_q of exp(lse_j - m_q) over them and the sum of
// exp(lse_j - m_q) o_j (o_j divided by its row sum where the partials are
// unnormalised); lane l holds latent lanes [8 l, 8 l + 8). The log-sum-exps
// are uniform per row and read with scalar loads, so no lane exchange is
// needed; the first eight partial loads are issued before them. The
// wavefronts of a row then merge through LDS: M = max m_q,
// S = sum s_q exp(m_q - M), o = sum_q acc_q exp(m_q - M) / S.
template <typename PT, int OT, int kWR>  // partial element type, output dtype, waves per row
__global__ __launch_bounds__(64 * (kWR > 4 ? kWR : 4)) void combine_kernel(const int32_t* __restrict__ page_start,
                                                      const PT* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const float* __restrict__ l_part,
                                                      void* __restrict__ o_latent,
                                                      float* __restrict__ lse_out,
                                                      int B, int rows, int d_c, int64_t G,
                                                      int skip_whole) {
  static_assert(kWR == 1 || kWR == 2 || kWR == 4 || kWR == 8, "waves per row");
  constexpr int kWaves = kWR > 4 ? kWR : 4;   // wavefronts per block
  __shared__ float red[kWR > 1 ? kWaves : 1][kWR > 1 ? 64 * 8 : 1];   // per wavefront of the block
  __shared__ float wms[kWaves][2];                                     // (m_q, s_q) per wavefront
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int q = wv % kWR;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (kWaves / kWR) + wv / kWR;
  if (pair >= static_cast<int64_t>(B) * rows) return;   // uniform per row's wavefronts
  const int64_t b = pair / rows;
  const int r = static_cast<int>(pair % rows);
  const int64_t P = page_start[B];
  const int64_t s0 = page_start[b], s1 = page_start[b + 1];
  const int64_t out_row = pair * d_c;

  // ranges [glo, glo + n) hold the sequence's pages; with more ranges than
  // pages some ranges are empty and wrote nothing (weight 0, never read)
  int64_t glo = 0, n = 0;
  if (s1 > s0) {
    glo = range_of_page_dev(s0, P, G);
    n = range_of_page_dev(s1 - 1, P, G) - glo + 1;
  }
  // one range holds the whole sequence: the decode kernel wrote its output
  // (all wavefronts of the row leave together)
  if (skip_whole && n == 1) return;
  const bool may_be_empty = G > P;
  auto nonempty = [&](int64_t j) {
    return !may_be_empty || range_begin_dev(glo + j + 1, P, G) != range_begin_dev(glo + j, P, G);
  };
  auto idx = [&](int64_t j) { return slot_of(glo + j, b) * rows + r; };
  auto lse_of = [&](int64_t j) { return nonempty(j) ? lse_part[idx(j)] : -INFINITY; };

  // the first batch of this wavefront's partials (column block 0)
  Raw8<PT> raw[8];
  {
    const int c0 = 8 * lane;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = q + u * kWR;
      if (j < n && c0 < d_c && nonempty(j)) raw[u].load(o_part + idx(j) * d_c + c0);
      else raw[u].zero();
    }
  }
  // The log-sum-exps and row sums are uniform per row: scalar loads, eight
  // ranges at a time, all issued before any is used. The first batch's are
  // kept for its weights; a row with more ranges per wavefront reads later
  // batches' again where they are used.
  float lb0[8], rb0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t j = q + u * kWR;
    lb0[u] = j < n && nonempty(j) ? lse_part[idx(j)] : -INFINITY;
    rb0[u] = j < n && l_part != nullptr ? l_part[idx(j)] : 1.f;
  }
  float mq = -INFINITY;   // max of this wavefront's log-sum-exps
#pragma unroll
  for (int u = 0; u < 8; ++u) mq = fmaxf(mq, lb0[u]);
  for (int64_t j0 = q + 8 * kWR; j0 < n; j0 += 8 * kWR) {
    float lb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + u * kWR;
      lb[u] = j < n && nonempty(j) ? lse_part[idx(j)] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) mq = fmaxf(mq, lb[u]);
  }
  float sq = 0.f;   // sum of exp(lse_j - m_q) over this wavefront's ranges

  // the column loop is uniform across the block (barriers inside)
  for (int cb = 0; cb < d_c; cb += 512) {
    const int c0 = cb + 8 * lane;
    const bool act = c0 < d_c;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t j0 = q; j0 < n && mq != -INFINITY; j0 += 8 * kWR) {
      const bool first = j0 == q;
      if (cb > 0 || !first) {   // later batches: load now
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t j = j0 + u * kWR;
          if (j < n && act && nonempty(j)) raw[u].load(o_part + idx(j) * d_c + c0);
          else raw[u].zero();
        }
      }
      float lb[8], rb[8];
      if (first) {
#pragma unroll
        for (int u = 0; u < 8; ++u) { lb[u] = lb0[u]; rb[u] = rb0[u]; }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t j = j0 + u * kWR;
          lb[u] = j < n && nonempty(j) ? lse_part[idx(j)] : -INFINITY;
          rb[u] = j < n && l_part != nullptr ? l_part[idx(j)] : 1.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (lb[u] == -INFINITY) continue;
        const float e = expf(lb[u] - mq);
        if (cb == 0) sq += e;
        const float w = e / rb[u];
        float v[8];
        raw[u].get(v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
      }
    }
    // merge the row's wavefronts: M, S and the rescaled sums
    float M = mq, S = sq;
    if constexpr (kWR > 1) {
      __syncthreads();   // an earlier column block's sums have been read
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wv][lane * 8 + i] = acc[i];
      if (lane == 0) { wms[wv][0] = mq; wms[wv][1] = sq; }
      __syncthreads();
      if (q != 0) continue;
      M = -INFINITY;
      for (int qq = 0; qq < kWR; ++qq) M = fmaxf(M, wms[wv + qq][0]);
      if (M != -INFINITY) {
        S = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int qq = 0; qq < kWR; ++qq) {
          const float mo = wms[wv + qq][0];
          if (mo == -INFINITY) continue;
          const float f = expf(mo - M);
          S += wms[wv + qq][1] * f;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(f, red[wv + qq][lane * 8 + i], acc[i]);
        }
      }
    }
    const float inv = S > 0.f ? 1.f / S : 0.f;
    if (cb == 0 && lse_out != nullptr && lane == 0)
      lse_out[pair] = S > 0.f ? M + logf(S) : -INFINITY;
    if (!act) continue;
    if constexpr (OT == MLA_FP32) {
      float* o = static_cast<float*>(o_latent) + out_row + c0;
      *reinterpret_cast<float4*>(o) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    } else {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = f32_to_bf16(acc[2 * i] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1] * inv)) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(o_latent) + out_row + c0) =
          make_uint4(u[0], u[1], u[2], u[3]);
    }
  }
}

}  // namespace

mla_status launch_plan(const int32_t* seq_lens, int B, int max_blocks, int32_t* page_start,
                       hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, seq_lens, B, max_blocks, page_start);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

template <typename PT, int OT>
void launch_combine_t(const DecodeArgs& a, const PT* op, hipStream_t st) {
  const int B = a.d->batch, rows = a.p->rows;
  const int64_t pairs = static_cast<int64_t>(B) * rows;
  // ranges per sequence (at most): more wavefronts per row when a row has
  // more than one batch of eight, as long as the grid still fits the chip in
  // one round (about 28 resident wavefronts per CU)
  const int64_t per_seq = (a.p->G + B - 1) / B + 1;
  const int64_t resident = static_cast<int64_t>(kNumCUs) * 28;
  int wr = 1;
  if (per_seq > 32 && pairs * 8 <= resident) wr = 8;
  else if (per_seq > 16 && pairs * 4 <= resident) wr = 4;
  else if (per_seq > 8 && pairs * 2 <= resident) wr = 2;
  const dim3 block(256), grid(static_cast<unsigned>((pairs * wr + 3) / 4));
  if (wr == 8)   // one row per block of eight wavefronts
    hipLaunchKernelGGL((combine_kernel<PT, OT, 8>), dim3(static_cast<unsigned>(pairs)), dim3(512), 0, st,
                       a.page_start, op, a.lse_part, a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c,
                       a.p->G, a.skip_whole ? 1 : 0);
  else if (wr == 4)
    hipLaunchKernelGGL((combine_kernel<PT, OT, 4>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G,
                       a.skip_whole ? 1 : 0);
  else if (wr == 2)
    hipLaunchKernelGGL((combine_kernel<PT, OT, 2>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G,
                       a.skip_whole ? 1 : 0);
  else
    hipLaunchKernelGGL((combine_kernel<PT, OT, 1>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G,
                       a.skip_whole ? 1 : 0);
}

mla_status launch_combine(const DecodeArgs& a, hipStream_t st) {
  const bool bf16_out = a.d->out_dtype == MLA_BF16;
  if (a.p->part_bf16) {
    const uint16_t* op = static_cast<const uint16_t*>(a.o_part);
    if (bf16_out) launch_combine_t<uint16_t, MLA_BF16>(a, op, st);
    else launch_combine_t<uint16_t, MLA_FP32>(a, op, st);
  } else {
    const float* op = static_cast<const float*>(a.o_part);
    if (bf16_out) launch_combine_t<float, MLA_BF16>(a, op, st);
    else launch_combine_t<float, MLA_FP32>(a, op, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
