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

// 8 consecutive partial elements of one row, as fp32
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 4);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// kWR wavefronts per output row (sequence b, row r); with kWR = 1 a block
// holds four rows. Lane j of every wavefront loads the log-sum-exp of range j
// of the row's ranges (64 at a time) and forms its weight exp(lse_j - LSE),
// divided by the partial's softmax row sum where the partials are
// unnormalised (l_part non-null);
// wavefront q then combines 8 consecutive latent lanes per lane over ranges
// q, q + kWR, ..., with eight partial loads in flight, and the kWR partial
// sums are added through LDS. Several wavefronts per row serve sequences cut
// into many ranges (long contexts with a small batch).
template <typename PT, int OT, int kWR>  // partial element type, output dtype, waves per row
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ page_start,
                                                      const PT* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const float* __restrict__ l_part,
                                                      void* __restrict__ o_latent,
                                                      float* __restrict__ lse_out,
                                                      int B, int rows, int d_c, int64_t G) {
  static_assert(kWR == 1 || kWR == 2 || kWR == 4, "waves per row");
  __shared__ float red[kWR > 1 ? 4 : 1][kWR > 1 ? 64 * 8 : 1];   // per wavefront of the block
  const int lane = threadIdx.x & 63;
  const int wv = static_cast<int>(threadIdx.x >> 6);
  const int q = wv % kWR;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (4 / kWR) + (threadIdx.x >> 6) / kWR;
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
    glo = range_of_page(s0, P, G);
    n = range_of_page(s1 - 1, P, G) - glo + 1;
  }
  const bool may_be_empty = G > P;
  auto lse_of = [&](int64_t j) {
    const int64_t g = glo + j;
    if (may_be_empty && range_begin(g + 1, P, G) == range_begin(g, P, G)) return -INFINITY;
    return lse_part[slot_of(g, b) * rows + r];
  };
  // 1 / row sum of range j's partial when the partials are unnormalised
  auto rl_of = [&](int64_t j) {
    return l_part != nullptr ? 1.f / l_part[slot_of(glo + j, b) * rows + r] : 1.f;
  };
  // lane j holds the log-sum-exp of range j (up to 64 ranges in registers;
  // rows with more ranges reload them per block of 64)
  float l0 = n > 0 && lane < n ? lse_of(lane) : -INFINITY;
  float mx = l0;
  for (int64_t j = lane + 64; j < n; j += 64) mx = fmaxf(mx, lse_of(j));
  mx = wave_max(mx);
  float wsum = 0.f;
  if (mx != -INFINITY) {
    wsum = l0 == -INFINITY ? 0.f : expf(l0 - mx);
    for (int64_t j = lane + 64; j < n; j += 64) {
      const float l = lse_of(j);
      if (l != -INFINITY) wsum += expf(l - mx);
    }
  }
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  // the column loop is uniform across the block (barriers inside)
  for (int cb = 0; cb < d_c; cb += 512) {
    const int c0 = cb + 8 * lane;
    const bool act = c0 < d_c;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t j0 = 0; j0 < n && mx != -INFINITY; j0 += 64) {
      float lj = l0;
      if (j0 > 0) lj = j0 + lane < n ? lse_of(j0 + lane) : -INFINITY;
      const float wj = lj == -INFINITY ? 0.f : expf(lj - mx) * inv * rl_of(j0 + lane);
      const int cnt = static_cast<int>(n - j0 < 64 ? n - j0 : 64);
      for (int j = q; j < cnt; j += 8 * kWR) {
        float wgt[8], v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int jj = j + u * kWR;
          wgt[u] = jj < cnt ? __shfl(wj, jj, 64) : 0.f;   // uniform
          if (wgt[u] != 0.f && act)
            load8(o_part + (slot_of(glo + j0 + jj, b) * rows + r) * static_cast<int64_t>(d_c) + c0, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (wgt[u] != 0.f && act)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wgt[u], v[u][i], acc[i]);
      }
    }
    if constexpr (kWR > 1) {
      __syncthreads();   // an earlier column block's sums have been read
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wv][lane * 8 + i] = acc[i];
      __syncthreads();
      if (q != 0) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        for (int qq = 1; qq < kWR; ++qq) acc[i] += red[wv + qq][lane * 8 + i];
    }
    if (!act) continue;
    if constexpr (OT == MLA_FP32) {
      float* o = static_cast<float*>(o_latent) + out_row + c0;
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = f32_to_bf16(acc[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(o_latent) + out_row + c0) =
          make_uint4(u[0], u[1], u[2], u[3]);
    }
  }
  if (lse_out != nullptr && lane == 0 && q == 0)
    lse_out[pair] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
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
  // ranges per sequence on average: more wavefronts per row when there are many
  const int64_t per_seq = (a.p->G + B - 1) / B + 1;
  const int wr = per_seq > 16 ? 4 : per_seq > 8 ? 2 : 1;
  const dim3 block(256), grid(static_cast<unsigned>((pairs * wr + 3) / 4));
  if (wr == 4)
    hipLaunchKernelGGL((combine_kernel<PT, OT, 4>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G);
  else if (wr == 2)
    hipLaunchKernelGGL((combine_kernel<PT, OT, 2>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G);
  else
    hipLaunchKernelGGL((combine_kernel<PT, OT, 1>), grid, block, 0, st, a.page_start, op, a.lse_part,
                       a.l_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G);
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
