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

template <int OT>  // output dtype
__global__ __launch_bounds__(128) void combine_kernel(const int32_t* __restrict__ page_start,
                                                      const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      void* __restrict__ o_latent,
                                                      float* __restrict__ lse_out,
                                                      int B, int rows, int d_c, int64_t G) {
  const int64_t b = blockIdx.x / rows;
  const int r = static_cast<int>(blockIdx.x % rows);
  const int64_t P = page_start[B];
  const int64_t s0 = page_start[b], s1 = page_start[b + 1];
  const int64_t out_row = (b * rows + r) * static_cast<int64_t>(d_c);

  int64_t glo = 0, ghi = -1;
  float mx = -INFINITY;
  if (s1 > s0) {
    glo = range_of_page(s0, P, G);
    ghi = range_of_page(s1 - 1, P, G);
    for (int64_t g = glo; g <= ghi; ++g) {
      if (range_begin(g + 1, P, G) == range_begin(g, P, G)) continue;  // empty range
      mx = fmaxf(mx, lse_part[slot_of(g, b) * rows + r]);
    }
  }
  float wsum = 0.f;
  if (mx != -INFINITY)
    for (int64_t g = glo; g <= ghi; ++g) {
      if (range_begin(g + 1, P, G) == range_begin(g, P, G)) continue;
      const float l = lse_part[slot_of(g, b) * rows + r];
      if (l != -INFINITY) wsum += expf(l - mx);
    }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int k0 = threadIdx.x * 4; k0 < d_c; k0 += 512) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (mx != -INFINITY) {
      for (int64_t g = glo; g <= ghi; ++g) {
        if (range_begin(g + 1, P, G) == range_begin(g, P, G)) continue;
        const int64_t slot = slot_of(g, b);
        const float l = lse_part[slot * rows + r];
        if (l == -INFINITY) continue;
        const float wgt = expf(l - mx) * inv;
        const float4 v = *reinterpret_cast<const float4*>(o_part + (slot * rows + r) * static_cast<int64_t>(d_c) + k0);
        acc.x = fmaf(wgt, v.x, acc.x);
        acc.y = fmaf(wgt, v.y, acc.y);
        acc.z = fmaf(wgt, v.z, acc.z);
        acc.w = fmaf(wgt, v.w, acc.w);
      }
    }
    if constexpr (OT == MLA_FP32) {
      *reinterpret_cast<float4*>(static_cast<float*>(o_latent) + out_row + k0) = acc;
    } else {
      const uint32_t lo = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
      const uint32_t hi = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o_latent) + out_row + k0) = make_uint2(lo, hi);
    }
  }
  if (lse_out != nullptr && threadIdx.x == 0)
    lse_out[b * rows + r] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

}  // namespace

mla_status launch_plan(const int32_t* seq_lens, int B, int max_blocks, int32_t* page_start,
                       hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, seq_lens, B, max_blocks, page_start);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status launch_combine(const DecodeArgs& a, hipStream_t st) {
  const int B = a.d->batch, rows = a.p->rows;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * rows)), block(128);
  if (a.d->out_dtype == MLA_FP32)
    hipLaunchKernelGGL(combine_kernel<MLA_FP32>, grid, block, 0, st, a.page_start, a.o_part,
                       a.lse_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G);
  else
    hipLaunchKernelGGL(combine_kernel<MLA_BF16>, grid, block, 0, st, a.page_start, a.o_part,
                       a.lse_part, a.o_latent, a.lse_out, B, rows, a.d->d_c, a.p->G);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
