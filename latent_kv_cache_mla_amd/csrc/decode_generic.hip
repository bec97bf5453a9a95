// decode_generic.hip — split-KV absorbed-MLA decode for any supported shape
// and dtype, on the vector ALUs (no matrix cores).
//
// One wavefront owns one query row (query token m, head i) of one page range.
// Per 64-token tile: lane j computes the logit of token j,
//   s_j = scale * (q_abs . c_j + q_rope . k^R_j)
// ([LLMsBlog] "Multi-Head Latent Attention: How Low-Rank KV Compression Scales
// LLM Serving", "Query Key Absorption"), the wavefront folds the tile into a
// running max and sum (online softmax, base-2 exponentials), and then every
// lane accumulates sum_j p_j c_j for its latent lanes: values are the cached
// latent itself ([Zhang] "Multi-head latent attention", "Value absorption:
// weight and sum first, project after"). Keys and values are never formed.
//
// This kernel serves small shapes (and the fp32 cache); the DeepSeek-sized
// shapes go to the MFMA kernel.
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

struct GenericParams {
  const void* q_abs;
  const void* q_rope;
  const uint8_t* cache;
  const float* cache_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_start;
  float* o_part;
  float* lse_part;
  float scale_log2;  // softmax scale * log2(e)
  int B, q_len, n_h, d_c, d_r, max_blocks, rows, row_groups;
  int64_t G;
  int64_t row_bytes;  // bytes of one cached token row
};

constexpr int kMaxLanes = 1280;  // d_c + d_r upper bound (1024 + 256)
constexpr int kMaxAcc = 16;      // d_c / 64 upper bound

template <int CT>  // cache dtype: MLA_FP32 | MLA_BF16 | MLA_FP8_E4M3
__device__ __forceinline__ float content_elem(const uint8_t* row, int k) {
  if constexpr (CT == MLA_FP32) return reinterpret_cast<const float*>(row)[k];
  else if constexpr (CT == MLA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[k]);
  else return e4m3_to_f32(row[k]);
}

template <int CT>
__device__ __forceinline__ float rope_elem(const uint8_t* row, int d_c, int k) {
  if constexpr (CT == MLA_FP32) return reinterpret_cast<const float*>(row)[d_c + k];
  else if constexpr (CT == MLA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[d_c + k]);
  else return bf16_to_f32(reinterpret_cast<const uint16_t*>(row + d_c)[k]);
}

template <int QT>
__device__ __forceinline__ float q_elem(const void* q, int64_t i) {
  if constexpr (QT == MLA_FP32) return static_cast<const float*>(q)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
}

template <int CT, int QT>
__global__ __launch_bounds__(256) void decode_generic_kernel(GenericParams p) {
  __shared__ float q_s[4][kMaxLanes];
  __shared__ float p_s[4][64];
  __shared__ int64_t roff_s[64];
  __shared__ float sc_s[64];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t g = blockIdx.x / p.row_groups;
  const int rg = static_cast<int>(blockIdx.x % p.row_groups);
  const int r = rg * 4 + w;
  const bool active = r < p.rows;
  const int m = active ? r / p.n_h : 0, h = active ? r % p.n_h : 0;

  const int64_t P = p.page_start[p.B];
  const int64_t pb = range_begin(g, P, p.G), pe = range_begin(g + 1, P, p.G);
  if (pb >= pe) return;  // uniform over the block

  // first sequence whose pages reach past pb
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p.page_start[mid + 1] > pb) hi = mid; else lo = mid + 1;
  }

  for (int b = lo; b < p.B && p.page_start[b] < pe; ++b) {
    const int64_t s0 = p.page_start[b], s1 = p.page_start[b + 1];
    if (s1 == s0) continue;
    const int64_t a0 = s0 > pb ? s0 : pb, a1 = s1 < pe ? s1 : pe;
    const int S = clamp_len(p.seq_lens[b], p.max_blocks);
    const int tok0 = static_cast<int>((a0 - s0) * 64);
    const int tok1 = min(S, static_cast<int>((a1 - s0) * 64));
    const int tend = min(tok1, S - p.q_len + m + 1);  // this row's visible end

    if (active) {
      const int64_t qrow = (static_cast<int64_t>(b) * p.q_len + m) * p.n_h + h;
      for (int k = lane; k < p.d_c; k += 64) q_s[w][k] = q_elem<QT>(p.q_abs, qrow * p.d_c + k);
      for (int k = lane; k < p.d_r; k += 64) q_s[w][p.d_c + k] = q_elem<QT>(p.q_rope, qrow * p.d_r + k);
    }
    float acc[kMaxAcc];
#pragma unroll
    for (int i = 0; i < kMaxAcc; ++i) acc[i] = 0.f;
    float mrun = -INFINITY, lrun = 0.f;
    __syncthreads();

    for (int t = tok0; t < tok1; t += 64) {
      const int j = t + lane;
      // row offset (and fp8 scale) of token j, shared by the block
      if (w == 0) {
        int64_t off = 0;
        float sc = 1.f;
        if (j < tok1) {
          const int64_t page = p.block_table[static_cast<int64_t>(b) * p.max_blocks + (j >> 6)];
          off = (page * 64 + (j & 63)) * p.row_bytes;
          if constexpr (CT == MLA_FP8_E4M3) sc = p.cache_scale[page * 64 + (j & 63)];
        }
        roff_s[lane] = off;
        sc_s[lane] = sc;
      }
      __syncthreads();
      float s = -INFINITY;
      if (active && j < tend) {
        const uint8_t* row = p.cache + roff_s[lane];
        float dc = 0.f, dr = 0.f;
        for (int k = 0; k < p.d_c; ++k) dc = fmaf(q_s[w][k], content_elem<CT>(row, k), dc);
        for (int k = 0; k < p.d_r; ++k) dr = fmaf(q_s[w][p.d_c + k], rope_elem<CT>(row, p.d_c, k), dr);
        if constexpr (CT == MLA_FP8_E4M3) dc *= sc_s[lane];
        s = (dc + dr) * p.scale_log2;
      }
      const float tmax = wave_max(s);
      const float mnew = fmaxf(mrun, tmax);
      float pj = 0.f, alpha = 1.f;
      if (mnew != -INFINITY) {
        pj = (s == -INFINITY) ? 0.f : exp2f(s - mnew);
        alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mnew);
      }
      lrun = lrun * alpha + wave_sum(pj);
      mrun = mnew;
      if constexpr (CT == MLA_FP8_E4M3) p_s[w][lane] = pj * sc_s[lane];
      else p_s[w][lane] = pj;
      __syncthreads();
      if (active) {
#pragma unroll
        for (int i = 0; i < kMaxAcc; ++i) acc[i] *= alpha;
        const int n = min(64, tend - t);
        for (int jj = 0; jj < n; ++jj) {
          const float pw = p_s[w][jj];
          const uint8_t* row = p.cache + roff_s[jj];
#pragma unroll
          for (int i = 0; i < kMaxAcc; ++i) {
            const int k = lane + 64 * i;
            if (k < p.d_c) acc[i] = fmaf(pw, content_elem<CT>(row, k), acc[i]);
          }
        }
      }
      __syncthreads();
    }

    if (active) {
      const int64_t slot = slot_of(g, b);
      float* o = p.o_part + (slot * p.rows + r) * static_cast<int64_t>(p.d_c);
      const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
      for (int i = 0; i < kMaxAcc; ++i) {
        const int k = lane + 64 * i;
        if (k < p.d_c) o[k] = acc[i] * inv;
      }
      if (lane == 0)
        p.lse_part[slot * p.rows + r] =
            lrun > 0.f ? (mrun + log2f(lrun)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();
  }
}

}  // namespace

mla_status launch_decode_generic(const DecodeArgs& a, hipStream_t st) {
  const mla_decode_desc* d = a.d;
  GenericParams p;
  p.q_abs = a.q_abs;
  p.q_rope = a.q_rope;
  p.cache = static_cast<const uint8_t*>(a.cache);
  p.cache_scale = a.cache_scale;
  p.block_table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.page_start = a.page_start;
  p.o_part = static_cast<float*>(a.o_part);
  p.lse_part = a.lse_part;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.B = d->batch;
  p.q_len = d->q_len;
  p.n_h = d->n_heads;
  p.d_c = d->d_c;
  p.d_r = d->d_rope;
  p.max_blocks = d->max_blocks_per_seq;
  p.rows = a.p->rows;
  p.row_groups = a.p->row_groups;
  p.G = a.p->G;
  const int ct = d->cache_dtype;
  p.row_bytes = ct == MLA_FP32 ? 4LL * (d->d_c + d->d_rope)
              : ct == MLA_BF16 ? 2LL * (d->d_c + d->d_rope)
                               : static_cast<int64_t>(d->d_c) + 2LL * d->d_rope;
  const dim3 grid(static_cast<unsigned>(a.p->G * a.p->row_groups)), block(256);
  if (ct == MLA_FP32)
    hipLaunchKernelGGL((decode_generic_kernel<MLA_FP32, MLA_FP32>), grid, block, 0, st, p);
  else if (ct == MLA_BF16 && d->q_dtype == MLA_BF16)
    hipLaunchKernelGGL((decode_generic_kernel<MLA_BF16, MLA_BF16>), grid, block, 0, st, p);
  else if (ct == MLA_BF16)
    hipLaunchKernelGGL((decode_generic_kernel<MLA_BF16, MLA_FP32>), grid, block, 0, st, p);
  else if (d->q_dtype == MLA_BF16)
    hipLaunchKernelGGL((decode_generic_kernel<MLA_FP8_E4M3, MLA_BF16>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((decode_generic_kernel<MLA_FP8_E4M3, MLA_FP32>), grid, block, 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode_generic launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
