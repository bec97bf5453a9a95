// gemm.hip — the dense projections around the decode step, and the kernels
// that finish them:
//   * offline folds W^UK_i^T W^UQ_i and W^O_i W^UV_i ([Mishra] "Multi-head
//     Latent Attention", "Step 2: absorb the up-projections");
//   * the latent-to-model output projection, merged or as two factors
//     ([Zhang] "Multi-head latent attention", "Value absorption: weight and
//     sum first, project after");
//   * the cache write for new tokens: c_t = W^DKV h_t ([Mishra] "Step 1: a
//     low-rank latent") and k^R_t = RoPE(W^KR h_t) stored rotated ([Zhang]
//     "Decoupled RoPE: content and position in separate branches"), with the
//     optional fp8 e4m3 per-token quantisation;
//   * the absorbed query projection ([LLMsBlog] "Multi-Head Latent Attention:
//     How Low-Rank KV Compression Scales LLM Serving", "Query Key Absorption").
// All are fp32 with fp32 accumulation through one LDS-tiled strided batched
// GEMM: these are offline or per-step projections off the attention loop.
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

constexpr int kT = 64;   // output tile edge
constexpr int kK = 16;   // k step

__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ float As[kK][kT + 4];
  __shared__ float Bs[kK][kT + 4];
  const int64_t bz = blockIdx.z;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  const float* Af = static_cast<const float*>(g.A);
  const uint16_t* Ah = static_cast<const uint16_t*>(g.A);
  for (int k0 = 0; k0 < g.K; k0 += kK) {
    for (int idx = threadIdx.x; idx < kK * kT; idx += 256) {
      const int kk = idx / kT, mm = idx % kT;
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < g.M && k < g.K) {
        const int64_t off = bz * g.sAb + m * g.sAm + k * g.sAk;
        v = g.a_bf16 ? bf16_to_f32(Ah[off]) : Af[off];
      }
      As[kk][mm] = v;
    }
    for (int idx = threadIdx.x; idx < kK * kT; idx += 256) {
      const int kk = idx / kT, nn = idx % kT;
      const int n = n0 + nn, k = k0 + kk;
      Bs[kk][nn] = (n < g.N && k < g.K) ? g.B[bz * g.sBb + k * g.sBk + n * g.sBn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < g.N) g.Y[bz * g.sYb + m * g.sYm + n * g.sYn] = acc[i][j];
    }
  }
}

// OCP e4m3fn encoding of a finite fp32 value, round to nearest even,
// saturating to +-448 (written from the format: bias 7, 3 mantissa bits,
// subnormal step 2^-9).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (!(a == a)) return 0x7Fu;                // NaN
  if (a >= 448.f) code = 0x7Eu;
  else if (a < 0.015625f) {                   // below 2^-6: subnormal grid 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.f));   // 8 rounds up to the first normal
  } else {
    const int E = static_cast<int>((__float_as_uint(a) >> 23) & 0xFF) - 127;   // -6..8
    float q = rintf(ldexpf(a, 3 - E));        // in [8, 16]
    int e = E;
    if (q >= 16.f) { q = 8.f; ++e; }
    code = (static_cast<uint32_t>(e + 7) << 3) | (static_cast<uint32_t>(q) - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// One block per new token: rotate the rope part, quantise (fp8), scatter.
// cr row t = [c (d_c) | unrotated k (d_r)] fp32.
template <int CT>
__global__ __launch_bounds__(256) void append_finish_kernel(const float* __restrict__ cr, int d_c,
                                                            int d_r, double theta,
                                                            const int32_t* __restrict__ positions,
                                                            const int32_t* __restrict__ slots,
                                                            void* __restrict__ cache,
                                                            float* __restrict__ cache_scale) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const float* row = cr + t * (d_c + d_r);
  const int pos = positions[t];
  __shared__ float red[256];
  float scale = 1.f;
  if constexpr (CT == MLA_FP8_E4M3) {
    float mx = 0.f;
    for (int k = threadIdx.x; k < d_c; k += 256) mx = fmaxf(mx, fabsf(row[k]));
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
      __syncthreads();
    }
    const float amax = red[0];
    scale = amax == 0.f ? 1.f : amax / 448.f;
    if (threadIdx.x == 0) cache_scale[slot] = scale;
  }
  // content lanes
  for (int k = threadIdx.x; k < d_c; k += 256) {
    const float v = row[k];
    if constexpr (CT == MLA_FP32) static_cast<float*>(cache)[slot * (d_c + d_r) + k] = v;
    else if constexpr (CT == MLA_BF16) static_cast<uint16_t*>(cache)[slot * (d_c + d_r) + k] = f32_to_bf16(v);
    else static_cast<uint8_t*>(cache)[slot * (d_c + 2 * d_r) + k] = static_cast<uint8_t>(f32_to_e4m3(v / scale));
  }
  // rope lanes: interleaved pairs (2k, 2k+1)
  for (int k = threadIdx.x; k < d_r / 2; k += 256) {
    float c, s;
    rope_cs(pos, k, d_r, theta, &c, &s);
    const float x0 = row[d_c + 2 * k], x1 = row[d_c + 2 * k + 1];
    const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    if constexpr (CT == MLA_FP32) {
      float* dst = static_cast<float*>(cache) + slot * (d_c + d_r) + d_c;
      dst[2 * k] = y0;
      dst[2 * k + 1] = y1;
    } else if constexpr (CT == MLA_BF16) {
      uint16_t* dst = static_cast<uint16_t*>(cache) + slot * (d_c + d_r) + d_c;
      dst[2 * k] = f32_to_bf16(y0);
      dst[2 * k + 1] = f32_to_bf16(y1);
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(cache) + slot * (d_c + 2 * d_r) + d_c);
      dst[2 * k] = f32_to_bf16(y0);
      dst[2 * k + 1] = f32_to_bf16(y1);
    }
  }
}

// One block per query token: rotate q^R per head, convert both outputs.
template <int QT>
__global__ __launch_bounds__(256) void query_finish_kernel(const float* __restrict__ qa32,
                                                           const float* __restrict__ qr32, int n_h,
                                                           int d_c, int d_r, double theta,
                                                           const int32_t* __restrict__ positions,
                                                           void* __restrict__ q_abs,
                                                           void* __restrict__ q_rope) {
  const int64_t t = blockIdx.x;
  const int pos = positions[t];
  const int64_t na = static_cast<int64_t>(n_h) * d_c;
  for (int64_t i = threadIdx.x; i < na; i += 256) {
    const float v = qa32[t * na + i];
    if constexpr (QT == MLA_FP32) static_cast<float*>(q_abs)[t * na + i] = v;
    else static_cast<uint16_t*>(q_abs)[t * na + i] = f32_to_bf16(v);
  }
  const int half = d_r / 2;
  for (int i = threadIdx.x; i < n_h * half; i += 256) {
    const int h = i / half, k = i % half;
    float c, s;
    rope_cs(pos, k, d_r, theta, &c, &s);
    const int64_t base = (t * n_h + h) * d_r;
    const float x0 = qr32[base + 2 * k], x1 = qr32[base + 2 * k + 1];
    const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    if constexpr (QT == MLA_FP32) {
      static_cast<float*>(q_rope)[base + 2 * k] = y0;
      static_cast<float*>(q_rope)[base + 2 * k + 1] = y1;
    } else {
      static_cast<uint16_t*>(q_rope)[base + 2 * k] = f32_to_bf16(y0);
      static_cast<uint16_t*>(q_rope)[base + 2 * k + 1] = f32_to_bf16(y1);
    }
  }
}

}  // namespace

mla_status launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return MLA_OK;
  const dim3 grid((g.N + kT - 1) / kT, (g.M + kT - 1) / kT, g.batch);
  if (grid.y > 65535u || grid.z > 65535u) return fail(MLA_ERR_UNSUPPORTED, "gemm too large");
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, st, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status launch_append_finish(const float* cr, int T, int d_c, int d_rope, float theta,
                                const int32_t* positions, const int32_t* slots,
                                int cache_dtype, void* cache, float* cache_scale,
                                hipStream_t st) {
  if (T <= 0) return MLA_OK;
  const double th = theta;
  if (cache_dtype == MLA_FP32)
    hipLaunchKernelGGL(append_finish_kernel<MLA_FP32>, dim3(T), dim3(256), 0, st, cr, d_c, d_rope,
                       th, positions, slots, cache, cache_scale);
  else if (cache_dtype == MLA_BF16)
    hipLaunchKernelGGL(append_finish_kernel<MLA_BF16>, dim3(T), dim3(256), 0, st, cr, d_c, d_rope,
                       th, positions, slots, cache, cache_scale);
  else
    hipLaunchKernelGGL(append_finish_kernel<MLA_FP8_E4M3>, dim3(T), dim3(256), 0, st, cr, d_c,
                       d_rope, th, positions, slots, cache, cache_scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status launch_query_finish(const float* q_abs32, const float* q_rope32, int T, int n_h,
                               int d_c, int d_rope, float theta, const int32_t* positions,
                               int q_dtype, void* q_abs, void* q_rope, hipStream_t st) {
  if (T <= 0) return MLA_OK;
  const double th = theta;
  if (q_dtype == MLA_FP32)
    hipLaunchKernelGGL(query_finish_kernel<MLA_FP32>, dim3(T), dim3(256), 0, st, q_abs32, q_rope32,
                       n_h, d_c, d_rope, th, positions, q_abs, q_rope);
  else
    hipLaunchKernelGGL(query_finish_kernel<MLA_BF16>, dim3(T), dim3(256), 0, st, q_abs32, q_rope32,
                       n_h, d_c, d_rope, th, positions, q_abs, q_rope);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "query finish launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
