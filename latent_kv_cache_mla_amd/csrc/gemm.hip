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
#include <type_traits>

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

// Block (token t, slice y of gridDim.y): convert a slice of q_abs, and rotate
// q^R of the heads of the slice. The rotation of pair k depends only on the
// token's position, so its cosine and sine are computed once per block (the
// first d_r / 2 threads, fp64) and shared through LDS. The source row of
// token t is q32 + t ld: n_h d_c values of q_abs, then n_h d_r of q_rope,
// summed over `splits` copies split_stride apart (the split sums of the
// projection, in split order).
template <int QT>
__global__ __launch_bounds__(256) void query_finish_kernel(const float* __restrict__ q32, int64_t ld,
                                                           int splits, int64_t split_stride, int n_h,
                                                           int d_c, int d_r, double theta,
                                                           const int32_t* __restrict__ positions,
                                                           void* __restrict__ q_abs,
                                                           void* __restrict__ q_rope) {
  __shared__ float cs_lds[2][128];
  const int64_t t = blockIdx.x;
  const int pos = positions[t];
  const int half = d_r / 2;
  for (int k = threadIdx.x; k < half; k += 256) rope_cs(pos, k, d_r, theta, &cs_lds[0][k], &cs_lds[1][k]);
  __syncthreads();
  const float* row = q32 + t * ld;
  auto src = [&](int64_t i) {
    float v = row[i];
    for (int z = 1; z < splits; ++z) v += row[z * split_stride + i];
    return v;
  };
  const int64_t na = static_cast<int64_t>(n_h) * d_c;
  const int64_t per = (na + gridDim.y - 1) / gridDim.y;
  const int64_t i0 = blockIdx.y * per, i1 = min(na, i0 + per);
  // 4 values per thread where rows, slices and split copies are 16-byte
  // aligned (all loads of a thread issued before they are summed)
  const uintptr_t out_al = QT == MLA_FP32 ? 15u : 7u;
  const bool vec = ((reinterpret_cast<uintptr_t>(q32) | (ld * 4) | (split_stride * 4) | (per * 4)) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(q_abs) & out_al) == 0 && na % 4 == 0 && (i1 - i0) % 4 == 0;
  if (vec) {
    typedef float f32x4q __attribute__((ext_vector_type(4)));
    for (int64_t i = i0 + 4 * threadIdx.x; i < i1; i += 4 * 256) {
      f32x4q v = *reinterpret_cast<const f32x4q*>(row + i);
      for (int z = 1; z < splits; ++z) v += *reinterpret_cast<const f32x4q*>(row + z * split_stride + i);
      if constexpr (QT == MLA_FP32) {
        *reinterpret_cast<f32x4q*>(static_cast<float*>(q_abs) + t * na + i) = v;
      } else {
        const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(q_abs) + t * na + i) = make_uint2(lo, hi);
      }
    }
  } else {
    for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) {
      const float v = src(i);
      if constexpr (QT == MLA_FP32) static_cast<float*>(q_abs)[t * na + i] = v;
      else static_cast<uint16_t*>(q_abs)[t * na + i] = f32_to_bf16(v);
    }
  }
  const int hp = (n_h + gridDim.y - 1) / gridDim.y;
  const int h0 = blockIdx.y * hp, h1 = min(n_h, h0 + hp);
  for (int i = threadIdx.x; i < (h1 - h0) * half; i += 256) {
    const int h = h0 + i / half, k = i % half;
    const float c = cs_lds[0][k], s = cs_lds[1][k];
    const int64_t base = (t * n_h + h) * d_r;
    const int64_t sb = na + static_cast<int64_t>(h) * d_r;
    const float x0 = src(sb + 2 * k), x1 = src(sb + 2 * k + 1);
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

// ---- the per-step projections: few rows (decode tokens), weights streamed once
//
// Y[b][m][n] = sum_k A[b](m, k) W[b](n, k) with A and W contiguous along k
// (activations [T, K], a weight stored [out, in]). fp32 products on the
// matrix cores (v_mfma_f32_32x32x2_f32: exact fp32 multiplies, fp32
// accumulation), so the result keeps the precision of the fp32 weights.
// Workgroup = 32 rows x 128 outputs (4 wavefronts x 32 outputs) over one
// split of K; A and W tiles of 32 k go through double-buffered LDS with rows
// padded to 36 words. Each weight element is read from memory once per row
// block; split-K (fp32 partial tiles, summed in split order) gives the
// skinny shapes enough workgroups to stream the weights at full bandwidth.
//
// Within a 32-k stage the MFMA k index is permuted: MFMA kk (0..15) takes k
// = kk from lanes 0..31 and k = 16 + kk from lanes 32..63, so a lane's 16
// values of a stage are contiguous (four 16-byte LDS reads per operand
// instead of sixteen 4-byte ones); A and W use the same order, so the sums
// are those of the plain order, term for term.
typedef float f32x16g __attribute__((ext_vector_type(16)));
typedef float f32x4g __attribute__((ext_vector_type(4)));
constexpr int kSM = 32, kSN = 128, kSK = 32, kSP = kSK + 4;

// A_BF16: activations in bf16. A_VEC: activation rows are 4-element aligned
// (16 bytes for fp32, 8 for bf16) with a row stride that is a multiple of 4,
// so a thread's 4 consecutive k load as one vector.
template <int A_BF16, int A_VEC>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(GemmArgs g, int splits, int k_per_split,
                                                          float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float As[2][kSM * kSP];
  __shared__ __attribute__((aligned(16))) float Ws[2][kSN * kSP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kSN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kSM;
  const int bz = blockIdx.z / splits, z = blockIdx.z % splits;
  const int kb = z * k_per_split, ke = min(g.K, kb + k_per_split);
  // thread tid stages A row tid / 8 and W rows tid / 8 + 32 j (j < 4), k
  // 4 (tid % 8) .. + 3 of a stage; rows past M or N read the last row (their
  // outputs are never stored). W offsets are 32-bit byte offsets from the
  // batch's weight base (the host checks they fit).
  const int r8 = tid >> 3, k4 = (tid & 7) * 4;
  const int64_t am = min(m0 + r8, static_cast<int64_t>(g.M) - 1);
  const float* Af = static_cast<const float*>(g.A) + bz * g.sAb + am * g.sAm;
  const uint16_t* Ah = static_cast<const uint16_t*>(g.A) + bz * g.sAb + am * g.sAm;
  // the workgroup's weight matrix: B, or B2 for the columns from N1 on (N1
  // is a multiple of 128, so a workgroup never straddles the two)
  const bool second = g.B2 != nullptr && n0 >= g.N1;
  const float* Wb = second ? g.B2 : g.B + bz * g.sBb;
  const int64_t wn0 = second ? n0 - g.N1 : n0;
  const int64_t wrows = g.B2 == nullptr ? g.N : (second ? g.N - g.N1 : g.N1);
  uint32_t woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = min(wn0 + r8 + 32 * j, wrows - 1);
    woff[j] = static_cast<uint32_t>(n * g.sBn * 4);
  }
  // two register sets: the loads of stage s + 2 are issued before stage s is
  // multiplied, so each stage's loads have two stages of MFMAs to arrive.
  // Every stage runs the same code (no branch around loads, so the loads'
  // registers need no waits beyond their own): a stage at or past the
  // split's last one re-reads that last stage (cached), and A values at k
  // past ke are 0, which zeroes their products (the weights read there are
  // finite: K is a multiple of 4, so no 4-element chunk reaches past a row's
  // K values into its padding).
  const int klast = kb + ((ke - kb - 1) / kSK) * kSK;   // the split's last stage
  f32x4g ra[2], rw[2][4];
  auto gload = [&](auto SET, int k0) {
    constexpr int set = decltype(SET)::value;
    // this thread's 4-element chunk, kept inside the rows' K values
    const int kl = min(min(k0, klast) + k4, g.K - 4);
    f32x4g a;
    if constexpr (A_VEC) {
      if constexpr (A_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(Ah + kl);
        a = f32x4g{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
      } else {
        a = *reinterpret_cast<const f32x4g*>(Af + kl);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = A_BF16 ? bf16_to_f32(Ah[kl + i]) : Af[kl + i];
    }
    ra[set] = a;
    const uint8_t* wk = reinterpret_cast<const uint8_t*>(Wb + kl);
#pragma unroll
    for (int j = 0; j < 4; ++j) rw[set][j] = *reinterpret_cast<const f32x4g*>(wk + woff[j]);
  };
  // (the zeroing waits for the loads, so it is done here, where the stage's
  // values are needed anyway)
  auto swrite = [&](auto SET, int buf, int k0) {
    constexpr int set = decltype(SET)::value;
    f32x4g a = ra[set];
    if (k0 + kSK > ke) {   // a partial or past-the-end stage (wave-uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = k0 + k4 + i < ke ? a[i] : 0.f;
    }
    *reinterpret_cast<f32x4g*>(&As[buf][r8 * kSP + k4]) = a;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4g*>(&Ws[buf][(r8 + 32 * j) * kSP + k4]) = rw[set][j];
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  f32x16g acc = f32x16g{};
  if (kb < ke) {   // (uniform over the workgroup)
    gload(S0{}, kb);
    gload(S1{}, kb + kSK);
    swrite(S0{}, 0, kb);
    __syncthreads();
    // stage at k0 sits in LDS buffer buf; its successor in register set
    // 1 - SET (SET alternates with the stage, at compile time through the
    // unrolled pair)
    auto stage = [&](auto SET, int k0, int buf) {
      constexpr int set = decltype(SET)::value;
      gload(std::integral_constant<int, set>{}, k0 + 2 * kSK);
      f32x4g av[4], wv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = *reinterpret_cast<const f32x4g*>(&As[buf][l32 * kSP + 16 * half + 4 * q]);
        wv[q] = *reinterpret_cast<const f32x4g*>(&Ws[buf][(32 * w + l32) * kSP + 16 * half + 4 * q]);
      }
#pragma unroll
      for (int kk = 0; kk < kSK / 2; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk >> 2][kk & 3], wv[kk >> 2][kk & 3], acc, 0, 0, 0);
      swrite(std::integral_constant<int, 1 - set>{}, buf ^ 1, k0 + kSK);
      __syncthreads();
    };
    // stages in pairs: an odd count runs one all-zero stage more
    for (int k0 = kb; k0 < ke; k0 += 2 * kSK) {
      stage(S0{}, k0, 0);
      stage(S1{}, k0 + kSK, 1);
    }
  }
  // register r: row m0 + 8 (r / 4) + 4 half + r % 4, output n0 + 32 w + l32
  const int64_t n = n0 + 32 * w + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t m = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (m >= g.M || n >= g.N) continue;
    if (splits > 1)
      partial[((static_cast<int64_t>(z) * g.batch + bz) * g.M + m) * g.N + n] = acc[r];
    else
      g.Y[bz * g.sYb + m * g.sYm + n * g.sYn] = acc[r];
  }
}

__global__ __launch_bounds__(256) void skinny_reduce_kernel(GemmArgs g, int splits,
                                                            const float* __restrict__ partial) {
  const int64_t per = static_cast<int64_t>(g.M) * g.N, total = per * g.batch;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < total; e += static_cast<int64_t>(gridDim.x) * 256) {
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += partial[z * total + e];
    const int64_t b = e / per, m = (e % per) / g.N, n = e % g.N;
    g.Y[b * g.sYb + m * g.sYm + n * g.sYn] = s;
  }
}

// The split sums for outputs whose rows are contiguous, 16-byte aligned and
// a multiple of 4 long: workgroup (x, row) sums 4 consecutive outputs per
// thread over the splits, in split order (the same order as above).
__global__ __launch_bounds__(256) void skinny_reduce4_kernel(GemmArgs g, int splits,
                                                             const float* __restrict__ partial) {
  typedef float f32x4r __attribute__((ext_vector_type(4)));
  const int row = blockIdx.y;   // b * M + m
  const int64_t n = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (n >= g.N) return;
  const int64_t total = static_cast<int64_t>(g.M) * g.N * g.batch;
  const float* p = partial + static_cast<int64_t>(row) * g.N + n;
  f32x4r s = *reinterpret_cast<const f32x4r*>(p);
  // eight splits' loads in flight at a time, added in split order
  for (int z0 = 1; z0 < splits; z0 += 8) {
    f32x4r v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) v[u] = *reinterpret_cast<const f32x4r*>(p + (z0 + u) * total);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) s += v[u];
  }
  const int b = row / g.M, m = row % g.M;
  *reinterpret_cast<f32x4r*>(g.Y + b * g.sYb + m * g.sYm + n) = s;
}

}  // namespace

bool skinny_ok(const GemmArgs& g) {
  // (a weight batch's row offsets are 32-bit byte offsets)
  const bool b2 = g.B2 == nullptr ||
                  (g.batch == 1 && g.N1 > 0 && g.N1 % kSN == 0 && g.N1 < g.N && aligned16(g.B2));
  return b2 && g.sAk == 1 && g.sBk == 1 && g.K % 4 == 0 && g.sBn % 4 == 0 && g.sBb % 4 == 0 &&
         aligned16(g.B) && g.M <= 8 * kSM && static_cast<int64_t>(g.N) * g.sBn * 4 < (int64_t{1} << 32);
}

namespace {
// activation rows load 4 elements at a time
bool skinny_a_vec(const GemmArgs& g) {
  const uintptr_t al = g.a_bf16 ? 7u : 15u;
  return g.sAm % 4 == 0 && g.sAb % 4 == 0 && (reinterpret_cast<uintptr_t>(g.A) & al) == 0;
}

}  // namespace

// Split count of the skinny GEMM. Three workgroups fit on a CU (their LDS
// tiles take 46 KB each), so the grid runs in rounds of 3 * 256 workgroups.
// First the split count (of at most 64, with at least 128 k per split) that
// fills its last round best, the smallest such: a grid of 1.33 rounds would
// leave two thirds of the chip idle in its second round. Then a smaller
// count if one already gives at least a full round and fills its last round
// to three quarters: every split adds partial traffic, and a last round that
// full still keeps the weight stream busy (measured on the absorbed-query
// shape, 576 tiles: two splits 0.114 ms, four 0.121 ms).
int skinny_splits(int batch, int M, int N, int K) {
  const int64_t base = static_cast<int64_t>(batch) * ((M + kSM - 1) / kSM) * ((N + kSN - 1) / kSN);
  constexpr int64_t kRound = 3LL * kNumCUs;
  int64_t smax = (K + 127) / 128;   // at least 128 k per split
  if (smax > 64) smax = 64;
  if (smax < 1) smax = 1;
  auto fill = [&](int64_t s) {
    const int64_t wg = base * s;
    const int64_t rounds = (wg + kRound - 1) / kRound;
    return static_cast<double>(wg) / static_cast<double>(rounds * kRound);
  };
  int64_t best = 1;
  double best_fill = -1.0;
  for (int64_t s = 1; s <= smax; ++s) {
    const double f = fill(s);
    if (f > best_fill + 1e-9) {
      best_fill = f;
      best = s;
    }
  }
  for (int64_t s = 1; s < best; ++s)
    if (base * s >= kRound && fill(s) >= 0.75) return static_cast<int>(s);
  return static_cast<int>(best);
}

size_t gemm_partial_bytes(int batch, int M, int N, int K) {
  const int s = skinny_splits(batch, M, N, K);
  return s > 1 ? sizeof(float) * static_cast<size_t>(s) * batch * M * N : 0;
}

mla_status launch_skinny(const GemmArgs& g, hipStream_t st, float* partial, size_t partial_bytes,
                         int* splits) {
  *splits = 1;
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return MLA_OK;
  if (!skinny_ok(g)) return fail(MLA_ERR_UNSUPPORTED, "skinny gemm: unsupported operands");
  int sp = skinny_splits(g.batch, g.M, g.N, g.K);
  if (partial == nullptr || gemm_partial_bytes(g.batch, g.M, g.N, g.K) > partial_bytes) sp = 1;
  const int kps = (g.K + sp - 1) / sp;
  const int kps_r = (kps + kSK - 1) / kSK * kSK;
  const int gz = sp > 1 ? (g.K + kps_r - 1) / kps_r : 1;
  const dim3 grid((g.N + kSN - 1) / kSN, (g.M + kSM - 1) / kSM, static_cast<unsigned>(g.batch * gz));
  if (grid.z > 65535u) return fail(MLA_ERR_UNSUPPORTED, "gemm too large");
  const bool av = skinny_a_vec(g);
  if (g.a_bf16 && av)
    hipLaunchKernelGGL((skinny_gemm_kernel<1, 1>), grid, dim3(256), 0, st, g, gz, kps_r, partial);
  else if (g.a_bf16)
    hipLaunchKernelGGL((skinny_gemm_kernel<1, 0>), grid, dim3(256), 0, st, g, gz, kps_r, partial);
  else if (av)
    hipLaunchKernelGGL((skinny_gemm_kernel<0, 1>), grid, dim3(256), 0, st, g, gz, kps_r, partial);
  else
    hipLaunchKernelGGL((skinny_gemm_kernel<0, 0>), grid, dim3(256), 0, st, g, gz, kps_r, partial);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
  *splits = gz;
  return MLA_OK;
}

mla_status launch_gemm(const GemmArgs& g, hipStream_t st, float* partial, size_t partial_bytes) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return MLA_OK;
  if (skinny_ok(g)) {
    int gz = 1;
    const mla_status s = launch_skinny(g, st, partial, partial_bytes, &gz);
    if (s != MLA_OK) return s;
    if (gz > 1) {
      const int64_t rows = static_cast<int64_t>(g.batch) * g.M;
      if (g.sYn == 1 && g.N % 4 == 0 && g.sYm % 4 == 0 && g.sYb % 4 == 0 && aligned16(g.Y) &&
          rows <= 65535) {
        const dim3 grid4(static_cast<unsigned>((g.N / 4 + 255) / 256), static_cast<unsigned>(rows));
        hipLaunchKernelGGL(skinny_reduce4_kernel, grid4, dim3(256), 0, st, g, gz,
                           static_cast<const float*>(partial));
      } else {
        const int64_t total = rows * g.N;
        const unsigned blocks = static_cast<unsigned>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
        hipLaunchKernelGGL(skinny_reduce_kernel, dim3(blocks), dim3(256), 0, st, g, gz,
                           static_cast<const float*>(partial));
      }
    }
  } else {
    if (g.B2 != nullptr) return fail(MLA_ERR_UNSUPPORTED, "gemm: two weight matrices need the skinny path");
    const dim3 grid((g.N + kT - 1) / kT, (g.M + kT - 1) / kT, g.batch);
    if (grid.y > 65535u || grid.z > 65535u) return fail(MLA_ERR_UNSUPPORTED, "gemm too large");
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, st, g);
  }
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

mla_status launch_query_finish(const float* q32, int64_t ld, int splits, int64_t split_stride, int T,
                               int n_h, int d_c, int d_rope, float theta, const int32_t* positions,
                               int q_dtype, void* q_abs, void* q_rope, hipStream_t st) {
  if (T <= 0) return MLA_OK;
  if (d_rope > 256) return fail(MLA_ERR_UNSUPPORTED, "query finish: d_rope above 256");
  const double th = theta;
  // enough blocks to fill the chip: heads are split over gridDim.y
  const int ny = n_h < 16 ? n_h : 16;
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(ny));
  if (q_dtype == MLA_FP32)
    hipLaunchKernelGGL(query_finish_kernel<MLA_FP32>, grid, dim3(256), 0, st, q32, ld, splits,
                       split_stride, n_h, d_c, d_rope, th, positions, q_abs, q_rope);
  else
    hipLaunchKernelGGL(query_finish_kernel<MLA_BF16>, grid, dim3(256), 0, st, q32, ld, splits,
                       split_stride, n_h, d_c, d_rope, th, positions, q_abs, q_rope);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "query finish launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
