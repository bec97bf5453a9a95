// prefill.hip — the unabsorbed MLA layer for a whole prompt (prefill), and
// the bf16 matrix-core GEMM entry point it is built from.
//
// For every position t of every sequence ([Mishra] "Multi-head Latent
// Attention", "Step 1: a low-rank latent", "Step 4: decoupled RoPE";
// [Zhang] "Multi-head latent attention", "The definitions: project down,
// then up", "Decoupled RoPE: content and position in separate branches",
// "Value absorption: weight and sum first, project after"):
//   [c_t ; k^R_t] = [W^DKV ; W^KR] h_t, k^R_t rotated by RoPE at its position
//       (the cached latent row, returned for the cache write);
//   x_t = W^DQ h_t (query latent) or h_t;
//   [q^C_t ; q^R_t] = [W^UQ ; W^QR] x_t, q^R rotated per head;
//   [k^C_t ; v_t] = [W^UK ; W^UV] c_t (expanded per-head keys and values);
//   o_{t,i} = softmax_j<=t((q^C_{t,i} . k^C_{j,i} + q^R_{t,i} . k^R_j) scale) v_{j,i};
//   out_t = W^O [o_{t,1} ; ... ; o_{t,n_h}].
// Unlike decode, nothing is absorbed: the pages keep the unabsorbed form
// where all positions are processed at once and the work is bound by
// arithmetic ([LLMsBlog] "Multi-Head Latent Attention: How Low-Rank KV
// Compression Scales LLM Serving", opening section and "Hardware Trade-offs
// and Tensor Parallelism"; [Mishra] "Step 2: absorb the up-projections").
// The projections run on gemm_mfma.hip, the attention on prefill_attn.hip;
// the two kernels here rotate the rope parts (angles in fp64) and round the
// GEMM outputs to bf16 for the next products.
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

size_t a256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Row t of X (fp32, row stride ldx): columns [0, width) are copied to Y
// (bf16, row stride ldy) except that the n_rope blocks of d_r columns
// starting at column r0 are first rotated by RoPE at positions[t]
// (interleaved pairs). With write_back the rotated fp32 values replace X's.
// One thread per (row, pair index k): the angle is computed once and applied
// to every block; a second loop copies the other columns.
__global__ __launch_bounds__(256) void rope_round_kernel(float* __restrict__ X, int64_t ldx, int width,
                                                         int r0, int n_rope, int d_r,
                                                         const int32_t* __restrict__ positions,
                                                         double theta, uint16_t* __restrict__ Y,
                                                         int64_t ldy, int write_back, int64_t T) {
  const int half_r = d_r / 2;
  const int64_t pairs = n_rope > 0 ? T * half_r : 0;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < pairs; e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / half_r;
    const int k = static_cast<int>(e % half_r);
    float cs, sn;
    rope_cs(positions[t], k, d_r, theta, &cs, &sn);
    float* x = X + t * ldx;
    uint16_t* y = Y + t * ldy;
    for (int hb = 0; hb < n_rope; ++hb) {
      const int col = r0 + hb * d_r + 2 * k;
      const float x0 = x[col], x1 = x[col + 1];
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      y[col] = f32_to_bf16(y0);
      y[col + 1] = f32_to_bf16(y1);
      if (write_back) {
        x[col] = y0;
        x[col + 1] = y1;
      }
    }
  }
  const int rope_end = r0 + n_rope * d_r;
  const int64_t total = T * width;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < total; e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / width;
    const int col = static_cast<int>(e % width);
    if (col >= r0 && col < rope_end) continue;
    Y[t * ldy + col] = f32_to_bf16(X[t * ldx + col]);
  }
}

// The same pass, one workgroup per row, 8 columns per thread and step (two
// 16-byte loads, one 16-byte store): the row's d_r / 2 angles are computed
// once into LDS (fp64, as above), then every 8-column unit is either rounded
// or, inside a rope block, rotated (4 pairs) and rounded. Needs X and Y rows
// 16-byte aligned, width a multiple of 8 and, with rope blocks, r0 and d_r
// multiples of 8 and d_r at most 256.
__global__ __launch_bounds__(256) void rope_round8_kernel(float* __restrict__ X, int64_t ldx, int width,
                                                          int r0, int n_rope, int d_r,
                                                          const int32_t* __restrict__ positions,
                                                          double theta, uint16_t* __restrict__ Y,
                                                          int64_t ldy, int write_back) {
  __shared__ float cs_lds[128], sn_lds[128];
  const int64_t t = blockIdx.x;
  const int half_r = d_r / 2;
  if (n_rope > 0) {
    if (threadIdx.x < half_r) {
      float c, sn;
      rope_cs(positions[t], static_cast<int>(threadIdx.x), d_r, theta, &c, &sn);
      cs_lds[threadIdx.x] = c;
      sn_lds[threadIdx.x] = sn;
    }
    __syncthreads();
  }
  float* x = X + t * ldx;
  uint16_t* y = Y + t * ldy;
  const int rope_end = r0 + n_rope * d_r;
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  for (int col = 8 * static_cast<int>(threadIdx.x); col < width; col += 8 * 256) {
    f4 v0 = *reinterpret_cast<const f4*>(x + col);
    f4 v1 = *reinterpret_cast<const f4*>(x + col + 4);
    float e[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    if (col >= r0 && col < rope_end) {
      const int k0 = ((col - r0) % d_r) / 2;   // first pair of the unit
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float c = cs_lds[k0 + p], sn = sn_lds[k0 + p];
        const float a = e[2 * p], b = e[2 * p + 1];
        e[2 * p] = a * c - b * sn;
        e[2 * p + 1] = a * sn + b * c;
      }
      if (write_back) {
        *reinterpret_cast<f4*>(x + col) = f4{e[0], e[1], e[2], e[3]};
        *reinterpret_cast<f4*>(x + col + 4) = f4{e[4], e[5], e[6], e[7]};
      }
    }
    u4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = static_cast<uint32_t>(f32_to_bf16(e[2 * p])) | (static_cast<uint32_t>(f32_to_bf16(e[2 * p + 1])) << 16);
    *reinterpret_cast<u4*>(y + col) = o;
  }
}

// cos and sin of every (row, pair) angle, fp64 as in rope_round8_kernel:
// cs[t * d_r + 2 k] = cos(pos_t theta^(-2k/d_r)), cs[t * d_r + 2 k + 1] = sin(..)
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ positions, int64_t T,
                                                         int d_r, double theta, float* __restrict__ cs) {
  const int half_r = d_r / 2;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= T * half_r) return;
  const int64_t t = e / half_r;
  const int k = static_cast<int>(e % half_r);
  float c, sn;
  rope_cs(positions[t], k, d_r, theta, &c, &sn);
  cs[t * d_r + 2 * k] = c;
  cs[t * d_r + 2 * k + 1] = sn;
}

mla_status launch_rope_round(float* X, int64_t ldx, int width, int r0, int n_rope, int d_r,
                             const int32_t* positions, float theta, uint16_t* Y, int64_t ldy,
                             int write_back, int64_t T, hipStream_t st) {
  if (T > 0 && T < 0x7FFFFFFF && aligned16(X) && aligned16(Y) && ldx % 4 == 0 && ldy % 8 == 0 &&
      width % 8 == 0 && (n_rope == 0 || (r0 % 8 == 0 && d_r % 8 == 0 && d_r <= 256))) {
    hipLaunchKernelGGL(rope_round8_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, st, X, ldx, width, r0,
                       n_rope, d_r, positions, static_cast<double>(theta), Y, ldy, write_back);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "rope launch: %s", hipGetErrorString(e));
    return MLA_OK;
  }
  const int64_t work = T * (width > d_r / 2 ? width : d_r / 2);
  const unsigned blocks = static_cast<unsigned>((work + 255) / 256 < 8192 ? (work + 255) / 256 : 8192);
  hipLaunchKernelGGL(rope_round_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, X, ldx, width, r0,
                     n_rope, d_r, positions, static_cast<double>(theta), Y, ldy, write_back, T);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "rope launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

// workspace layout of mla_prefill (byte offsets)
struct PrefillLayout {
  size_t lat, cb, krb, x, q32, qb, kv, ob, total;
};

mla_status prefill_layout(const mla_prefill_desc* d, int64_t T, PrefillLayout* L) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 1 || d->max_seq_len < 1 || d->d_model < 8 || d->n_heads < 1 || d->d_head < 8 ||
      d->d_rope < 0 || d->d_c < 8 || d->d_cq < 0 || T < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "prefill: bad sizes");
  if (d->d_model % 8 || d->d_head % 8 || d->d_rope % 8 || d->d_c % 8 || d->d_cq % 8)
    return fail(MLA_ERR_UNSUPPORTED, "prefill: every width must be a multiple of 8");
  if (!prefill_attn_supported(d->d_head, d->d_rope, d->d_head))
    return fail(MLA_ERR_UNSUPPORTED, "prefill: attention is built for (d_h, d_R) in "
                "{(128, 64), (64, 16), (64, 32), (128, 0)}, got (%d, %d)", d->d_head, d->d_rope);
  const size_t t = static_cast<size_t>(T);
  const size_t nh = d->n_heads, dh = d->d_head, dr = d->d_rope;
  size_t off = 0;
  L->lat = off; off = a256(off + 4 * t * (d->d_c + dr));
  L->cb = off;  off = a256(off + 2 * t * d->d_c);
  L->krb = off; off = a256(off + 2 * t * (dr > 0 ? dr : 8));
  L->x = off;   off = a256(off + 2 * t * d->d_cq);
  L->q32 = off; off = a256(off + 4 * t * nh * (dh + dr));
  L->qb = off;  off = a256(off + 2 * t * nh * (dh + dr));
  L->kv = off;  off = a256(off + 2 * t * 2 * nh * dh);
  L->ob = off;  off = a256(off + 2 * t * nh * dh);
  L->total = off;
  return MLA_OK;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

mla_status mla_gemm_bf16(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B,
                         int64_t ldb, void* C, int64_t ldc, int32_t c_dtype, int32_t splits,
                         float* partial, void* stream) {
  clear_error();
  if (M < 0 || N < 0 || K < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: negative size");
  if (M == 0 || N == 0) return MLA_OK;
  if (!A || !B || !C) return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: NULL pointer");
  if (lda < K || ldb < K || ldc < N) return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: leading dimension too small");
  if (c_dtype != MLA_FP32 && c_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: c_dtype must be MLA_FP32 or MLA_BF16");
  if (splits < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: splits must be >= 1");
  if (splits > 1 && partial == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "gemm: split-K needs a partial buffer");
  MfmaGemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = static_cast<const uint16_t*>(A); g.lda = lda;
  g.B = static_cast<const uint16_t*>(B); g.ldb = ldb;
  g.C = C; g.ldc = ldc; g.c_bf16 = c_dtype == MLA_BF16;
  g.splits = splits; g.partial = partial;
  return launch_gemm_bf16(g, static_cast<hipStream_t>(stream));
}

size_t mla_gemm_bf16_partial_size(int32_t M, int32_t N, int32_t K, int32_t splits) {
  if (M < 0 || N < 0 || K < 0 || splits < 1) return 0;
  if (splits == 1) return 0;
  const int kps = gemm_bf16_k_per_split(K, splits);
  const int gz = kps > 0 ? (K + kps - 1) / kps : 1;
  return sizeof(float) * static_cast<size_t>(gz) * M * N;
}

mla_status mla_prefill_attention(const mla_prefill_desc* d, int64_t T, const void* q, int64_t ldq,
                                 const void* q_rope, int64_t ldqr, const void* k, int64_t ldk,
                                 const void* k_rope, int64_t ldkr, const void* v, int64_t ldv,
                                 const int32_t* cu_seqlens, float scale, void* o, int64_t ldo,
                                 float* lse, void* stream) {
  clear_error();
  PrefillLayout L;
  mla_status s = prefill_layout(d, T, &L);
  if (s != MLA_OK) return s;
  if (!q || !k || !v || !o || !cu_seqlens || (d->d_rope > 0 && (!q_rope || !k_rope)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "prefill attention: NULL pointer");
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(MLA_ERR_INVALID_ARGUMENT, "prefill attention: scale must be positive and finite");
  const int64_t nh = d->n_heads;
  if (ldq < nh * d->d_head || ldk < nh * d->d_head || ldv < nh * d->d_head || ldo < nh * d->d_head ||
      (d->d_rope > 0 && (ldqr < nh * d->d_rope || ldkr < d->d_rope)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "prefill attention: row stride below the row width");
  if (ldq % 8 || ldk % 8 || ldv % 8 || ldo % 4 || (d->d_rope > 0 && (ldqr % 8 || ldkr % 8)) ||
      !aligned16(q) || !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(o) & 7u) ||
      (d->d_rope > 0 && (!aligned16(q_rope) || !aligned16(k_rope))))
    return fail(MLA_ERR_MISALIGNED, "prefill attention: inputs must be 16-byte aligned rows, o 8-byte");
  if (T == 0) return MLA_OK;
  PrefillAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q); a.ldq = ldq;
  a.qr = static_cast<const uint16_t*>(d->d_rope > 0 ? q_rope : q); a.ldqr = d->d_rope > 0 ? ldqr : ldq;
  a.k = static_cast<const uint16_t*>(k); a.ldk = ldk;
  a.kr = static_cast<const uint16_t*>(d->d_rope > 0 ? k_rope : k); a.ldkr = d->d_rope > 0 ? ldkr : ldk;
  a.v = static_cast<const uint16_t*>(v); a.ldv = ldv;
  a.cu_seqlens = cu_seqlens;
  a.o = static_cast<uint16_t*>(o); a.ldo = ldo;
  a.lse = lse;
  a.c_log2 = scale * 1.4426950408889634f;
  a.batch = d->batch; a.n_heads = d->n_heads; a.max_seq_len = d->max_seq_len; a.T = T;
  return launch_prefill_attn(a, d->d_head, d->d_rope, d->d_head, static_cast<hipStream_t>(stream));
}

size_t mla_prefill_workspace_size(const mla_prefill_desc* d, int64_t T) {
  clear_error();
  PrefillLayout L;
  return prefill_layout(d, T, &L) == MLA_OK ? L.total : 0;
}

mla_status mla_prefill(const mla_prefill_desc* d, const void* h, int64_t T, const int32_t* cu_seqlens,
                       const int32_t* positions, const mla_prefill_weights* w, float scale, float* out,
                       float* latent, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  clear_error();
  PrefillLayout L;
  mla_status s = prefill_layout(d, T, &L);
  if (s != MLA_OK) return s;
  if (!h || !cu_seqlens || !positions || !w || !out || !workspace || !w->W_DKVR || !w->W_UQR ||
      !w->W_UKV || !w->W_O || (d->d_cq > 0 && !w->W_DQ))
    return fail(MLA_ERR_INVALID_ARGUMENT, "prefill: NULL pointer");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "prefill: workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "prefill: workspace needs %zu bytes, got %zu", L.total,
                workspace_bytes);
  if (!aligned16(h) || !aligned16(w->W_DKVR) || !aligned16(w->W_UQR) || !aligned16(w->W_UKV) ||
      !aligned16(w->W_O) || (w->W_DQ && !aligned16(w->W_DQ)))
    return fail(MLA_ERR_MISALIGNED, "prefill: h and the weights must be 16-byte aligned");
  if (T == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int D = d->d_model, nh = d->n_heads, dh = d->d_head, dr = d->d_rope, dc = d->d_c;
  const int T32 = static_cast<int>(T);
  if (T > 0x7FFFFFFF) return fail(MLA_ERR_UNSUPPORTED, "prefill: too many tokens");
  float* lat = latent ? latent : reinterpret_cast<float*>(ws + L.lat);
  uint16_t* cb = reinterpret_cast<uint16_t*>(ws + L.cb);
  uint16_t* krb = reinterpret_cast<uint16_t*>(ws + L.krb);
  uint16_t* xb = reinterpret_cast<uint16_t*>(ws + L.x);
  float* q32 = reinterpret_cast<float*>(ws + L.q32);
  uint16_t* qb = reinterpret_cast<uint16_t*>(ws + L.qb);
  uint16_t* kv = reinterpret_cast<uint16_t*>(ws + L.kv);
  uint16_t* ob = reinterpret_cast<uint16_t*>(ws + L.ob);
  const uint16_t* hb = static_cast<const uint16_t*>(h);
  auto gemm = [&](int M, int N, int K, const uint16_t* A, int64_t lda, const void* B, int64_t ldb,
                  void* C, int64_t ldc, int c_bf16, int splits = 1, float* partial = nullptr) {
    MfmaGemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.A = A; g.lda = lda;
    g.B = static_cast<const uint16_t*>(B); g.ldb = ldb;
    g.C = C; g.ldc = ldc; g.c_bf16 = c_bf16; g.splits = splits; g.partial = partial;
    return launch_gemm_bf16(g, st);
  };
  const int LW = dc + dr;   // latent row width
  // 1. the latent row [c ; k^R] (fp32), k^R rotated in place; bf16 copies.
  // Its few output columns give few 128 x 128 tiles (160 at 4096 tokens and
  // a 576-wide latent, a third of one round of the chip's 512 workgroup
  // slots), so K is split (up to four parts) while the grid stays within one
  // round; the partial tiles go to the q32 region, not yet written.
  {
    const int64_t tiles = static_cast<int64_t>((T32 + 127) / 128) * ((LW + 127) / 128);
    int sl = 1;
    for (int sp = 2; sp <= 4; ++sp) {
      const int kps = gemm_bf16_k_per_split(D, sp);
      const int gz = (D + kps - 1) / kps;
      const size_t need = sizeof(float) * static_cast<size_t>(gz) * static_cast<size_t>(T) * LW;
      if (kps < 256 || tiles * gz > 2 * kNumCUs || need > L.qb - L.q32) break;
      sl = sp;
    }
    if ((s = gemm(T32, LW, D, hb, D, w->W_DKVR, D, lat, LW, 0, sl, sl > 1 ? q32 : nullptr)) != MLA_OK)
      return s;
  }
  if ((s = launch_rope_round(lat, LW, dc, 0, 0, 2, positions, d->rope_theta, cb, dc, 0, T, st)) != MLA_OK)
    return s;
  if (dr > 0 && (s = launch_rope_round(lat + dc, LW, dr, 0, 1, dr, positions, d->rope_theta, krb, dr, 1, T,
                                       st)) != MLA_OK)
    return s;
  // 2. the query input: the query latent W^DQ h, or h itself
  const uint16_t* x = hb;
  int din = D;
  if (d->d_cq > 0) {
    if ((s = gemm(T32, d->d_cq, D, hb, D, w->W_DQ, D, xb, d->d_cq, 1)) != MLA_OK) return s;
    x = xb;
    din = d->d_cq;
  }
  // 3. [q^C ; q^R] for every head into the bf16 rows qb: q^C = W^UQ x
  // straight to bf16 (the GEMM rounds), q^R = W^QR x in fp32 (compact rows
  // of n_h d_R), then rotated per head and rounded into its columns of qb.
  const int QW = nh * (dh + dr);
  const int QC = nh * dh, QR = nh * dr;
  if ((s = gemm(T32, QC, din, x, din, w->W_UQR, din, qb, QW, 1)) != MLA_OK) return s;
  if (dr > 0) {
    const uint16_t* wqr = static_cast<const uint16_t*>(w->W_UQR) + static_cast<int64_t>(QC) * din;
    // where the large tile takes it, q^R leaves its GEMM rotated and in bf16
    // (the angles from a table of T x d_R values in the q32 region); else the
    // fp32 GEMM and the RoPE pass
    bool fused = false;
    if (dr % 4 == 0) {
      const int64_t n_ang = static_cast<int64_t>(T) * (dr / 2);
      hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((n_ang + 255) / 256)), dim3(256), 0, st,
                         positions, static_cast<int64_t>(T), dr, static_cast<double>(d->rope_theta), q32);
      if (hipGetLastError() != hipSuccess) return fail(MLA_ERR_HIP, "rope table launch failed");
      MfmaGemmArgs g{};
      g.M = T32; g.N = QR; g.K = din; g.A = x; g.lda = din; g.B = wqr; g.ldb = din;
      g.C = qb + QC; g.ldc = QW; g.c_bf16 = 1; g.splits = 1; g.partial = nullptr;
      g.rope_cs = q32; g.rope_dr = dr;
      s = launch_gemm_bf16(g, st);
      if (s == MLA_OK) fused = true;
      else if (s != MLA_ERR_UNSUPPORTED) return s;
      else clear_error();
    }
    if (!fused) {
      if ((s = gemm(T32, QR, din, x, din, wqr, din, q32, QR, 0)) != MLA_OK) return s;
      if ((s = launch_rope_round(q32, QR, QR, 0, nh, dr, positions, d->rope_theta, qb + QC, QW, 0, T,
                                 st)) != MLA_OK)
        return s;
    }
  }
  // 4. expanded keys and values [k^C ; v] = [W^UK ; W^UV] c
  if ((s = gemm(T32, 2 * nh * dh, dc, cb, dc, w->W_UKV, dc, kv, 2 * nh * dh, 1)) != MLA_OK) return s;
  // 5. causal attention per head
  s = mla_prefill_attention(d, T, qb, QW, qb + static_cast<int64_t>(nh) * dh, QW, kv, 2 * nh * dh,
                            krb, dr > 0 ? dr : 8, kv + static_cast<int64_t>(nh) * dh, 2 * nh * dh,
                            cu_seqlens, scale, ob, static_cast<int64_t>(nh) * dh, lse, stream);
  if (s != MLA_OK) return s;
  // 6. out = W^O [o_1 ; ... ; o_{n_h}]. 320 tiles of 256 x 256 at 4096 tokens
  // and d 5120 are 1.25 rounds of the chip's 256 workgroups; splitting K
  // fills the last round. The fp32 partial tiles go to the q32 region, which
  // nothing reads once the attention has run.
  const int KO = nh * dh;
  const int64_t tiles = static_cast<int64_t>((T32 + 255) / 256) * ((D + 255) / 256);
  // Whole rounds of unsplit tiles first, then the remaining columns with K
  // split so that they fill one more round: the same matrix work as
  // splitting every tile, but partial tiles (written, then summed) only for
  // the remainder (at 4096 tokens and d 5120: 256 tiles over 4096 columns,
  // then 64 tiles of the last 1024 columns in four splits).
  {
    const int tm = (T32 + 255) / 256, tn = (D + 255) / 256;
    if (tiles > 256 && tiles % 256 != 0 && 256 % tm == 0) {
      const int n1t = static_cast<int>(tiles / 256) * (256 / tm);   // column tiles left unsplit
      const int64_t tiles2 = static_cast<int64_t>(tm) * (tn - n1t);
      const int s2 = tiles2 > 0 ? static_cast<int>(256 / tiles2 < 4 ? 256 / tiles2 : 4) : 0;
      const int N1 = n1t * 256, N2 = D - N1;
      if (n1t < tn && s2 >= 2 && N1 % 8 == 0) {
        const int kps = gemm_bf16_k_per_split(KO, s2);
        const int gz = (KO + kps - 1) / kps;
        const size_t need = sizeof(float) * static_cast<size_t>(gz) * static_cast<size_t>(T) * N2;
        if (kps >= 1024 && need <= L.qb - L.q32) {
          const uint16_t* wo2 = static_cast<const uint16_t*>(w->W_O) + static_cast<int64_t>(N1) * KO;
          if ((s = gemm(T32, N1, KO, ob, KO, w->W_O, KO, out, D, 0)) != MLA_OK) return s;
          return gemm(T32, N2, KO, ob, KO, wo2, KO, out + N1, D, 0, s2, q32);
        }
      }
    }
  }
  int so = 1;
  double best = static_cast<double>((tiles + 255) / 256);
  for (int sp = 2; sp <= 4; ++sp) {
    const int kps = gemm_bf16_k_per_split(KO, sp);
    const int gz = (KO + kps - 1) / kps;
    const size_t need = sizeof(float) * static_cast<size_t>(gz) * static_cast<size_t>(T) * D;
    if (kps < 1024 || need > L.qb - L.q32) break;
    const double cost = static_cast<double>((tiles * gz + 255) / 256) / gz;
    if (cost < best - 1e-9) { best = cost; so = sp; }
  }
  return gemm(T32, D, KO, ob, KO, w->W_O, KO, out, D, 0, so, so > 1 ? q32 : nullptr);
}

}  // extern "C"
