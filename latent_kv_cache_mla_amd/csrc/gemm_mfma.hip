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
// groups. The next K step's global loads are in flight during the current
// step's MFMAs. Rows past M or N and K steps past the end load zeros.
// Split-K (for skinny M, where the output tiles alone do not fill the chip)
// writes fp32 partial tiles that a second kernel sums in split order.
#include "internal.h"
#include "device_common.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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
  // row c / 8, elements 8 (c % 8) .. + 7
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j, row = c >> 3, kc = (c & 7) * 8;
      const int k = k0 + kc;
      const int64_t m = m0 + row, n = n0 + row;
      ra[j] = (m < g.M && k < ke) ? *reinterpret_cast<const uint4*>(g.A + m * g.lda + k)
                                  : make_uint4(0u, 0u, 0u, 0u);
      rb[j] = (n < g.N && k < ke) ? *reinterpret_cast<const uint4*>(g.B + n * g.ldb + k)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j, row = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[buf][row * kPitch + kc]) = ra[j];
      *reinterpret_cast<uint4*>(&Bs[buf][row * kPitch + kc]) = rb[j];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  if (kb < ke) {
    gload(kb);
    swrite(0);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += kBK) {
    const bool more = k0 + kBK < ke;
    if (more) gload(k0 + kBK);
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
    if (more) swrite(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // acc[i][j] register r holds C[m][n] with m = 8 (r / 4) + 4 half + r % 4 and
  // n = l32 within the 32 x 32 tile (i, j)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + l32;
        if (m >= g.M || n >= g.N) continue;
        const float v = acc[i][j][r];
        if (g.splits > 1) {
          g.partial[(static_cast<int64_t>(kz) * g.M + m) * g.N + n] = v;
        } else if (g.c_bf16) {
          static_cast<uint16_t*>(g.C)[m * g.ldc + n] = f32_to_bf16(v);
        } else {
          static_cast<float*>(g.C)[m * g.ldc + n] = v;
        }
      }
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
  const dim3 grid(static_cast<unsigned>((g.N + kBN - 1) / kBN), static_cast<unsigned>((g.M + kBM - 1) / kBM),
                  static_cast<unsigned>(gz));
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, a, kps);
  if (gz > 1) {
    const int64_t total = static_cast<int64_t>(g.M) * g.N;
    const unsigned blocks = static_cast<unsigned>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(gemm_split_reduce, dim3(blocks), dim3(256), 0, st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "bf16 GEMM launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace mla
