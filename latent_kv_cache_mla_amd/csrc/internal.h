// internal.h — declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"
#include "partition.h"

namespace mla {

// Compute units of an MI355X. Planning uses this constant (not a device
// query) so that workspace sizes are a pure function of the descriptor.
constexpr int kNumCUs = 256;
// Rows (query token x head) one workgroup of the MFMA decode kernel covers.
constexpr int kMfmaRows = 128;
// Rows one workgroup of the generic decode kernel covers (one per wavefront).
constexpr int kGenericRows = 4;

enum class Path { Generic, Mfma };

struct DecodePlan {
  Path path;
  int rows;          // q_len * n_heads
  int row_groups;    // workgroups per range along the row dimension
  int64_t G;         // number of page ranges (partitions)
  int64_t slots;     // G + B partial slots
  int part_bf16;     // partials stored as bf16 (MFMA path with a bf16 output), else fp32
  size_t plan_off, opart_off, lse_off, lsum_off, total;  // workspace layout (bytes)
};

// Validates the descriptor (sets the thread's last error) and lays out the
// workspace. Returns MLA_OK or the failure status.
mla_status make_plan(const mla_decode_desc* d, DecodePlan* p);

// thread-local error message
mla_status fail(mla_status s, const char* fmt, ...);
void clear_error();

// ---- launchers (each returns MLA_OK or MLA_ERR_HIP) ----
mla_status launch_plan(const int32_t* seq_lens, int B, int max_blocks, int32_t* page_start,
                       hipStream_t st);

struct DecodeArgs {
  const mla_decode_desc* d;
  const DecodePlan* p;
  const void* q_abs;
  const void* q_rope;
  const void* cache;
  const float* cache_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_start;
  float scale;
  void* o_part;      // bf16 or fp32, per DecodePlan::part_bf16
  float* lse_part;
  // row sums of unnormalised partials (MFMA path); nullptr: the partials are
  // already normalised (generic path)
  float* l_part;
  // final output; the matrix-core kernel writes the rows of every sequence
  // that one piece covers whole straight here (nullptr: partials only)
  void* o_latent;
  float* lse_out;
  // the combine skips sequences covered by one piece (their output is written)
  bool skip_whole;
};

mla_status launch_decode_generic(const DecodeArgs& a, hipStream_t st);
mla_status launch_decode_mfma(const DecodeArgs& a, hipStream_t st);
bool mfma_supports(const mla_decode_desc* d);
// An fp8 cache whose descriptor asks for MLA_DECODE_FP8_MATH.
bool mfma_fp8_math(const mla_decode_desc* d);
// The MFMA kernel forms the page prefix sums itself (and stores them for the
// combine), so no plan launch is needed.
bool mfma_lds_plan(const mla_decode_desc* d);
mla_status launch_combine(const DecodeArgs& a, hipStream_t st);

// fp32 strided batched GEMM: Y[b][m][n] = sum_k A[b](m,k) * B[b](k,n)
// with element (m,k) of A at A + b*sAb + m*sAm + k*sAk (same for B, Y).
// With B2 set (batch 1 only), output columns n >= N1 take their weight row
// n - N1 from B2 (same row stride) instead of B: two weight matrices that
// share the activations in one launch.
struct GemmArgs {
  int batch, M, N, K;
  const void* A; int a_bf16; int64_t sAb, sAm, sAk;
  const float* B; int64_t sBb, sBk, sBn;
  float* Y; int64_t sYb, sYm, sYn;
  const float* B2 = nullptr; int N1 = 0;
};
// Row counts up to 256 with operands contiguous along k run on the fp32
// matrix cores with split-K when `partial` holds gemm_partial_bytes (else
// without splitting); other shapes on an LDS-tiled fp32 vector kernel.
mla_status launch_gemm(const GemmArgs& g, hipStream_t st, float* partial = nullptr,
                       size_t partial_bytes = 0);
size_t gemm_partial_bytes(int batch, int M, int N, int K);
int skinny_splits(int batch, int M, int N, int K);
// The skinny matrix-core GEMM alone (skinny_ok shapes), without the split
// sums: with *splits > 1 on return the result is the sum over z < *splits of
// partial[z * batch * M * N + (b * M + m) * N + n]; with *splits == 1 it is
// in Y.
bool skinny_ok(const GemmArgs& g);
mla_status launch_skinny(const GemmArgs& g, hipStream_t st, float* partial, size_t partial_bytes,
                         int* splits);

// bf16 matrix-core GEMM: C[m, n] = sum_k A[m, k] B[n, k] with A [M, K] (row
// stride lda) and B [N, K] (row stride ldb) in bf16, fp32 accumulation, C in
// fp32 or bf16 (row stride ldc). K, lda, ldb multiples of 8; A, B 16-byte
// aligned. splits > 1 cuts K into that many pieces (fp32 partial tiles in
// `partial` [splits, M, N], summed in split order by a second kernel).
struct MfmaGemmArgs {
  int M, N, K;
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  void* C; int64_t ldc; int c_bf16;
  int splits;
  float* partial;
  // RoPE in the epilogue (bf16 output, no split, the 256 x 256 tile only;
  // launch_gemm_bf16 returns MLA_ERR_UNSUPPORTED otherwise): outputs
  // (2k, 2k + 1) of every rope_dr-column block of row m are rotated by the
  // angle whose cosine and sine are rope_cs[m * rope_dr + 2 k] and [.. + 1]
  const float* rope_cs = nullptr;
  int rope_dr = 0;
};
mla_status launch_gemm_bf16(const MfmaGemmArgs& g, hipStream_t st);
int gemm_bf16_k_per_split(int K, int splits);

// Causal attention of the unabsorbed form over expanded per-head keys and
// values (bf16 rows; head i of a row at column i * width of its part).
struct PrefillAttnArgs {
  const uint16_t* q; int64_t ldq;     // content queries, head i at i * d_h
  const uint16_t* qr; int64_t ldqr;   // rotated rope queries, head i at i * d_R
  const uint16_t* k; int64_t ldk;     // expanded content keys, head i at i * d_h
  const uint16_t* kr; int64_t ldkr;   // the shared rotated rope key
  const uint16_t* v; int64_t ldv;     // expanded values, head i at i * d_v
  const int32_t* cu_seqlens;          // [batch + 1] token offsets of the sequences
  uint16_t* o; int64_t ldo;           // attention output, head i at i * d_v
  float* lse;                         // [n_heads, T] natural log, or nullptr
  float c_log2;                       // scale * log2(e), > 0
  int batch, n_heads, max_seq_len;
  int64_t T;
};
bool prefill_attn_supported(int d_h, int d_rope, int d_v);
mla_status launch_prefill_attn(const PrefillAttnArgs& a, int d_h, int d_rope, int d_v, hipStream_t st);

// RoPE (interleaved pairs) of rows of width d at per-row positions, in place
// on fp32 rows with stride ld: x[r, c0 : c0 + d].
mla_status launch_append_finish(const float* cr, int T, int d_c, int d_rope, float theta,
                                const int32_t* positions, const int32_t* slots,
                                int cache_dtype, void* cache, float* cache_scale,
                                hipStream_t st);
// q32 rows of n_h (d_c + d_rope) values (q_abs, then q_rope), row stride
// ld, summed over `splits` copies split_stride apart.
mla_status launch_query_finish(const float* q32, int64_t ld, int splits, int64_t split_stride, int T,
                               int n_h, int d_c, int d_rope, float theta, const int32_t* positions,
                               int q_dtype, void* q_abs, void* q_rope, hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace mla
