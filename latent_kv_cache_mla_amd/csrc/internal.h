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
struct GemmArgs {
  int batch, M, N, K;
  const void* A; int a_bf16; int64_t sAb, sAm, sAk;
  const float* B; int64_t sBb, sBk, sBn;
  float* Y; int64_t sYb, sYm, sYn;
};
mla_status launch_gemm(const GemmArgs& g, hipStream_t st);

// RoPE (interleaved pairs) of rows of width d at per-row positions, in place
// on fp32 rows with stride ld: x[r, c0 : c0 + d].
mla_status launch_append_finish(const float* cr, int T, int d_c, int d_rope, float theta,
                                const int32_t* positions, const int32_t* slots,
                                int cache_dtype, void* cache, float* cache_scale,
                                hipStream_t st);
mla_status launch_query_finish(const float* q_abs32, const float* q_rope32, int T, int n_h,
                               int d_c, int d_rope, float theta, const int32_t* positions,
                               int q_dtype, void* q_abs, void* q_rope, hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace mla
