// api.hip — the exported C ABI (include/mla.h): argument checks, workspace
// layout, and the launch sequence plan -> split-KV decode -> combine.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "internal.h"

namespace mla {

namespace {
thread_local char g_err[512] = "";

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

mla_status make_plan(const mla_decode_desc* d, DecodePlan* p) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 1 || d->q_len < 1 || d->n_heads < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch, q_len and n_heads must be >= 1");
  if (d->d_c < 8 || d->d_c > 1024 || d->d_c % 8 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_c must be a multiple of 8 in [8, 1024], got %d", d->d_c);
  if (d->d_rope < 0 || d->d_rope > 256 || d->d_rope % 8 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_rope must be a multiple of 8 in [0, 256], got %d", d->d_rope);
  if (d->page_size != kPage)
    return fail(MLA_ERR_UNSUPPORTED, "page_size must be %d, got %d", kPage, d->page_size);
  if (d->max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1");
  if (d->cache_dtype < MLA_FP32 || d->cache_dtype > MLA_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown cache_dtype %d", d->cache_dtype);
  if (d->q_dtype != MLA_FP32 && d->q_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_dtype must be MLA_FP32 or MLA_BF16");
  if (d->q_dtype == MLA_FP32 && d->cache_dtype != MLA_FP32)
    return fail(MLA_ERR_UNSUPPORTED, "fp32 queries are built for the fp32 cache only");
  if (d->out_dtype != MLA_FP32 && d->out_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "out_dtype must be MLA_FP32 or MLA_BF16");
  if (d->num_partitions < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_partitions < 0");
  if ((d->flags & ~MLA_DECODE_FP8_MATH) != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", static_cast<unsigned>(d->flags));
  const int64_t rows = static_cast<int64_t>(d->q_len) * d->n_heads;
  if (rows > (1 << 20)) return fail(MLA_ERR_UNSUPPORTED, "q_len * n_heads too large");
  if (static_cast<int64_t>(d->batch) * d->max_blocks_per_seq > (1LL << 30))
    return fail(MLA_ERR_UNSUPPORTED, "batch * max_blocks_per_seq too large");

  p->rows = static_cast<int>(rows);
  p->path = mfma_supports(d) ? Path::Mfma : Path::Generic;
  const int per_wg = p->path == Path::Mfma ? kMfmaRows : kGenericRows;
  p->row_groups = static_cast<int>((rows + per_wg - 1) / per_wg);
  const int64_t max_pages = static_cast<int64_t>(d->batch) * d->max_blocks_per_seq;
  int64_t G = d->num_partitions;
  if (G == 0) {
    // one wave of workgroups over the chip: one workgroup per CU for the MFMA
    // kernel, four for the generic kernel
    const int64_t target = p->path == Path::Mfma ? kNumCUs : 4 * kNumCUs;
    G = target / p->row_groups;
    if (G < 1) G = 1;
    if (G > max_pages) G = max_pages;
  }
  if (static_cast<int64_t>(G) * p->row_groups > 0x7FFFFFFFLL)
    return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  p->G = G;
  p->slots = G + d->batch;
  p->part_bf16 = (p->path == Path::Mfma && d->out_dtype == MLA_BF16) ? 1 : 0;
  p->plan_off = 0;
  p->opart_off = align256(sizeof(int32_t) * (static_cast<size_t>(d->batch) + 1));
  const size_t part_elem = p->part_bf16 ? 2 : 4;   // bytes per partial element
  p->lse_off = align256(p->opart_off + part_elem * static_cast<size_t>(p->slots) * rows * d->d_c);
  p->lsum_off = align256(p->lse_off + sizeof(float) * static_cast<size_t>(p->slots) * rows);
  p->total = align256(p->lsum_off + sizeof(float) * static_cast<size_t>(p->slots) * rows);
  return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" {

size_t mla_decode_workspace_size(const mla_decode_desc* d) {
  clear_error();
  DecodePlan p;
  if (make_plan(d, &p) != MLA_OK) return 0;
  return p.total;
}

mla_status mla_decode_plan(const mla_decode_desc* d, const int32_t* seq_lens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  clear_error();
  DecodePlan p;
  mla_status s = make_plan(d, &p);
  if (s != MLA_OK) return s;
  if (seq_lens == nullptr || workspace == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens and workspace must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total, workspace_bytes);
  return launch_plan(seq_lens, d->batch, d->max_blocks_per_seq,
                     reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.plan_off),
                     static_cast<hipStream_t>(stream));
}

namespace {
// Shared checks of mla_decode and mla_decode_partial; fills `a`.
mla_status prepare(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                   const void* cache, const float* cache_scale, const int32_t* block_table,
                   const int32_t* seq_lens, float scale, void* workspace, size_t workspace_bytes,
                   DecodePlan* p, DecodeArgs* a) {
  mla_status s = make_plan(d, p);
  if (s != MLA_OK) return s;
  if (q_abs == nullptr || cache == nullptr || block_table == nullptr || seq_lens == nullptr ||
      workspace == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (d->d_rope > 0 && q_rope == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "q_rope is NULL");
  if (d->cache_dtype == MLA_FP8_E4M3 && cache_scale == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "the fp8 cache needs cache_scale");
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(MLA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!aligned16(q_abs) || (q_rope && !aligned16(q_rope)) || !aligned16(cache) ||
      (cache_scale && !aligned16(cache_scale)))
    return fail(MLA_ERR_MISALIGNED, "q_abs, q_rope, cache and cache_scale must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (workspace_bytes < p->total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p->total,
                workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  a->d = d;
  a->p = p;
  a->q_abs = q_abs;
  a->q_rope = q_rope;
  a->cache = cache;
  a->cache_scale = cache_scale;
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->page_start = reinterpret_cast<const int32_t*>(ws + p->plan_off);
  a->scale = scale;
  a->o_part = ws + p->opart_off;
  a->lse_part = reinterpret_cast<float*>(ws + p->lse_off);
  a->l_part = p->path == Path::Mfma ? reinterpret_cast<float*>(ws + p->lsum_off) : nullptr;
  a->o_latent = nullptr;
  a->lse_out = nullptr;
  a->skip_whole = false;
  return MLA_OK;
}

mla_status run_partial(const DecodeArgs& a, hipStream_t st) {
  const bool in_kernel = a.p->path == Path::Mfma && mfma_lds_plan(a.d);
  if (!a.d->plan_ready && !in_kernel) {
    mla_status s = launch_plan(a.seq_lens, a.d->batch, a.d->max_blocks_per_seq,
                               const_cast<int32_t*>(a.page_start), st);
    if (s != MLA_OK) return s;
  }
  return a.p->path == Path::Mfma ? launch_decode_mfma(a, st) : launch_decode_generic(a, st);
}
}  // namespace

mla_status mla_decode(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                      const void* cache, const float* cache_scale, const int32_t* block_table,
                      const int32_t* seq_lens, float scale, void* o_latent, float* lse_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  DecodePlan p;
  DecodeArgs a;
  mla_status s = prepare(d, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                         workspace, workspace_bytes, &p, &a);
  if (s != MLA_OK) return s;
  if (o_latent == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "o_latent is NULL");
  if (!aligned16(o_latent)) return fail(MLA_ERR_MISALIGNED, "o_latent must be 16-byte aligned");
  a.o_latent = o_latent;
  a.lse_out = lse_out;
  a.skip_whole = p.path == Path::Mfma;   // that kernel writes whole sequences' output
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = run_partial(a, st);
  if (s != MLA_OK) return s;
  return launch_combine(a, st);
}

// ---- the allocation-free decode -----------------------------------------
// Its workspace is this file-scope device array (one per GPU, alive until the
// process ends). Host code never uses the array's name as an address: the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t{72} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure,
// with the last error set).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(MLA_ERR_HIP, "mla_decode_noalloc: no current device (or device id >= %d)", kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      fail(MLA_ERR_HIP, "mla_decode_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

size_t mla_decode_noalloc_max_workspace(void) { return kScratchBytes; }

mla_status mla_decode_noalloc(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                              const void* cache, const float* cache_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float scale,
                              void* o_latent, float* lse_out, void* stream) {
  clear_error();
  DecodePlan p;
  mla_status s = make_plan(d, &p);
  if (s != MLA_OK) return s;
  if (p.total > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "mla_decode_noalloc: this call needs %zu bytes of workspace, above the fixed "
                "%zu-byte device scratch array (use mla_decode with a workspace)",
                p.total, kScratchBytes);
  void* ws = scratch_ptr();
  if (ws == nullptr) return MLA_ERR_HIP;
  // the plan in the shared array may belong to another call: always form it
  mla_decode_desc dd = *d;
  dd.plan_ready = 0;
  return mla_decode(&dd, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                    o_latent, lse_out, ws, kScratchBytes, stream);
}

mla_status mla_decode_partial(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                              const void* cache, const float* cache_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  DecodePlan p;
  DecodeArgs a;
  mla_status s = prepare(d, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                         workspace, workspace_bytes, &p, &a);
  if (s != MLA_OK) return s;
  return run_partial(a, static_cast<hipStream_t>(stream));
}

mla_status mla_decode_combine(const mla_decode_desc* d, void* workspace, size_t workspace_bytes,
                              void* o_latent, float* lse_out, void* stream) {
  clear_error();
  DecodePlan p;
  mla_status s = make_plan(d, &p);
  if (s != MLA_OK) return s;
  if (workspace == nullptr || o_latent == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "workspace and o_latent must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!aligned16(o_latent)) return fail(MLA_ERR_MISALIGNED, "o_latent must be 16-byte aligned");
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total,
                workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  DecodeArgs a{};
  a.d = d;
  a.p = &p;
  a.page_start = reinterpret_cast<const int32_t*>(ws + p.plan_off);
  a.o_part = ws + p.opart_off;
  a.lse_part = reinterpret_cast<float*>(ws + p.lse_off);
  a.l_part = p.path == Path::Mfma ? reinterpret_cast<float*>(ws + p.lsum_off) : nullptr;
  a.o_latent = o_latent;
  a.lse_out = lse_out;
  return launch_combine(a, static_cast<hipStream_t>(stream));
}

mla_status mla_decode_validate(const mla_decode_desc* d, const int32_t* seq_lens,
                               const int32_t* block_table, int64_t n_pages, void* stream) {
  clear_error();
  DecodePlan p;
  mla_status s = make_plan(d, &p);
  if (s != MLA_OK) return s;
  if (seq_lens == nullptr || block_table == nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens and block_table must be non-NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<int32_t> lens(d->batch);
  std::vector<int32_t> bt(static_cast<size_t>(d->batch) * d->max_blocks_per_seq);
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MLA_ERR_HIP, "validate: copy to host failed");
  for (int b = 0; b < d->batch; ++b) {
    const int S = lens[b];
    if (S < 0 || static_cast<int64_t>(S) > static_cast<int64_t>(kPage) * d->max_blocks_per_seq)
      return fail(MLA_ERR_BAD_CONTENTS, "seq_lens[%d] = %d outside [0, %d]", b, S,
                  kPage * d->max_blocks_per_seq);
    // a non-empty sequence holds its own query tokens (they are appended to
    // the cache before attention), so it is at least q_len long
    if (S > 0 && S < d->q_len)
      return fail(MLA_ERR_BAD_CONTENTS, "seq_lens[%d] = %d is shorter than q_len = %d", b, S,
                  d->q_len);
    for (int64_t k = 0; k < pages_of(S); ++k) {
      const int32_t pg = bt[static_cast<size_t>(b) * d->max_blocks_per_seq + k];
      if (pg < 0 || pg >= n_pages)
        return fail(MLA_ERR_BAD_CONTENTS, "block_table[%d][%lld] = %d outside [0, %lld)", b,
                    static_cast<long long>(k), pg, static_cast<long long>(n_pages));
    }
  }
  return MLA_OK;
}

mla_status mla_fold_query(const float* W_UQ, const float* W_UK, int32_t n_h, int32_t d_h,
                          int32_t d_c, int32_t d_in, float* W_qabs, void* stream) {
  clear_error();
  if (!W_UQ || !W_UK || !W_qabs) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (n_h < 1 || d_h < 1 || d_c < 1 || d_in < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  GemmArgs g{};
  g.batch = n_h; g.M = d_c; g.N = d_in; g.K = d_h;
  g.A = W_UK; g.a_bf16 = 0; g.sAb = static_cast<int64_t>(d_h) * d_c; g.sAm = 1; g.sAk = d_c;
  g.B = W_UQ; g.sBb = static_cast<int64_t>(d_h) * d_in; g.sBk = d_in; g.sBn = 1;
  g.Y = W_qabs; g.sYb = static_cast<int64_t>(d_c) * d_in; g.sYm = d_in; g.sYn = 1;
  return launch_gemm(g, static_cast<hipStream_t>(stream));
}

mla_status mla_fold_output(const float* W_O, const float* W_UV, int32_t n_h, int32_t d_h,
                           int32_t d_c, int32_t d, float* W_ov, void* stream) {
  clear_error();
  if (!W_O || !W_UV || !W_ov) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (n_h < 1 || d_h < 1 || d_c < 1 || d < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  GemmArgs g{};
  g.batch = n_h; g.M = d; g.N = d_c; g.K = d_h;
  g.A = W_O; g.a_bf16 = 0; g.sAb = d_h; g.sAm = static_cast<int64_t>(n_h) * d_h; g.sAk = 1;
  g.B = W_UV; g.sBb = static_cast<int64_t>(d_h) * d_c; g.sBk = d_c; g.sBn = 1;
  g.Y = W_ov; g.sYb = d_c; g.sYm = static_cast<int64_t>(n_h) * d_c; g.sYn = 1;
  return launch_gemm(g, static_cast<hipStream_t>(stream));
}

namespace {
size_t a256b(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
size_t max2(size_t a, size_t b) { return a > b ? a : b; }
}  // namespace

size_t mla_output_proj_workspace_size(int32_t T, int32_t n_h, int32_t d_c, int32_t d_h, int32_t d,
                                      int32_t mode) {
  if (T < 0 || n_h < 1 || d_c < 1 || d < 1) return 0;
  if (mode == MLA_PROJ_MERGED) return a256b(gemm_partial_bytes(1, T, d, n_h * d_c)) + 256;
  if (mode != MLA_PROJ_TWO_STAGE || d_h < 1) return 0;
  return a256b(sizeof(float) * static_cast<size_t>(T) * n_h * d_h) +
         a256b(max2(gemm_partial_bytes(n_h, T, d_h, d_c), gemm_partial_bytes(1, T, d, n_h * d_h))) + 256;
}

mla_status mla_output_proj(const void* o_latent, int32_t o_dtype, int32_t T, int32_t n_h,
                           int32_t d_c, int32_t d_h, int32_t d, int32_t mode, const float* W1,
                           const float* W2, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  clear_error();
  if (!o_latent || !W1 || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (T < 0 || n_h < 1 || d_c < 1 || d < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes");
  if (o_dtype != MLA_FP32 && o_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "o_dtype must be MLA_FP32 or MLA_BF16");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t K = static_cast<int64_t>(n_h) * d_c;
  if (mode != MLA_PROJ_MERGED && mode != MLA_PROJ_TWO_STAGE)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown mode %d", mode);
  if (mode == MLA_PROJ_TWO_STAGE && !W2) return fail(MLA_ERR_INVALID_ARGUMENT, "two-stage projection needs W_O");
  if (mode == MLA_PROJ_TWO_STAGE && d_h < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "d_h must be >= 1");
  const size_t need = mla_output_proj_workspace_size(T, n_h, d_c, d_h, d, mode);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  if (mode == MLA_PROJ_MERGED) {
    GemmArgs g{};
    g.batch = 1; g.M = T; g.N = d; g.K = static_cast<int>(K);
    g.A = o_latent; g.a_bf16 = o_dtype == MLA_BF16; g.sAb = 0; g.sAm = K; g.sAk = 1;
    g.B = W1; g.sBb = 0; g.sBk = 1; g.sBn = K;
    g.Y = out; g.sYb = 0; g.sYm = d; g.sYn = 1;
    return launch_gemm(g, st, reinterpret_cast<float*>(ws), workspace_bytes);
  }
  float* U = static_cast<float*>(workspace);
  const size_t u_bytes = a256b(sizeof(float) * static_cast<size_t>(T) * n_h * d_h);
  float* part = reinterpret_cast<float*>(ws + u_bytes);
  const size_t part_bytes = workspace_bytes - u_bytes;
  GemmArgs g{};
  g.batch = n_h; g.M = T; g.N = d_h; g.K = d_c;
  g.A = o_latent; g.a_bf16 = o_dtype == MLA_BF16; g.sAb = d_c; g.sAm = K; g.sAk = 1;
  g.B = W1; g.sBb = static_cast<int64_t>(d_h) * d_c; g.sBk = 1; g.sBn = d_c;
  g.Y = U; g.sYb = d_h; g.sYm = static_cast<int64_t>(n_h) * d_h; g.sYn = 1;
  mla_status s = launch_gemm(g, st, part, part_bytes);
  if (s != MLA_OK) return s;
  GemmArgs g2{};
  const int64_t K2 = static_cast<int64_t>(n_h) * d_h;
  g2.batch = 1; g2.M = T; g2.N = d; g2.K = static_cast<int>(K2);
  g2.A = U; g2.a_bf16 = 0; g2.sAb = 0; g2.sAm = K2; g2.sAk = 1;
  g2.B = W2; g2.sBb = 0; g2.sBk = 1; g2.sBn = K2;
  g2.Y = out; g2.sYb = 0; g2.sYm = d; g2.sYn = 1;
  return launch_gemm(g2, st, part, part_bytes);
}

size_t mla_cache_append_workspace_size(int32_t T, int32_t d, int32_t d_c, int32_t d_rope) {
  if (T < 0 || d < 1 || d_c < 1 || d_rope < 0) return 0;
  return a256b(sizeof(float) * static_cast<size_t>(T) * (d_c + d_rope)) +
         a256b(max2(gemm_partial_bytes(1, T, d_c + d_rope, d),
                    max2(gemm_partial_bytes(1, T, d_c, d), gemm_partial_bytes(1, T, d_rope, d)))) +
         256;
}

mla_status mla_cache_write(const float* rows, int32_t T, int32_t d_c, int32_t d_rope, float theta,
                           const int32_t* positions, const int32_t* slots, int32_t cache_dtype,
                           void* cache, float* cache_scale, void* stream) {
  clear_error();
  if (!rows || !positions || !slots || !cache) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (T < 0 || d_c < 1 || d_rope < 0 || d_rope % 2 != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes");
  if (cache_dtype < MLA_FP32 || cache_dtype > MLA_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown cache_dtype");
  if (cache_dtype == MLA_FP8_E4M3 && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "the fp8 cache needs cache_scale");
  return launch_append_finish(rows, T, d_c, d_rope, theta, positions, slots, cache_dtype, cache,
                              cache_scale, static_cast<hipStream_t>(stream));
}

mla_status mla_cache_append(const float* h, int32_t T, int32_t d, const float* W_DKV,
                            const float* W_KR, int32_t d_c, int32_t d_rope, float theta,
                            const int32_t* positions, const int32_t* slots, int32_t cache_dtype,
                            void* cache, float* cache_scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  clear_error();
  if (!h || !W_DKV || (d_rope > 0 && !W_KR) || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (T < 0 || d < 1 || d_c < 1 || d_rope < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes");
  if (workspace_bytes < mla_cache_append_workspace_size(T, d, d_c, d_rope))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* cr = static_cast<float*>(workspace);
  const size_t cr_bytes = a256b(sizeof(float) * static_cast<size_t>(T) * (d_c + d_rope));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + cr_bytes);
  const size_t part_bytes = workspace_bytes - cr_bytes;
  const int L = d_c + d_rope;
  GemmArgs g{};
  g.batch = 1; g.M = T; g.N = d_c; g.K = d;
  g.A = h; g.a_bf16 = 0; g.sAm = d; g.sAk = 1;
  g.B = W_DKV; g.sBk = 1; g.sBn = d;
  g.Y = cr; g.sYm = L; g.sYn = 1;
  if (d_rope > 0) {   // one GEMM over both weight matrices where the skinny path takes it
    GemmArgs gc = g;
    gc.N = L; gc.B2 = W_KR; gc.N1 = d_c;
    if (skinny_ok(gc)) {
      mla_status s = launch_gemm(gc, st, part, part_bytes);
      if (s != MLA_OK) return s;
      return mla_cache_write(cr, T, d_c, d_rope, theta, positions, slots, cache_dtype, cache,
                             cache_scale, stream);
    }
  }
  mla_status s = launch_gemm(g, st, part, part_bytes);
  if (s != MLA_OK) return s;
  if (d_rope > 0) {
    GemmArgs g2 = g;
    g2.N = d_rope; g2.B = W_KR; g2.Y = cr + d_c;
    s = launch_gemm(g2, st, part, part_bytes);
    if (s != MLA_OK) return s;
  }
  return mla_cache_write(cr, T, d_c, d_rope, theta, positions, slots, cache_dtype, cache,
                         cache_scale, stream);
}

size_t mla_absorb_query_workspace_size(int32_t T, int32_t d_in, int32_t n_h, int32_t d_c,
                                       int32_t d_rope) {
  if (T < 0 || d_in < 1 || n_h < 1 || d_c < 1 || d_rope < 0) return 0;
  // the fp32 rows [q_abs | q_rope] (one GEMM over both weight matrices) and
  // its split partials, or the two GEMMs' partials
  return a256b(sizeof(float) * static_cast<size_t>(T) * n_h * (d_c + d_rope)) +
         a256b(max2(gemm_partial_bytes(1, T, n_h * (d_c + d_rope), d_in),
                    max2(gemm_partial_bytes(n_h, T, d_c, d_in), gemm_partial_bytes(1, T, n_h * d_rope, d_in)))) +
         256;
}

mla_status mla_absorb_query(const float* x, int32_t T, int32_t d_in, const float* W_qabs,
                            const float* W_QR, int32_t n_h, int32_t d_c, int32_t d_rope,
                            float theta, const int32_t* positions, int32_t q_dtype, void* q_abs,
                            void* q_rope, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (!x || !W_qabs || !positions || !q_abs || !workspace || (d_rope > 0 && (!W_QR || !q_rope)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (T < 0 || d_in < 1 || n_h < 1 || d_c < 1 || d_rope < 0 || d_rope % 2 != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes");
  if (q_dtype != MLA_FP32 && q_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_dtype must be MLA_FP32 or MLA_BF16");
  if (workspace_bytes < mla_absorb_query_workspace_size(T, d_in, n_h, d_c, d_rope))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* q32 = static_cast<float*>(workspace);
  const size_t q_bytes = a256b(sizeof(float) * static_cast<size_t>(T) * n_h * (d_c + d_rope));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + q_bytes);
  const size_t part_bytes = workspace_bytes - q_bytes;
  // One GEMM over both weight matrices (W_qabs for the first n_h d_c columns,
  // W_QR for the rest) into rows [q_abs | q_rope]; the finish pass sums its
  // split partials, applies RoPE and converts.
  const int64_t ld = static_cast<int64_t>(n_h) * (d_c + d_rope);
  GemmArgs gc{};
  gc.batch = 1; gc.M = T; gc.N = static_cast<int>(ld); gc.K = d_in;
  gc.A = x; gc.a_bf16 = 0; gc.sAm = d_in; gc.sAk = 1;
  gc.B = W_qabs; gc.sBk = 1; gc.sBn = d_in;
  gc.Y = q32; gc.sYm = ld; gc.sYn = 1;
  if (d_rope > 0) { gc.B2 = W_QR; gc.N1 = n_h * d_c; }
  if (ld <= INT32_MAX && skinny_ok(gc)) {
    int splits = 1;
    mla_status s = launch_skinny(gc, st, part, part_bytes, &splits);
    if (s != MLA_OK) return s;
    return splits > 1 ? launch_query_finish(part, ld, splits, static_cast<int64_t>(T) * ld, T, n_h, d_c,
                                            d_rope, theta, positions, q_dtype, q_abs, q_rope, st)
                      : launch_query_finish(q32, ld, 1, 0, T, n_h, d_c, d_rope, theta, positions, q_dtype,
                                            q_abs, q_rope, st);
  }
  // other shapes: one GEMM per weight matrix, each with its own split sums
  GemmArgs g{};
  g.batch = n_h; g.M = T; g.N = d_c; g.K = d_in;
  g.A = x; g.a_bf16 = 0; g.sAb = 0; g.sAm = d_in; g.sAk = 1;
  g.B = W_qabs; g.sBb = static_cast<int64_t>(d_c) * d_in; g.sBk = 1; g.sBn = d_in;
  g.Y = q32; g.sYb = d_c; g.sYm = ld; g.sYn = 1;
  mla_status s = launch_gemm(g, st, part, part_bytes);
  if (s != MLA_OK) return s;
  if (d_rope > 0) {
    GemmArgs g2{};
    g2.batch = 1; g2.M = T; g2.N = n_h * d_rope; g2.K = d_in;
    g2.A = x; g2.a_bf16 = 0; g2.sAm = d_in; g2.sAk = 1;
    g2.B = W_QR; g2.sBk = 1; g2.sBn = d_in;
    g2.Y = q32 + static_cast<int64_t>(n_h) * d_c; g2.sYm = ld; g2.sYn = 1;
    s = launch_gemm(g2, st, part, part_bytes);
    if (s != MLA_OK) return s;
  }
  return launch_query_finish(q32, ld, 1, 0, T, n_h, d_c, d_rope, theta, positions, q_dtype, q_abs,
                             q_rope, st);
}

size_t mla_cache_bytes_per_token(int32_t d_c, int32_t d_rope, int32_t cache_dtype) {
  if (d_c < 1 || d_rope < 0) return 0;
  switch (cache_dtype) {
    case MLA_FP32: return 4u * static_cast<size_t>(d_c + d_rope);
    case MLA_BF16: return 2u * static_cast<size_t>(d_c + d_rope);
    case MLA_FP8_E4M3: return static_cast<size_t>(d_c) + 2u * static_cast<size_t>(d_rope) + 4u;
    default: return 0;
  }
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_BAD_CONTENTS: return "MLA_ERR_BAD_CONTENTS";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_err; }

int32_t mla_version(void) { return 100; }

}  // extern "C"
