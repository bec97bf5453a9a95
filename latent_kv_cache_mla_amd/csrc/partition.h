// partition.h — split-KV work partition shared by the planner, the decode
// kernels, the combine kernel and the host.
//
// The pages of all sequences are concatenated in batch order: sequence b owns
// global pages [page_start[b], page_start[b+1]) with
// page_start[b+1] - page_start[b] = ceil(S_b / 64). The P pages are cut into
// G ranges of (almost) equal size: range g is [floor(g P / G), floor((g+1) P / G)).
// One workgroup processes one range; where a range crosses sequence
// boundaries it produces one partial (o, lse) per sequence piece. The piece of
// (range g, sequence b) is stored in partial slot g + b, so G + B slots
// suffice and the slots of one sequence are found again from the same
// arithmetic, with no list written anywhere.
//
// Plain C++ with no HIP types, so the host tests compile it with g++.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int kPage = 64;

MLA_HD int64_t pages_of(int64_t seq_len) { return (seq_len + kPage - 1) / kPage; }

// First global page of range g of G over P pages.
MLA_HD int64_t range_begin(int64_t g, int64_t P, int64_t G) { return (g * P) / G; }

// Largest g in [0, G) with range_begin(g) <= x, for 0 <= x < P.
MLA_HD int64_t range_of_page(int64_t x, int64_t P, int64_t G) {
  // range_begin(g) <= x  <=>  g * P < (x + 1) * G  <=>  g <= ceil((x+1) G / P) - 1
  int64_t g = ((x + 1) * G + P - 1) / P - 1;
  return g < G - 1 ? g : G - 1;
}

// Partial slot of (range g, sequence b).
MLA_HD int64_t slot_of(int64_t g, int64_t b) { return g + b; }

}  // namespace mla
