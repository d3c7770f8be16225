// Internal declarations shared by the HIP sources of the routed-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mdr.h"

namespace mdr {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kPairsPerChunk = 64;  // (query, slot) pairs one remote work-group handles
constexpr int kMaxProbes = 16;
constexpr int kMaxRemote = 16;
constexpr int kMaxSubspaces = 4;
constexpr int kMaxCodesTotal = 64;  // subspaces * codes
constexpr int kMaxAddresses = 4096;
constexpr int kMaxBlocks = 8192;

// Every size of one call, resolved once on the host.
struct Shape {
  int B, H, S, D, W, blk, nb, G, C, A, cap, P, M, R, L, dtype;
  float scale;      // softmax scale (1/sqrt(D) unless given)
  float rope_base;  // mixer only
  long long bins_per_bh;   // capacity of the per-(b,h) pair bins
  int chunks_per_bh;       // upper bound of remote work items per (b,h)
};

// Device buffers of one call (workspace regions or caller-provided outputs).
struct Buffers {
  float* ksum;
  int32_t* addr;
  int32_t* off;
  int32_t* idx;
  int32_t* overflow;
  int32_t* sel;
  int32_t* ncand;
  int32_t* cnt;        // [B,H,nb] selections per block
  int32_t* chunk_off;  // [B,H,nb+1] exclusive scan of per-block remote chunks
  int32_t* bins;       // [B,H,bins_per_bh] (t*R + r) grouped by selected block
  void* part_o;        // [B,H,S,R,D] remote partial outputs (normalised), io dtype
  float* part_ml;      // [B,H,S,R,2] remote partial (max in log2 units, sum)
  void* mq;            // mixer: Q, K, V, O in [B,H,S,D]
  void* mk;
  void* mv;
  void* mo;
};

// First bin slot of block i: blocks before i can be chosen by (nb - L - i') * blk tokens each.
__host__ __device__ inline long long bin_offset(int i, int nb, int L, int blk) {
  long long n = nb - L;
  long long ii = i;
  return (long long)blk * (ii * n - ii * (ii - 1) / 2);
}

// Selection entry r of a token in query block j is used iff it is an eligible block
// (0 <= i <= j - L) not repeated by an earlier entry of the same token.
__device__ inline bool sel_entry_valid(const int32_t* row, int r, int j, int L) {
  const int i = row[r];
  if (i < 0 || i > j - L) return false;
  for (int p = 0; p < r; ++p)
    if (row[p] == i) return false;
  return true;
}

// Launchers (return hipGetLastError()).
hipError_t launch_address(const Shape& s, const void* k, const float* codebook, const float* bias,
                          float* ksum, int32_t* addr, int32_t* cnt_zero, hipStream_t st);
hipError_t launch_post(const Shape& s, const int32_t* addr, int32_t* off, int32_t* idx,
                       int32_t* overflow, hipStream_t st);
hipError_t launch_probe_rerank(const Shape& s, const void* q, const float* codebook, const float* bias,
                               const float* ksum, const int32_t* off, const int32_t* idx,
                               const int32_t* force, int32_t* sel, int32_t* ncand, int32_t* cnt,
                               int32_t* bins, hipStream_t st);
hipError_t launch_fill(int32_t* p, long long n, int32_t value, hipStream_t st);
hipError_t launch_pair_bin(const Shape& s, const int32_t* sel, int32_t* cnt, int32_t* bins,
                           hipStream_t st);
hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v,
                         const int32_t* sel, void* out, const Buffers& b, hipStream_t st);
hipError_t launch_project_heads(const Shape& s, const void* x, const void* w, void* out, bool rope,
                                hipStream_t st);
hipError_t launch_project_out(const Shape& s, const void* o, const void* wo, void* delta,
                              hipStream_t st);

}  // namespace mdr
