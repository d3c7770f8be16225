// Block key summary and product address of one block, shared by the prefill address kernel and
// the decode filing kernel so that both produce bit-identical summaries and addresses.
//
// Summary: the mean of the block's post-RoPE key rows, in fp32 (a fixed order of additions: each
// thread sums a fixed set of rows of one 16-byte column chunk, the row groups are then added in
// order).  Address: per subspace g, code_g = argmax_c <codebook[h,g,c], summary> + bias[h,g,c]
// (first maximum wins), combined as a mixed-radix number with subspace 0 most significant
// (remio.ai, "Monodratic turns sparse attention into a retrieval decision": a product address
// combines the decisions of several learned code components).
#pragma once

#include "mdr_internal.h"

namespace mdr {

template <typename T>
struct Vec16;  // 16-byte vector of T
template <>
struct Vec16<float> {
  typedef float4 type;
  static constexpr int n = 4;
};
template <>
struct Vec16<bf16> {
  typedef bf16x8 type;
  static constexpr int n = 8;
};

__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(bf16 x) { return (float)x; }

template <typename T, int D, int NB = 1>
struct AddressLds {
  static constexpr int NCH = D / Vec16<T>::n;  // 16-byte chunks per row
  static constexpr int RG = 256 / NCH;         // row groups
  float red[NB][RG][D + 1];
  float kbar[NB][D];
  float logit[NB][kMaxCodesTotal];
};

// The codebook slice one thread of a 256-thread work-group holds for the logits: four adjacent
// lanes share one code cc (of the G*C codes of head h), each a quarter of D.  Requested early so
// that it arrives while the keys are read.
template <int D>
struct CodeSlice {
  static constexpr int LPC = 256 / kMaxCodesTotal;  // lanes per code
  static constexpr int DPL = D / LPC;               // codebook dims per lane
  static_assert(DPL % 4 == 0, "whole float4 per lane");
  float w[DPL];
  float bv;
  int cc, part;
  __device__ __forceinline__ void load(const float* __restrict__ cb, const float* __restrict__ bias, int h,
                                       const Shape& s) {
    const int tid = threadIdx.x;
    const int GC = s.G * s.C;
    cc = tid / LPC;
    part = tid % LPC;
    const float* wr = cb + ((size_t)h * GC + (cc < GC ? cc : 0)) * D + part * DPL;
#pragma unroll
    for (int d = 0; d < DPL; d += 4) {
      const float4 v = *(const float4*)(wr + d);
      w[d] = v.x;
      w[d + 1] = v.y;
      w[d + 2] = v.z;
      w[d + 3] = v.w;
    }
    bv = (bias && cc < GC) ? bias[h * GC + cc] : 0.f;
  }
};

// Address (and optional alternate) of one block from its summary kbar (LDS, D floats): the code
// logits <codebook[h,g,c], kbar> + bias (the four lanes of a code each add a quarter of D in a fixed
// order), then one wave takes each subspace's argmax with a butterfly over (logit, code).  All 256
// threads call it (it contains a barrier); `logit` is LDS scratch of kMaxCodesTotal floats.  Thread
// 0 writes *addr_out and, when given, *alt_out: in the subspace with the smallest fp32 margin
// top1 - top2 (ties to the smaller subspace) the runner-up code (the best of the others, smaller
// code on ties) replaces the top code; -1 when C == 1.  margin_out (optional) receives that smallest
// margin (+inf when C == 1): how close the address came to a tie.
template <int D>
__device__ __forceinline__ float code_logit_part(const CodeSlice<D>& cs, const float* kbar) {
  constexpr int LPC = CodeSlice<D>::LPC, DPL = CodeSlice<D>::DPL;
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc = fmaf(cs.w[d], kbar[cs.part * DPL + d], acc);
#pragma unroll
  for (int x = 1; x < LPC; x <<= 1) acc += __shfl_xor(acc, x);
  return acc;
}

// One wave: the per-subspace argmaxes of the logits, the address and (optionally) the alternate and
// the smallest margin; lane 0 writes them.
__device__ __forceinline__ void address_from_logits(const float* logit, int lane, int32_t* __restrict__ addr_out,
                                                    int32_t* __restrict__ alt_out, const Shape& s,
                                                    float* __restrict__ margin_out) {
  int a = 0;
  float best_m = INFINITY;
  int gs = -1, dc = 0;  // subspace of the smallest margin, runner-up code minus top code
  for (int g = 0; g < s.G; ++g) {
    // lanes 0..C-1 hold the subspace's logits; the butterfly keeps the larger logit, the
    // smaller code on ties
    const float lv = lane < s.C ? logit[g * s.C + lane] : -INFINITY;
    float v = lv;
    int c = lane < s.C ? lane : 0x7fffffff;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) {
      const float ov = __shfl_xor(v, x);
      const int oc = __shfl_xor(c, x);
      if (ov > v || (ov == v && oc < c)) {
        v = ov;
        c = oc;
      }
    }
    a = a * s.C + c;
    if (alt_out || margin_out) {
      float v2 = (lane < s.C && lane != c) ? lv : -INFINITY;
      int c2 = (lane < s.C && lane != c) ? lane : 0x7fffffff;
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) {
        const float ov = __shfl_xor(v2, x);
        const int oc = __shfl_xor(c2, x);
        if (ov > v2 || (ov == v2 && oc < c2)) {
          v2 = ov;
          c2 = oc;
        }
      }
      const float m = v - v2;  // +inf when C == 1
      if (m < best_m) {
        best_m = m;
        gs = g;
        dc = c2 - c;
      }
    }
  }
  if (lane == 0) {
    *addr_out = a;
    if (margin_out) *margin_out = best_m;
    if (alt_out) {
      int pw = 1;  // place value of subspace gs (subspace 0 most significant)
      for (int g = gs + 1; g < s.G; ++g) pw *= s.C;
      *alt_out = gs >= 0 ? a + dc * pw : -1;
    }
  }
}

template <int D>
__device__ __forceinline__ void address_from_summary(const CodeSlice<D>& cs, const float* kbar, float* logit,
                                                     int32_t* __restrict__ addr_out, int32_t* __restrict__ alt_out,
                                                     const Shape& s, float* __restrict__ margin_out = nullptr) {
  const int tid = threadIdx.x;
  const float acc = code_logit_part<D>(cs, kbar);
  if (cs.part == 0 && cs.cc < s.G * s.C) logit[cs.cc] = acc + cs.bv;
  __syncthreads();
  if (tid < 64) address_from_logits(logit, tid, addr_out, alt_out, s, margin_out);
}

// All 256 threads of the work-group call it (it contains barriers).  The codebook rows are
// requested together with the key rows.  Writes ksum[bh, i, :] and addr[bh, i], and when `alt` is
// given the block's alternate address (see address_from_summary), for the blocks i0 .. i0 + nv - 1
// (nv <= NB): every block is summed, scored and ranked by the same threads in the same order as a
// single block, so each gets the same bits whatever NB; the blocks' reads are all issued at once and
// their argmaxes run on waves 0 .. NB - 1 side by side.
template <typename T, int D, int BLK = 128, int NB = 1>
__device__ __forceinline__ void block_address(const T* __restrict__ K, const float* __restrict__ cb,
                                              const float* __restrict__ bias, float* __restrict__ ksum,
                                              int32_t* __restrict__ addr, int i0, int bh, AddressLds<T, D, NB>& sm,
                                              const Shape& s, int32_t* __restrict__ alt = nullptr,
                                              float* __restrict__ margin = nullptr, int nv = NB) {
  static_assert(NB * D <= 256 && NB <= 4, "one thread per summary column, one wave per block's argmax");
  constexpr int VEC = Vec16<T>::n;
  constexpr int NCH = AddressLds<T, D, NB>::NCH;
  constexpr int RG = AddressLds<T, D, NB>::RG;
  const int tid = threadIdx.x;
  const int h = bh % s.H;
  CodeSlice<D> cs;
  cs.load(cb, bias, h, s);
  const int ch = tid % NCH, rg = tid / NCH;
  // rows rg, rg + RG, ... of each block, all requested before the first is added (BLK: the largest
  // block this instantiation takes; a slot past the block reads its last row and adds nothing; a block
  // past nv reads the last valid one and is not stored), then added in that order.  No branches
  // around the reads, so that the compiler need not wait on one before issuing the next.
  constexpr int RMAX = (BLK + RG - 1) / RG;
  typename Vec16<T>::type v[NB][RMAX];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const T* base = K + ((size_t)bh * s.S + (size_t)(i0 + min(b, nv - 1)) * s.blk) * D;
#pragma unroll
    for (int u = 0; u < RMAX; ++u) {
      const int r = min(rg + u * RG, s.blk - 1);
      v[b][u] = *(const typename Vec16<T>::type*)(base + (size_t)r * D + ch * VEC);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float acc4[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc4[e] = 0.f;
#pragma unroll
    for (int u = 0; u < RMAX; ++u) {
      const bool in = rg + u * RG < s.blk;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = acc4[e] + to_f(v[b][u][e]);
        acc4[e] = in ? x : acc4[e];
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.red[b][rg][ch * VEC + e] = acc4[e];
  }
  __syncthreads();
  if (tid < NB * D) {  // thread b D + d: column d of block b
    const int b = tid / D, d = tid % D;
    float acc = 0.f;
    for (int g = 0; g < RG; ++g) acc += sm.red[b][g][d];
    const float m = acc / (float)s.blk;
    sm.kbar[b][d] = m;
    if (b < nv) ksum[((size_t)bh * s.nb + i0 + b) * D + d] = m;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float acc = code_logit_part<D>(cs, sm.kbar[b]);
    if (cs.part == 0 && cs.cc < s.G * s.C) sm.logit[b][cs.cc] = acc + cs.bv;
  }
  __syncthreads();
  const int wave = tid >> 6;
  if (wave < nv) {
    const size_t o = (size_t)bh * s.nb + i0 + wave;
    address_from_logits(sm.logit[wave], tid & 63, addr + o, alt ? alt + o : nullptr, s, margin ? margin + o : nullptr);
  }
}

}  // namespace mdr
