// MFMA tile helpers of the attention kernels (forward and backward): K/V blocks staged row-major in
// LDS, the query operand of S^T = K Q^T held in registers with lane l owning query l%16, and the
// accumulation O^T += V^T P^T from the score layout without any shuffle.
#pragma once

#include <type_traits>

#include "mdr_internal.h"

namespace mdr {
namespace tiles {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int BLK>
struct Tile {
  static constexpr bool bf = std::is_same<T, bf16>::value;
  // K and V rows in LDS (elements), row-major.  For bf16 the row stride is D + 16 elements: the eight
  // rows that half a wave's transposing reads (tr_keys4) touch then fall in disjoint bank windows.
  // One stride for both, since score_tile also takes V rows (the backward's dP = dO V^T).
  static constexpr int KST = bf ? D + 16 : D + 4;
  static constexpr int VST = KST;
  static_assert(VST == KST, "score_tile reads V rows with the K stride");
  static constexpr int K_ELEMS = BLK * KST;
  static constexpr int V_ELEMS = BLK * VST;
  static constexpr int NQF = bf ? D / 32 : D / 4;    // query operand registers
  static constexpr int NT = BLK / 16;                // 16-key sub-tiles
  static constexpr int ND = D / 16;                  // 16-wide d tiles
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr size_t LDS_BYTES = (size_t)(K_ELEMS + V_ELEMS) * sizeof(T);
};

template <typename T, int D>
struct QFrag;
template <int D>
struct QFrag<bf16, D> {
  bf16x8 v[D / 32];
};
template <int D>
struct QFrag<float, D> {
  float v[D / 4];
};

// Query operand of S^T = K Q^T for the query row qp (lane's query is l%16).
template <typename T, int D>
__device__ inline void load_q(QFrag<T, D>& qf, const T* qp, int lane) {
  const int s = lane >> 4;
  if constexpr (std::is_same<T, bf16>::value) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf.v[kk] = *(const bf16x8*)(qp + 32 * kk + 8 * s);
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const float4 v = *(const float4*)(qp + s * (D / 4) + 4 * c);
      qf.v[4 * c + 0] = v.x;
      qf.v[4 * c + 1] = v.y;
      qf.v[4 * c + 2] = v.z;
      qf.v[4 * c + 3] = v.w;
    }
  }
}

// S^T tile n (keys 16n..16n+15 as rows, the wave's 16 queries as columns).
template <typename T, int D, int BLK>
__device__ inline f32x4 score_tile(const QFrag<T, D>& qf, const T* Ks, int n, int lane) {
  using TL = Tile<T, D, BLK>;
  const int s = lane >> 4, r = lane & 15;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (TL::bf) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const bf16x8 a = *(const bf16x8*)(Ks + (16 * n + r) * TL::KST + 32 * kk + 8 * s);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf.v[kk], acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const float4 a = *(const float4*)(Ks + (16 * n + r) * TL::KST + s * (D / 4) + 4 * c);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, qf.v[4 * c + 0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, qf.v[4 * c + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, qf.v[4 * c + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, qf.v[4 * c + 3], acc, 0, 0, 0);
    }
  }
  return acc;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, local lane l receives
// in slot k the (l % 4)-th 16-bit value at the address that local lane 4k + l / 4 supplies.  So if
// lane r supplies row r / 4 of a 4-row tile, columns 4 (r % 4) .. + 3, lane r receives the four
// rows' values in column r (rows 0..3 in slots 0..3); the layout was checked on gfx950 with an
// in-bounds probe.  tile: the tile's first row and column (LDS, bf16), stride: row stride in
// elements (a multiple of 4); tr_keys4 puts the values in slots at .. at + 3 of a.
__device__ __forceinline__ bf16x4 tr_col4(const bf16* tile, int stride, int r) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const bf16* src = tile + (r >> 2) * stride + 4 * (r & 3);
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src));
  bf16x4 w;
  __builtin_memcpy(&w, &v, 8);
  return w;
}
__device__ __forceinline__ void tr_keys4(bf16x8& a, int at, const bf16* tile, int stride, int r) {
  const bf16x4 w = tr_col4(tile, stride, r);
#pragma unroll
  for (int e = 0; e < 4; ++e) a[at + e] = w[e];
}

// O^T += V^T P^T over one block; p[n][k] = P^T[16n + 4(l/16) + k][l%16].  For bf16 the MFMA's
// k-slot 8(l/16) + e stands for key 32pp + 4(l/16) + e (e < 4) or 32pp + 16 + 4(l/16) + e - 4 (e >= 4),
// the same permutation on both operands, so P needs no shuffle.
template <typename T, int D, int BLK>
__device__ inline void pv_block(f32x4 (&o)[D / 16], const f32x4 (&p)[BLK / 16], const T* Vx, int lane) {
  using TL = Tile<T, D, BLK>;
  const int s = lane >> 4, r = lane & 15;
  if constexpr (TL::bf) {
#pragma unroll
    for (int pp = 0; pp < BLK / 32; ++pp) {
      bf16x8 b;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        b[k] = (bf16)p[2 * pp][k];
        b[4 + k] = (bf16)p[2 * pp + 1][k];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        // V^T[d][key] for the 8 keys of this lane's k-slots (32pp + 4s + {0..3} and + 16 + {0..3}) at
        // d = 16dt + r, by two transposing LDS reads
        bf16x8 a;
        tr_keys4(a, 0, Vx + (32 * pp + 4 * s) * TL::VST + 16 * dt, TL::VST, r);
        tr_keys4(a, 4, Vx + (32 * pp + 16 + 4 * s) * TL::VST + 16 * dt, TL::VST, r);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[dt], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < BLK / 16; ++n) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const float a = Vx[(16 * n + 4 * s + k) * TL::VST + 16 * dt + r];
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[n][k], o[dt], 0, 0, 0);
        }
      }
    }
  }
}

// 2^x with the hardware instruction alone (no rescaling of denormal results: those flush to zero,
// which is below anything a softmax weight here can resolve).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <typename T>
__device__ inline void store4(T* dst, const f32x4& v, float mul) {
  if constexpr (std::is_same<T, bf16>::value) {
    const bf16x4 b = {(bf16)(v[0] * mul), (bf16)(v[1] * mul), (bf16)(v[2] * mul), (bf16)(v[3] * mul)};
    *(bf16x4*)dst = b;
  } else {
    *(float4*)dst = make_float4(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
  }
}

// Raw 16- and 8-byte register vectors (native vector types, so they stay in registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive values of T as raw bits (a partial's or an output's column quad).
template <typename T>
using Raw4 = typename std::conditional<std::is_same<T, bf16>::value, u32x2, u32x4>::type;

template <typename T>
__device__ inline f32x4 unpack4(const Raw4<T>& r) {
  if constexpr (std::is_same<T, bf16>::value) {
    const bf16x4 b = *(const bf16x4*)&r;
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  } else {
    const float4 v = *(const float4*)&r;
    return f32x4{v.x, v.y, v.z, v.w};
  }
}

// pv_block for bf16 with P^T already in bf16, four values per sub-tile: p[n] = P^T[16n + 4(l/16) + 0..3][l%16].
template <int D, int BLK>
__device__ inline void pv_block_bf16(f32x4 (&o)[D / 16], const bf16x4 (&p)[BLK / 16], const bf16* Vx, int lane) {
  using TL = Tile<bf16, D, BLK>;
  const int s = lane >> 4, r = lane & 15;
#pragma unroll
  for (int pp = 0; pp < BLK / 32; ++pp) {
    bf16x8 b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      b[k] = p[2 * pp][k];
      b[4 + k] = p[2 * pp + 1][k];
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      bf16x8 a;
      tr_keys4(a, 0, Vx + (32 * pp + 4 * s) * TL::VST + 16 * dt, TL::VST, r);
      tr_keys4(a, 4, Vx + (32 * pp + 16 + 4 * s) * TL::VST + 16 * dt, TL::VST, r);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[dt], 0, 0, 0);
    }
  }
}

// One block of K and V held in registers between its global read and its LDS store, so that the
// read can be issued long before the LDS is free.
template <typename T, int D, int BLK, int NTHR>
struct KVRegs {
  using TL = Tile<T, D, BLK>;
  static constexpr int NCH = D / TL::VEC;
  static constexpr int TOTAL = BLK * NCH;
  static constexpr int NL = (TOTAL + NTHR - 1) / NTHR;
  u32x4 k[NL], v[NL];
  __device__ __forceinline__ void load(const T* __restrict__ Kg, const T* __restrict__ Vg, int tid) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int c = u * NTHR + tid;
      if (TOTAL % NTHR == 0 || c < TOTAL) {
        const int row = c / NCH, ch = c % NCH;
        k[u] = *(const u32x4*)(Kg + (size_t)row * D + ch * TL::VEC);
        v[u] = *(const u32x4*)(Vg + (size_t)row * D + ch * TL::VEC);
      }
    }
  }
  __device__ __forceinline__ void store(T* Ks, T* Vx, int tid) const {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int c = u * NTHR + tid;
      if (TOTAL % NTHR == 0 || c < TOTAL) {
        const int row = c / NCH, ch = c % NCH;
        *(u32x4*)(Ks + row * TL::KST + ch * TL::VEC) = k[u];
        *(u32x4*)(Vx + row * TL::VST + ch * TL::VEC) = v[u];
      }
    }
  }
};


}  // namespace tiles
}  // namespace mdr
