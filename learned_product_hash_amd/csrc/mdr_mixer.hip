// Boundary of the stateless mixer: [batch, sequence, width] -> attention delta
// (aitechinspire.com write-up of Monodratic, "Snapshot: key facts from the report": a stateless
// [batch, sequence, width] -> attention-delta mixer; normalisation, residuals, feed-forward
// layers and scheduling stay with the host model).  RoPE is applied to queries and keys before
// routing (same section; remio.ai, "Monodratic claims learned routing can make sparse causal
// attention more selective", section "Monodratic turns sparse attention into a retrieval
// decision").
//
//   k_gemm   C = A B on MFMA with 64x64 tiles staged in LDS; A may be read from the head-split
//            [B,H,S,D] layout (as a [B*S, H*D] matrix) and C written to it.
//   k_rope   in place on [B,H,S,D]: pairs (i, i + D/2) rotate by pos * base^(-2i/D); the angle
//            and its sine/cosine are taken in double so fp32 outputs keep full precision.
//   k_mm     C = A B with register-prefetched 64 x NT tiles; as the fused projection it computes Q, K
//            and V in one launch and, in its epilogue, applies RoPE to Q and K, stores whole rows, and
//            for K forms each block's summary (the mean of the block's stored key rows) and its
//            product address -- the address stage of the core then has nothing left to do (blocks of
//            up to 64 tokens and widths divisible by 8; otherwise k_gemm, k_rope and the address
//            kernel); as the output projection it reads the head-split O directly.
#include "mdr_address.h"
#include "mdr_internal.h"

#include <type_traits>

namespace mdr {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct HeadMap {
  int S, H, D;
  // element (m, n) of a [B*S, H*D] matrix stored as [B,H,S,D]
  __device__ size_t operator()(int m, int n) const {
    const int b = m / S, s = m % S, h = n / D, d = n % D;
    return (((size_t)b * H + h) * S + s) * D + d;
  }
};

template <typename T, bool A_HEADS, bool C_HEADS>
__global__ __launch_bounds__(256) void k_gemm(const T* __restrict__ A, const T* __restrict__ Bm, T* __restrict__ C,
                                              int M, int N, int Kd, HeadMap hm) {
  constexpr bool bf = std::is_same<T, bf16>::value;
  constexpr int KT = bf ? 32 : 16;
  constexpr int KS = KT + (bf ? 8 : 4);
  __shared__ __align__(16) T As[64 * KS];
  __shared__ __align__(16) T Bt[64 * KS];  // B tile transposed: [n][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int s = lane >> 4, r = lane & 15;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < Kd; k0 += KT) {
    for (int e = tid; e < 64 * KT; e += 256) {
      const int row = e / KT, col = e % KT;
      const int m = m0 + row, kk = k0 + col;
      T av = (T)0.f;
      if (m < M && kk < Kd) av = A_HEADS ? A[hm(m, kk)] : A[(size_t)m * Kd + kk];
      As[row * KS + col] = av;
    }
    for (int e = tid; e < 64 * KT; e += 256) {
      const int kr = e / 64, nc = e % 64;
      const int kk = k0 + kr, n = n0 + nc;
      T bv = (T)0.f;
      if (kk < Kd && n < N) bv = Bm[(size_t)kk * N + n];
      Bt[nc * KS + kr] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj) {
        const T* ar = As + (wm + 16 * ti + r) * KS;
        const T* br = Bt + (wn + 16 * tj + r) * KS;
        if constexpr (bf) {
          const bf16x8 a = *(const bf16x8*)(ar + 8 * s);
          const bf16x8 b = *(const bf16x8*)(br + 8 * s);
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[ti][tj], 0, 0, 0);
        } else {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[4 * kk + s], br[4 * kk + s], acc[ti][tj], 0, 0, 0);
        }
      }
    __syncthreads();
  }
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m = m0 + wm + 16 * ti + 4 * s + k, n = n0 + wn + 16 * tj + r;
        if (m < M && n < N) {
          const T v = (T)acc[ti][tj][k];
          if (C_HEADS)
            C[hm(m, n)] = v;
          else
            C[(size_t)m * N + n] = v;
        }
      }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rope(T* __restrict__ X, long long rows, int S, int D, double base) {
  const int half = D / 2;
  const long long n = rows * half;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const long long row = e / half;
    const int i = (int)(e % half);
    const int pos = (int)(row % S);
    const double theta = pow(base, -2.0 * i / D);
    double sn, cs;
    sincos((double)pos * theta, &sn, &cs);
    T* x = X + row * D;
    const float x1 = (float)x[i], x2 = (float)x[i + half];
    const float c = (float)cs, sv = (float)sn;
    x[i] = (T)(x1 * c - x2 * sv);
    x[i + half] = (T)(x2 * c + x1 * sv);
  }
}

// C = A B on MFMA for MT x NT output tiles, 256 threads (2 x 2 waves of MT/2 x NT/2), contraction
// steps of KT (64 bf16 / 32 fp32): the next step's A and B tiles are read into registers while the
// current step is multiplied out of LDS.  B is passed transposed ([n][k], k contiguous: the mixer
// transposes its weights once per call), so both tiles are plain 16-byte row copies into LDS.  The
// tile then goes through LDS once more so that every row leaves as 16-byte vectors.
//   AHEADS  A is the head-split [B,H,S,D] layout read as a [B*S, H*D] matrix
//   QKV     three products at once (B0/B1/B2 = Wq/Wk/Wv, C0/C1/C2 = Q/K/V in [B,H,S,D]); the
//           epilogue applies RoPE to Q and K and, for K, forms each block's summary from the stored
//           rows and its product address (and alternate) with address_from_summary
// Requires Kd % (16 / sizeof(T)) == 0 and Nm % NT == 0 (with NT % D == 0 for QKV).
struct QkvEpilogue {
  const float* cb;
  const float* bias;
  float* ksum;
  int32_t* addr;
  int32_t* alt;
  int32_t* pair_zero;
  float* amargin;
};

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 l (lds uniform
// over the wave).
__device__ __forceinline__ void lds_load16(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

template <typename T, int MT, int NT, bool AHEADS, bool QKV, int D>
__global__ __launch_bounds__(256) void k_mm(const T* __restrict__ A, const T* __restrict__ B0,
                                            const T* __restrict__ B1, const T* __restrict__ B2, T* __restrict__ C0,
                                            T* __restrict__ C1, T* __restrict__ C2, int M, int Nm, int Kd, HeadMap hm,
                                            QkvEpilogue ep, Shape s) {
  constexpr bool bf = std::is_same<T, bf16>::value;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int KT = bf ? 64 : 32;
  constexpr int KS = KT + VEC;                 // LDS row stride: 16 bytes of padding
  constexpr int TI = MT / 32;                  // 16-row tiles per wave (waves split MT in halves)
  constexpr int TJ = NT / 32;                  // 16-column tiles per wave
  constexpr int AR = MT * KT / VEC / 256;      // A vectors per thread per step
  constexpr int BR = KT * NT / VEC / 256;      // B vectors per thread per step
  static_assert(AR >= 1 && BR >= 1 && MT * KT / VEC % 256 == 0 && KT * NT / VEC % 256 == 0, "whole vectors");
  constexpr int CST = NT + 1;                  // output rows of 64 at a time (floats)
  constexpr size_t STAGE = (size_t)(MT + NT) * KS * sizeof(T);
  constexpr size_t EPIB = (size_t)64 * CST * 4;
  constexpr int DRB = KT * (int)sizeof(T);  // bytes of a row per contraction step (direct path)
  static_assert(DRB == 128, "eight 16-byte chunks per row and step");
  constexpr size_t DSTAGE = (size_t)(MT + NT) * DRB;
  constexpr size_t SM0 = STAGE > EPIB ? STAGE : EPIB;
  __shared__ __align__(16) char smem[SM0 > 2 * DSTAGE ? SM0 : 2 * DSTAGE];
  T* As = (T*)smem;
  T* Bt = As + MT * KS;
  float* Cs = (float*)smem;  // after the main loop
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * MT;
  const int ng = blockIdx.y * NT;
  const int which = QKV ? ng / Nm : 0, n0 = QKV ? ng % Nm : ng;
  const T* Bm = which == 0 ? B0 : which == 1 ? B1 : B2;
  T* Cm = which == 0 ? C0 : which == 1 ? C1 : C2;
  const int wm = (wave >> 1) * (MT / 2), wn = (wave & 1) * (NT / 2);
  const int sl = lane >> 4, r = lane & 15;
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int b = 0; b < TJ; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ar[AR], br[BR];
  auto gload = [&](int k0) __attribute__((always_inline)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < AR; ++u) {
      const int c = u * 256 + tid;
      const int row = c / (KT / VEC), cv = c % (KT / VEC);
      const int m = m0 + row, kk = k0 + cv * VEC;
      const bool ok = m < M && kk < Kd;
      const size_t off = AHEADS ? hm(ok ? m : 0, ok ? kk : 0) : (size_t)(ok ? m : 0) * Kd + (ok ? kk : 0);
      ar[u] = ok ? *(const u32x4*)(A + off) : z;
    }
#pragma unroll
    for (int u = 0; u < BR; ++u) {
      const int c = u * 256 + tid;
      const int row = c / (KT / VEC), cv = c % (KT / VEC);
      const int kk = k0 + cv * VEC;
      const bool ok = kk < Kd;
      br[u] = ok ? *(const u32x4*)(Bm + (size_t)(n0 + row) * Kd + (ok ? kk : 0)) : z;
    }
  };
  auto lstore = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < AR; ++u) {
      const int c = u * 256 + tid;
      const int row = c / (KT / VEC), cv = c % (KT / VEC);
      *(u32x4*)(As + row * KS + cv * VEC) = ar[u];
    }
#pragma unroll
    for (int u = 0; u < BR; ++u) {
      const int c = u * 256 + tid;
      const int row = c / (KT / VEC), cv = c % (KT / VEC);
      *(u32x4*)(Bt + row * KS + cv * VEC) = br[u];
    }
  };
  if (Kd % KT == 0) {
    // ---- two LDS stages filled by direct global-to-LDS loads: a wave's 16-byte load per lane fills
    // eight consecutive 128-byte rows of a stage (lane l lands at byte 16 l), one contraction step of
    // a row per 128 bytes.  Lane l of such a load fetches the row's chunk (l % 8) ^ (row % 8), so
    // chunk c of a row sits in slot c ^ (row % 8): the 16 rows of an operand fragment then spread
    // over all banks.  Rows past M read row M - 1 (never stored).  Step s + 1 is requested right after
    // the barrier that opens step s, so it arrives while step s is multiplied.
    constexpr int NG = (MT + NT) / 8;  // 8-row groups per stage
    static_assert(NG % 4 == 0, "whole groups per wave");
    char* sb = smem;
    auto dload = [&](int k0, char* buf) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NG / 4; ++u) {
        const int g = u * 4 + wave;
        const int row = 8 * g + (lane >> 3);
        const int kk = k0 + (((lane & 7) ^ (row & 7)) * VEC);
        const T* src;
        if (8 * g < MT) {  // uniform: a group is all A rows or all B rows
          const int m = min(m0 + row, M - 1);
          src = A + (AHEADS ? hm(m, kk) : (size_t)m * Kd + kk);
        } else {
          src = Bm + (size_t)(n0 + row - MT) * Kd + kk;
        }
        lds_load16(src, buf + g * 8 * DRB);
      }
    };
    auto frag = [&](const char* buf, int row, int chunk) -> const char* {
      return buf + row * DRB + ((chunk ^ (row & 7)) << 4);
    };
    const int nst = Kd / KT;
    dload(0, sb);
    for (int st = 0; st < nst; ++st) {
      const char* cur = sb + (st & 1) * DSTAGE;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of step st are in LDS
      __syncthreads();                // everyone's are; step st - 1 is multiplied everywhere
      if (st + 1 < nst) dload((st + 1) * KT, sb + ((st + 1) & 1) * DSTAGE);
#pragma unroll
      for (int ks = 0; ks < (bf ? KT / 32 : KT / 4); ++ks) {
        if constexpr (bf) {
          bf16x8 af[TI], bfr[TJ];
#pragma unroll
          for (int ti = 0; ti < TI; ++ti) af[ti] = *(const bf16x8*)frag(cur, wm + 16 * ti + r, 4 * ks + sl);
#pragma unroll
          for (int tj = 0; tj < TJ; ++tj) bfr[tj] = *(const bf16x8*)frag(cur, MT + wn + 16 * tj + r, 4 * ks + sl);
#pragma unroll
          for (int ti = 0; ti < TI; ++ti)
#pragma unroll
            for (int tj = 0; tj < TJ; ++tj)
              acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ti], bfr[tj], acc[ti][tj], 0, 0, 0);
        } else {
          float af[TI], bfr[TJ];
#pragma unroll
          for (int ti = 0; ti < TI; ++ti) af[ti] = *(const float*)(frag(cur, wm + 16 * ti + r, ks) + 4 * sl);
#pragma unroll
          for (int tj = 0; tj < TJ; ++tj) bfr[tj] = *(const float*)(frag(cur, MT + wn + 16 * tj + r, ks) + 4 * sl);
#pragma unroll
          for (int ti = 0; ti < TI; ++ti)
#pragma unroll
            for (int tj = 0; tj < TJ; ++tj)
              acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ti], bfr[tj], acc[ti][tj], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the epilogue reuses the stages
  } else {
    gload(0);
    for (int k0 = 0; k0 < Kd; k0 += KT) {
      lstore();
      __syncthreads();
      if (k0 + KT < Kd) gload(k0 + KT);  // in flight during this step's products
  #pragma unroll
      for (int ks = 0; ks < (bf ? KT / 32 : KT / 4); ++ks) {
        // the step's operand fragments of this wave, each used for TJ (A) or TI (B) products
        if constexpr (bf) {
          bf16x8 af[TI], bfr[TJ];
  #pragma unroll
          for (int ti = 0; ti < TI; ++ti) af[ti] = *(const bf16x8*)(As + (wm + 16 * ti + r) * KS + 32 * ks + 8 * sl);
  #pragma unroll
          for (int tj = 0; tj < TJ; ++tj) bfr[tj] = *(const bf16x8*)(Bt + (wn + 16 * tj + r) * KS + 32 * ks + 8 * sl);
  #pragma unroll
          for (int ti = 0; ti < TI; ++ti)
  #pragma unroll
            for (int tj = 0; tj < TJ; ++tj)
              acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ti], bfr[tj], acc[ti][tj], 0, 0, 0);
        } else {
          float af[TI], bfr[TJ];
  #pragma unroll
          for (int ti = 0; ti < TI; ++ti) af[ti] = As[(wm + 16 * ti + r) * KS + 4 * ks + sl];
  #pragma unroll
          for (int tj = 0; tj < TJ; ++tj) bfr[tj] = Bt[(wn + 16 * tj + r) * KS + 4 * ks + sl];
  #pragma unroll
          for (int ti = 0; ti < TI; ++ti)
  #pragma unroll
            for (int tj = 0; tj < TJ; ++tj)
              acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ti], bfr[tj], acc[ti][tj], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
  // ---- epilogue, 64 rows at a time through LDS (lane holds rows 4(l/16) + k, column l%16 of each
  // 16x16 tile)
  [[maybe_unused]] double* theta = nullptr;
  if constexpr (QKV) {
    __shared__ double th[D / 2];  // RoPE frequencies base^(-2i/D), in double
    if (tid < D / 2) th[tid] = pow((double)s.rope_base, -2.0 * tid / D);
    theta = th;
  }
  for (int hf = 0; hf < MT / 64; ++hf) {
    const int mh = m0 + hf * 64;
    if (hf > 0) __syncthreads();  // the previous rows are no longer read
    if (wm / 64 == hf) {
#pragma unroll
      for (int ti = 0; ti < TI; ++ti)
#pragma unroll
        for (int tj = 0; tj < TJ; ++tj)
#pragma unroll
          for (int k = 0; k < 4; ++k) Cs[(wm % 64 + 16 * ti + 4 * sl + k) * CST + wn + 16 * tj + r] = acc[ti][tj][k];
    }
    __syncthreads();
    if constexpr (QKV) {
      if (which < 2) {
        // RoPE on pairs (d, d + D/2) of each head in the tile, at the token's position in its sequence.
        // A thread keeps one pair column and walks the rows RSTEP apart.  Its first row's angle
        // pos * theta is formed in double, reduced to [-pi, pi] in double, and its sine / cosine taken
        // in float; each further row rotates that (cosine, sine) by the angle of RSTEP positions (a
        // few float ulps per step, at most 64 / RSTEP - 1 steps), unless the rows cross into the next
        // sequence, where the angle is formed afresh.
        constexpr double kTwoPi = 6.283185307179586476925286766559;
        constexpr int PCN = NT / 2;        // pair columns per row of the tile
        constexpr int RSTEP = 256 / PCN;   // rows between a thread's consecutive elements
        static_assert(256 % PCN == 0 && RSTEP <= 32, "whole rows per pass");
        const int pc = tid % PCN;
        const int hc = pc / (D / 2), i = pc % (D / 2);
        const int col = hc * D + i;
        auto angle = [&](int p, float* sv, float* c) __attribute__((always_inline)) {
          const double ang = (double)p * theta[i];
          const double red = fma(-rint(ang * (1.0 / kTwoPi)), kTwoPi, ang);
          sincosf((float)red, sv, c);
        };
        float sstep, cstep;
        angle(RSTEP, &sstep, &cstep);
        float sv = 0.f, c = 1.f;
        int pos = -1;
        for (int row = tid / PCN; row < 64; row += RSTEP) {
          if (pos >= 0 && pos + RSTEP < s.S) {
            pos += RSTEP;
            const float c2 = c * cstep - sv * sstep;
            sv = fmaf(sv, cstep, c * sstep);
            c = c2;
          } else {
            pos = (mh + row) % s.S;
            angle(pos, &sv, &c);
          }
          const float x1 = Cs[row * CST + col], x2 = Cs[row * CST + col + D / 2];
          Cs[row * CST + col] = x1 * c - x2 * sv;
          Cs[row * CST + col + D / 2] = x2 * c + x1 * sv;
        }
        __syncthreads();
      }
    }
    // ---- the rows out as 16-byte vectors.  Thread tid keeps row tid % 64 and takes its column
    // chunks tid / 64, + 4, ...: the 64 lanes of a read are 64 rows (an odd row stride), so the reads
    // hit distinct banks.  The K tile's stored (rounded) values stay in LDS for its summaries.
    {
      const int row = tid % 64;
      const int m = mh + row;
      [[maybe_unused]] int b = 0, t = 0;
      if constexpr (QKV) {
        b = m / s.S;
        t = m % s.S;
      }
      for (int cv = tid / 64; cv < NT / VEC; cv += 4) {
        T v[VEC];
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
          v[x] = (T)Cs[row * CST + cv * VEC + x];
          if (QKV && which == 1) Cs[row * CST + cv * VEC + x] = (float)v[x];
        }
        if (m < M) {
          const int n = n0 + cv * VEC;
          size_t off;
          if constexpr (QKV)
            off = (((size_t)b * s.H + n / D) * s.S + t) * D + n % D;
          else
            off = (size_t)m * Nm + n;
          *(u32x4*)(Cm + off) = *(const u32x4*)v;
        }
      }
    }
    if constexpr (QKV) {
      if (which == 1) {  // uniform for the work-group
        __shared__ float kbar[D];
        __shared__ float logit[kMaxCodesTotal];
        __syncthreads();
        // ---- K: each (head, block) in these rows: summary = mean of its stored key rows (added in
        // row order), then its product address (and alternate)
        for (int hc = 0; hc < NT / D; ++hc) {
          const int h = (n0 + hc * D) / D;
          CodeSlice<D> cs;
          cs.load(ep.cb, ep.bias, h, s);
          for (int u = 0; u < 64 / s.blk; ++u) {
            const int mb = mh + u * s.blk;  // first row of the block (blocks never straddle sequences)
            if (mb >= M) break;             // uniform
            const int b = mb / s.S, i = (mb % s.S) / s.blk;
            const int bh = b * s.H + h;
            if (tid < D) {
              float a = 0.f;
              for (int rr = 0; rr < s.blk; ++rr) a += Cs[(u * s.blk + rr) * CST + hc * D + tid];
              const float mval = a / (float)s.blk;
              kbar[tid] = mval;
              ep.ksum[((size_t)bh * s.nb + i) * D + tid] = mval;
            }
            if (ep.pair_zero) clear_pair_counts(ep.pair_zero, s, bh, i, tid, 256);
            __syncthreads();
            address_from_summary<D>(cs, kbar, logit, ep.addr + (size_t)bh * s.nb + i,
                                    ep.alt ? ep.alt + (size_t)bh * s.nb + i : nullptr, s,
                                    ep.amargin ? ep.amargin + (size_t)bh * s.nb + i : nullptr);
            __syncthreads();  // kbar and logit are rewritten next
          }
        }
      }
    }
  }
}

// The mixer's weights transposed into the workspace in one launch: matrix z = first + blockIdx.z of
// (Wq, Wk, Wv: W x N; Wo: N x W) goes to wt + z N W, out[c][r] = in[r][c], through a padded 32 x 32
// LDS tile; tiles past a matrix's edge do nothing.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ w0, const T* __restrict__ w1,
                                                   const T* __restrict__ w2, const T* __restrict__ w3,
                                                   T* __restrict__ wt, int W, int N, int first) {
  __shared__ T tile[32][33];
  const int z = first + blockIdx.z;
  const T* in = z == 0 ? w0 : z == 1 ? w1 : z == 2 ? w2 : w3;
  const int R = z < 3 ? W : N, Cc = z < 3 ? N : W;
  T* out = wt + (size_t)z * N * W;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  for (int y = ty; y < 32; y += 8)
    if (r0 + y < R && c0 + tx < Cc) tile[y][tx] = in[(size_t)(r0 + y) * Cc + c0 + tx];
  __syncthreads();
  for (int y = ty; y < 32; y += 8)
    if (c0 + y < Cc && r0 + tx < R) out[(size_t)(c0 + y) * R + r0 + tx] = tile[tx][y];
}

template <typename T>
hipError_t transpose_weights(const Shape& s, const void* wq, const void* wk, const void* wv, const void* wo, void* wt,
                             int first, int count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const int W = s.W, N = s.H * s.D, side = (W > N ? W : N) + 31;
  hipLaunchKernelGGL(k_transpose<T>, dim3(side / 32, side / 32, count), dim3(256), 0, st, (const T*)wq,
                     (const T*)wk, (const T*)wv, (const T*)wo, (T*)wt, W, N, first);
  return hipGetLastError();
}

// The output projection over at least this many rows uses 128-row tiles (64 x 64 per wave: half the
// LDS operand reads per flop of 64-row tiles; 45 -> 40 us at 32K x 512 x 512).  The fused projection
// keeps 64-row tiles: at 128 rows its registers allow two waves per SIMD and it ran slower
// (143 -> 172 us).
constexpr int kBigM = 16384;

// Largest output tile width (128, 64, 32) dividing Nm and, for the fused projection, holding whole
// heads; 0 when none.
int mm_tile(int Nm, int D, bool qkv) {
  for (int nt = 128; nt >= 32; nt >>= 1)
    if (Nm % nt == 0 && (!qkv || nt % D == 0)) return nt;
  return 0;
}

template <typename T, int NT, int D>
hipError_t qkv_launch(const Shape& s, const void* x, void* q, void* k, void* v, const QkvEpilogue& ep, const void* wt,
                      hipStream_t st) {
  const int M = s.B * s.S, Nm = s.H * s.D;
  HeadMap hm{s.S, s.H, s.D};
  const T* t0 = (const T*)wt;  // Wq, Wk, Wv transposed by launch_transpose_weights
  const T* t1 = t0 + (size_t)Nm * s.W;
  const T* t2 = t1 + (size_t)Nm * s.W;
  hipLaunchKernelGGL((k_mm<T, 64, NT, false, true, D>), dim3((M + 63) / 64, 3 * Nm / NT), dim3(256), 0, st,
                     (const T*)x, t0, t1, t2, (T*)q, (T*)k, (T*)v, M, Nm, s.W, hm, ep, s);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t qkv_fused_d(const Shape& s, const void* x, void* q, void* k, void* v, const QkvEpilogue& ep, const void* wt,
                       hipStream_t st) {
  switch (mm_tile(s.H * s.D, D, true)) {
    case 128: return qkv_launch<T, 128, D>(s, x, q, k, v, ep, wt, st);
    case 64: if constexpr (D <= 64) return qkv_launch<T, 64, D>(s, x, q, k, v, ep, wt, st); break;
    case 32: if constexpr (D <= 32) return qkv_launch<T, 32, D>(s, x, q, k, v, ep, wt, st); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t qkv_fused(const Shape& s, const void* x, void* q, void* k, void* v, const QkvEpilogue& ep, const void* wt,
                     hipStream_t st) {
  switch (s.D) {
    case 32: return qkv_fused_d<T, 32>(s, x, q, k, v, ep, wt, st);
    case 64: return qkv_fused_d<T, 64>(s, x, q, k, v, ep, wt, st);
    case 128: return qkv_fused_d<T, 128>(s, x, q, k, v, ep, wt, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int NT>
hipError_t out_launch(const Shape& s, const void* o, const void* wo, void* delta, void* wt, hipStream_t st) {
  const int M = s.B * s.S, Nm = s.W, Kd = s.H * s.D;
  HeadMap hm{s.S, s.H, s.D};
  const QkvEpilogue none{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const T* t = (const T*)wt + 3 * (size_t)Kd * s.W;  // Wo transposed, after the three projection weights
  if (M >= kBigM)
    hipLaunchKernelGGL((k_mm<T, 128, NT, true, false, 0>), dim3((M + 127) / 128, Nm / NT), dim3(256), 0, st,
                       (const T*)o, t, t, t, (T*)delta, (T*)delta, (T*)delta, M, Nm, Kd, hm, none, s);
  else
    hipLaunchKernelGGL((k_mm<T, 64, NT, true, false, 0>), dim3((M + 63) / 64, Nm / NT), dim3(256), 0, st,
                       (const T*)o, t, t, t, (T*)delta, (T*)delta, (T*)delta, M, Nm, Kd, hm, none, s);
  return hipGetLastError();
}

template <typename T>
hipError_t project_heads(const Shape& s, const void* x, const void* w, void* out, bool rope, hipStream_t st) {
  const int M = s.B * s.S, N = s.H * s.D, Kd = s.W;
  HeadMap hm{s.S, s.H, s.D};
  hipLaunchKernelGGL((k_gemm<T, false, true>), dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, st, (const T*)x,
                     (const T*)w, (T*)out, M, N, Kd, hm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !rope) return e;
  const long long rows = (long long)s.B * s.H * s.S;
  long long blocks = (rows * (s.D / 2) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((k_rope<T>), dim3((unsigned)blocks), dim3(256), 0, st, (T*)out, rows, s.S, s.D,
                     (double)s.rope_base);
  return hipGetLastError();
}

template <typename T>
hipError_t project_out(const Shape& s, const void* o, const void* wo, void* delta, void* wt, hipStream_t st) {
  switch (wt ? mm_tile(s.W, 0, false) : 0) {
    case 128: return out_launch<T, 128>(s, o, wo, delta, wt, st);
    case 64: return out_launch<T, 64>(s, o, wo, delta, wt, st);
    case 32: return out_launch<T, 32>(s, o, wo, delta, wt, st);
    default: break;
  }
  const int M = s.B * s.S, N = s.W, Kd = s.H * s.D;
  HeadMap hm{s.S, s.H, s.D};
  hipLaunchKernelGGL((k_gemm<T, true, false>), dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, st, (const T*)o,
                     (const T*)wo, (T*)delta, M, N, Kd, hm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project_heads(const Shape& s, const void* x, const void* w, void* out, bool rope, hipStream_t st) {
  if (s.dtype == MDR_BF16) return project_heads<bf16>(s, x, w, out, rope, st);
  return project_heads<float>(s, x, w, out, rope, st);
}

bool qkv_fuses_address(const Shape& s) { return s.blk <= 64 && s.W % 8 == 0 && mm_tile(s.H * s.D, s.D, true) > 0; }

hipError_t launch_qkv_fused(const Shape& s, const void* x, void* q, void* k, void* v, const float* cb,
                            const float* bias, float* ksum, int32_t* addr, int32_t* alt, int32_t* pair_zero,
                            const void* wt, hipStream_t st, float* amargin) {
  if (!qkv_fuses_address(s)) return hipErrorInvalidValue;
  const QkvEpilogue ep{cb, bias, ksum, addr, alt, pair_zero, amargin};
  if (s.dtype == MDR_BF16) return qkv_fused<bf16>(s, x, q, k, v, ep, wt, st);
  return qkv_fused<float>(s, x, q, k, v, ep, wt, st);
}

bool project_out_tiled(const Shape& s) { return mm_tile(s.W, 0, false) != 0; }

hipError_t launch_transpose_weights(const Shape& s, const void* wq, const void* wk, const void* wv, const void* wo,
                                    void* wt, int first, int count, hipStream_t st) {
  if (s.dtype == MDR_BF16) return transpose_weights<bf16>(s, wq, wk, wv, wo, wt, first, count, st);
  return transpose_weights<float>(s, wq, wk, wv, wo, wt, first, count, st);
}

hipError_t launch_project_out(const Shape& s, const void* o, const void* wo, void* delta, void* wt, hipStream_t st) {
  if (s.dtype == MDR_BF16) return project_out<bf16>(s, o, wo, delta, wt, st);
  return project_out<float>(s, o, wo, delta, wt, st);
}

}  // namespace mdr
