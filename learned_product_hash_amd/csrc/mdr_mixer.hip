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
#include "mdr_internal.h"

#include <type_traits>

namespace mdr {

namespace {

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
hipError_t project_out(const Shape& s, const void* o, const void* wo, void* delta, hipStream_t st) {
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

hipError_t launch_project_out(const Shape& s, const void* o, const void* wo, void* delta, hipStream_t st) {
  if (s.dtype == MDR_BF16) return project_out<bf16>(s, o, wo, delta, st);
  return project_out<float>(s, o, wo, delta, st);
}

}  // namespace mdr
