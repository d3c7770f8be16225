// Routing kernels of Monodratic routed sparse causal attention on gfx950:
//   k_address        block key summaries and product addresses
//   k_post           causal posting lists (histogram, wavefront scan, stable scatter) + overflow
//   k_probe_rerank   per query token: probe scores, top-P addresses, candidate views,
//                    rerank against the block summaries, top-R selection (+ forced target)
//
// The method (remio.ai, "Monodratic claims learned routing can make sparse causal attention
// more selective", section "Monodratic turns sparse attention into a retrieval decision";
// aitechinspire.com write-up, "Snapshot: key facts from the report"): after RoPE each source
// block receives a product address that combines the decisions of several learned code
// components; the address points to a bounded posting list; a query probes addresses,
// collects candidates, reranks them and keeps a fixed number of remote blocks.  A block may
// never be visible to a query placed before it.
#include "mdr_internal.h"

#include <float.h>

namespace mdr {

namespace {

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

// ---------------------------------------------------------------------------------------------
// Block key summary (mean of the block's key rows, fp32) and product address.
// One work-group of 256 threads per (b,h, block).  Each thread sums a fixed set of rows of one
// 16-byte column chunk; the row groups are then added in a fixed order, so the result is
// deterministic.  Codes are argmaxes of <codebook[h,g,c], summary> + bias[h,g,c] (first
// maximum wins), the address is the mixed-radix number with subspace 0 most significant.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_address(const T* __restrict__ K, const float* __restrict__ cb,
                                                 const float* __restrict__ bias, float* __restrict__ ksum,
                                                 int32_t* __restrict__ addr, int32_t* __restrict__ cnt_zero,
                                                 Shape s) {
  constexpr int VEC = Vec16<T>::n;
  constexpr int NCH = D / VEC;
  constexpr int RG = 256 / NCH;
  __shared__ float red[RG][D + 1];
  __shared__ float kbar[D];
  __shared__ float logit[kMaxCodesTotal];
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % s.H;
  const T* base = K + ((size_t)bh * s.S + (size_t)i * s.blk) * D;
  const int ch = tid % NCH, rg = tid / NCH;
  float part[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[e] = 0.f;
  for (int r = rg; r < s.blk; r += RG) {
    typename Vec16<T>::type v = *(const typename Vec16<T>::type*)(base + (size_t)r * D + ch * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) part[e] += to_f(v[e]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rg][ch * VEC + e] = part[e];
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    for (int g = 0; g < RG; ++g) acc += red[g][tid];
    const float m = acc / (float)s.blk;
    kbar[tid] = m;
    ksum[((size_t)bh * s.nb + i) * D + tid] = m;
  }
  __syncthreads();
  const int GC = s.G * s.C;
  if (tid < GC) {
    const float* w = cb + ((size_t)h * GC + tid) * D;
    float acc = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = fmaf(w[d], kbar[d], acc);
    if (bias) acc += bias[h * GC + tid];
    logit[tid] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    for (int g = 0; g < s.G; ++g) {
      int best = 0;
      float bv = logit[g * s.C];
      for (int c = 1; c < s.C; ++c) {
        const float v = logit[g * s.C + c];
        if (v > bv) {
          bv = v;
          best = c;
        }
      }
      a = a * s.C + best;
    }
    addr[(size_t)bh * s.nb + i] = a;
    if (cnt_zero) cnt_zero[(size_t)bh * s.nb + i] = 0;
  }
}

// ---------------------------------------------------------------------------------------------
// Posting lists of one (b,h) as CSR.  Blocks i < nb - L are filed (the last L blocks are never
// visible to any query of this sequence).  Histogram with LDS atomics, exclusive scan over the
// A addresses, then a stable counting-sort scatter by wave 0: per 64-block chunk each lane finds
// the lanes holding the same address with a ballot per address bit, so its slot is the number
// of earlier equal lanes plus the running cursor of that address.  Blocks therefore appear in
// ascending order within each list.  overflow = sum_a max(0, n_a - capacity).
__global__ __launch_bounds__(256) void k_post(const int32_t* __restrict__ addr, int32_t* __restrict__ off,
                                              int32_t* __restrict__ idx, int32_t* __restrict__ overflow,
                                              Shape s) {
  __shared__ int hist[kMaxAddresses];
  __shared__ int part[256];
  __shared__ int ovf[256];
  __shared__ int total;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int A = s.A;
  const int n_elig = s.nb > s.L ? s.nb - s.L : 0;
  const int32_t* ad = addr + (size_t)bh * s.nb;
  for (int a = tid; a < A; a += 256) hist[a] = 0;
  __syncthreads();
  for (int i = tid; i < n_elig; i += 256) {
    const int a = ad[i];
    if (a >= 0 && a < A) atomicAdd(&hist[a], 1);  // out-of-range addresses are not filed
  }
  __syncthreads();
  // exclusive scan: thread tid owns the contiguous address segment [a0, a1)
  const int seg = (A + 255) / 256;
  const int a0 = min(A, tid * seg), a1 = min(A, a0 + seg);
  int sum = 0, over = 0;
  for (int a = a0; a < a1; ++a) {
    sum += hist[a];
    over += max(0, hist[a] - s.cap);
  }
  part[tid] = sum;
  ovf[tid] = over;
  __syncthreads();
  if (tid == 0) {
    int run = 0, tot = 0;
    for (int w = 0; w < 256; ++w) {
      const int v = part[w];
      part[w] = run;
      run += v;
      tot += ovf[w];
    }
    overflow[bh] = tot;
    off[(size_t)bh * (A + 1) + A] = run;
    total = run;
  }
  __syncthreads();
  {
    int run = part[tid];
    for (int a = a0; a < a1; ++a) {
      const int v = hist[a];
      off[(size_t)bh * (A + 1) + a] = run;
      hist[a] = run;  // becomes the scatter cursor of address a
      run += v;
    }
  }
  __syncthreads();
  int32_t* out = idx + (size_t)bh * s.nb;
  if (tid < kWave) {
    const int lane = tid;
    int nbits = 0;
    while ((1 << nbits) < A) ++nbits;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < n_elig; c0 += kWave) {
      const int i = c0 + lane;
      int a = i < n_elig ? ad[i] : -1;
      const bool valid = a >= 0 && a < A;
      if (!valid) a = 0;
      unsigned long long same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (a >> b) & 1;
        const unsigned long long m1 = __ballot(bit);
        same &= bit ? m1 : ~m1;
      }
      if (valid) {
        const int rank = __popcll(same & lt);
        const int count = __popcll(same);
        const int cur = hist[a];
        out[cur + rank] = i;
        __builtin_amdgcn_wave_barrier();
        if (rank == count - 1) hist[a] = cur + count;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int i = total + tid; i < s.nb; i += 256) out[i] = -1;
}

// ---------------------------------------------------------------------------------------------
// Probe + rerank, one lane per query token, one wave per work-group (per-lane scratch lives in
// LDS, laid out [slot][lane] so lanes never conflict).
//   mu[g,c]   = <codebook[h,g,c], q_t> + bias[h,g,c]
//   probes    = top-P addresses by sigma(a) = sum_g mu[g, c_g(a)] (summed in subspace order),
//               ties to the smaller address.  Only the top-min(P,C) codes of each subspace can
//               take part in a top-P address (any other code is beaten by P addresses that swap
//               it for a better code of the same subspace), so those combinations are scored.
//   candidates= for each probe in rank order, the newest `capacity` CSR entries <= j - L,
//               newest first, until M candidates
//   selection = top-R candidates by <q_t, summary_i>, ties to the smaller block
// Optionally the selected (token, slot) pairs are appended to per-block bins for the
// block-grouped attention (cnt must be zero on entry).
template <typename T, int D>
__global__ __launch_bounds__(64) void k_probe_rerank(const T* __restrict__ Q, const float* __restrict__ cb,
                                                     const float* __restrict__ bias,
                                                     const float* __restrict__ ksum,
                                                     const int32_t* __restrict__ off,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ force,
                                                     int32_t* __restrict__ sel, int32_t* __restrict__ ncand,
                                                     int32_t* __restrict__ cnt, int32_t* __restrict__ bins,
                                                     Shape s) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x;
  const int GC = s.G * s.C;
  const int P = s.P, R = s.R, C = s.C, G = s.G;
  float* mu = smem;                           // [GC][64]
  int* tc = (int*)(mu + GC * kWave);           // [G][P][64] top codes per subspace
  float* tpv = (float*)(tc + G * P * kWave);   // [P][64] top-P scores
  int* tpa = (int*)(tpv + P * kWave);          // [P][64] top-P addresses
  float* trv = (float*)(tpa + P * kWave);      // [R][64] top-R scores
  int* tri = (int*)(trv + R * kWave);          // [R][64] top-R blocks
  const int bh = blockIdx.y, h = bh % s.H;
  const int t = blockIdx.x * kWave + lane;
  if (t >= s.S) return;  // no barriers below
  const int j = t / s.blk;
  const int cutoff = j - s.L;

  float qv[D];
  {
    const T* qp = Q + ((size_t)bh * s.S + t) * D;
    constexpr int VEC = Vec16<T>::n;
#pragma unroll
    for (int c = 0; c < D / VEC; ++c) {
      typename Vec16<T>::type v = *(const typename Vec16<T>::type*)(qp + c * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[c * VEC + e] = to_f(v[e]);
    }
  }
  const float* cbh = cb + (size_t)h * GC * D;
  for (int gc = 0; gc < GC; ++gc) {
    const float* w = cbh + (size_t)gc * D;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = fmaf(w[d], qv[d], acc);
    if (bias) acc += bias[h * GC + gc];
    mu[gc * kWave + lane] = acc;
  }
  // top-min(P, C) codes of every subspace, by (mu desc, code asc)
  const int Pg = min(P, C);
  for (int g = 0; g < G; ++g) {
    float pv = FLT_MAX;
    int pc = -1;
    bool first = true;
    for (int p = 0; p < Pg; ++p) {
      int bc = -1;
      float bv = -FLT_MAX;
      for (int c = 0; c < C; ++c) {
        const float v = mu[(g * C + c) * kWave + lane];
        const bool after = first || (v < pv) || (v == pv && c > pc);
        if (after && (bc < 0 || v > bv)) {
          bc = c;
          bv = v;
        }
      }
      tc[(g * P + p) * kWave + lane] = bc;
      pv = bv;
      pc = bc;
      first = false;
    }
  }
  // score the Pg^G code combinations, keep the top-P addresses
  int ncomb = 1;
  for (int g = 0; g < G; ++g) ncomb *= Pg;
  int np = 0;
  for (int kc = 0; kc < ncomb; ++kc) {
    int code[kMaxSubspaces];
    int rem = kc;
#pragma unroll
    for (int g = kMaxSubspaces - 1; g >= 0; --g) {
      if (g < G) {
        code[g] = tc[(g * P + rem % Pg) * kWave + lane];
        rem /= Pg;
      }
    }
    float sig = mu[code[0] * kWave + lane];
    int a = code[0];
#pragma unroll
    for (int g = 1; g < kMaxSubspaces; ++g) {
      if (g < G) {
        sig += mu[(g * C + code[g]) * kWave + lane];
        a = a * C + code[g];
      }
    }
    int pos;
    if (np == P) {
      const float wv = tpv[(P - 1) * kWave + lane];
      const int wa = tpa[(P - 1) * kWave + lane];
      if (!(sig > wv || (sig == wv && a < wa))) continue;
      pos = P - 1;
    } else {
      pos = np++;
    }
    while (pos > 0) {
      const float pvv = tpv[(pos - 1) * kWave + lane];
      const int pa = tpa[(pos - 1) * kWave + lane];
      if (!(sig > pvv || (sig == pvv && a < pa))) break;
      tpv[pos * kWave + lane] = pvv;
      tpa[pos * kWave + lane] = pa;
      --pos;
    }
    tpv[pos * kWave + lane] = sig;
    tpa[pos * kWave + lane] = a;
  }
  // candidates in probe rank order, rerank by <q_t, summary>
  int nc = 0, nr = 0;
  if (cutoff >= 0 && R > 0) {
    const int32_t* offh = off + (size_t)bh * (s.A + 1);
    const int32_t* idxh = idx + (size_t)bh * s.nb;
    const float* ksh = ksum + (size_t)bh * s.nb * D;
    for (int p = 0; p < np && nc < s.M; ++p) {
      const int a = tpa[p * kWave + lane];
      const int lo = offh[a], hi = offh[a + 1];
      int l0 = lo, l1 = hi;  // first entry > cutoff
      while (l0 < l1) {
        const int mid = (l0 + l1) >> 1;
        if (idxh[mid] <= cutoff)
          l0 = mid + 1;
        else
          l1 = mid;
      }
      const int take = min(s.cap, l0 - lo);
      for (int e = 0; e < take && nc < s.M; ++e) {
        const int i = idxh[l0 - 1 - e];
        ++nc;
        const float4* kr = (const float4*)(ksh + (size_t)i * D);
        float rho = 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
          const float4 kv = kr[c];
          rho = fmaf(kv.x, qv[4 * c + 0], rho);
          rho = fmaf(kv.y, qv[4 * c + 1], rho);
          rho = fmaf(kv.z, qv[4 * c + 2], rho);
          rho = fmaf(kv.w, qv[4 * c + 3], rho);
        }
        int pos;
        if (nr == R) {
          const float wv = trv[(R - 1) * kWave + lane];
          const int wi = tri[(R - 1) * kWave + lane];
          if (!(rho > wv || (rho == wv && i < wi))) continue;
          pos = R - 1;
        } else {
          pos = nr++;
        }
        while (pos > 0) {
          const float pvv = trv[(pos - 1) * kWave + lane];
          const int pi = tri[(pos - 1) * kWave + lane];
          if (!(rho > pvv || (rho == pvv && i < pi))) break;
          trv[pos * kWave + lane] = pvv;
          tri[pos * kWave + lane] = pi;
          --pos;
        }
        trv[pos * kWave + lane] = rho;
        tri[pos * kWave + lane] = i;
      }
    }
  }
  if (force && R > 0) {
    const int f = force[(size_t)bh * s.S + t];
    if (f >= 0 && f <= cutoff) {
      bool present = false;
      for (int r = 0; r < nr; ++r) present |= (tri[r * kWave + lane] == f);
      if (!present) {
        if (nr < R)
          tri[(nr++) * kWave + lane] = f;
        else
          tri[(R - 1) * kWave + lane] = f;
      }
    }
  }
  int32_t* srow = sel + ((size_t)bh * s.S + t) * R;
  for (int r = 0; r < R; ++r) srow[r] = r < nr ? tri[r * kWave + lane] : -1;
  if (ncand) ncand[(size_t)bh * s.S + t] = nc;
  if (bins) {
    for (int r = 0; r < nr; ++r) {
      const int i = tri[r * kWave + lane];
      const int pos = atomicAdd(&cnt[(size_t)bh * s.nb + i], 1);
      if (pos < (s.nb - s.L - i) * s.blk)
        bins[(size_t)bh * s.bins_per_bh + bin_offset(i, s.nb, s.L, s.blk) + pos] = t * R + r;
    }
  }
}

template <typename T>
hipError_t address_dispatch(const Shape& s, const void* k, const float* cb, const float* bias, float* ksum,
                            int32_t* addr, int32_t* cnt, hipStream_t st) {
  dim3 grid(s.nb, s.B * s.H);
  switch (s.D) {
    case 32:
      hipLaunchKernelGGL((k_address<T, 32>), grid, dim3(256), 0, st, (const T*)k, cb, bias, ksum, addr, cnt, s);
      break;
    case 64:
      hipLaunchKernelGGL((k_address<T, 64>), grid, dim3(256), 0, st, (const T*)k, cb, bias, ksum, addr, cnt, s);
      break;
    case 128:
      hipLaunchKernelGGL((k_address<T, 128>), grid, dim3(256), 0, st, (const T*)k, cb, bias, ksum, addr, cnt, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t probe_dispatch(const Shape& s, const void* q, const float* cb, const float* bias, const float* ksum,
                          const int32_t* off, const int32_t* idx, const int32_t* force, int32_t* sel,
                          int32_t* ncand, int32_t* cnt, int32_t* bins, hipStream_t st) {
  dim3 grid((s.S + kWave - 1) / kWave, s.B * s.H);
  const size_t lds = (size_t)(s.G * s.C + s.G * s.P + 2 * s.P + 2 * s.R) * kWave * 4;
  switch (s.D) {
    case 32:
      hipLaunchKernelGGL((k_probe_rerank<T, 32>), grid, dim3(kWave), lds, st, (const T*)q, cb, bias, ksum, off,
                         idx, force, sel, ncand, cnt, bins, s);
      break;
    case 64:
      hipLaunchKernelGGL((k_probe_rerank<T, 64>), grid, dim3(kWave), lds, st, (const T*)q, cb, bias, ksum, off,
                         idx, force, sel, ncand, cnt, bins, s);
      break;
    case 128:
      hipLaunchKernelGGL((k_probe_rerank<T, 128>), grid, dim3(kWave), lds, st, (const T*)q, cb, bias, ksum, off,
                         idx, force, sel, ncand, cnt, bins, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_address(const Shape& s, const void* k, const float* codebook, const float* bias, float* ksum,
                          int32_t* addr, int32_t* cnt_zero, hipStream_t st) {
  if (s.dtype == MDR_BF16) return address_dispatch<bf16>(s, k, codebook, bias, ksum, addr, cnt_zero, st);
  return address_dispatch<float>(s, k, codebook, bias, ksum, addr, cnt_zero, st);
}

hipError_t launch_post(const Shape& s, const int32_t* addr, int32_t* off, int32_t* idx, int32_t* overflow,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_post, dim3(s.B * s.H), dim3(256), 0, st, addr, off, idx, overflow, s);
  return hipGetLastError();
}

hipError_t launch_probe_rerank(const Shape& s, const void* q, const float* codebook, const float* bias,
                               const float* ksum, const int32_t* off, const int32_t* idx, const int32_t* force,
                               int32_t* sel, int32_t* ncand, int32_t* cnt, int32_t* bins, hipStream_t st) {
  if (s.dtype == MDR_BF16)
    return probe_dispatch<bf16>(s, q, codebook, bias, ksum, off, idx, force, sel, ncand, cnt, bins, st);
  return probe_dispatch<float>(s, q, codebook, bias, ksum, off, idx, force, sel, ncand, cnt, bins, st);
}

}  // namespace mdr
