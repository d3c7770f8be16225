// Streaming decode of Monodratic routed attention: posting lists kept as ring buffers, fed one
// block at a time, and the routing + exact softmax of a few new tokens against a K/V cache.
//
// The pages name incremental routing updates for decoding as the open systems question (remio.ai,
// "What sparse attention researchers should watch next"), and bound every posting list by a
// strict capacity with overflow dropping blocks ("Monodratic turns sparse attention into a
// retrieval decision").  A ring buffer of `capacity` entries per address, fed block i once it is
// eligible (for query block i + L) and evicting its oldest entry when full, holds exactly the
// newest `capacity` eligible blocks of that address: the view the prefill path reads from its
// lists.  So decoding a token reproduces the prefill routing of that token, and its output is the
// same exact softmax over the selected blocks plus the L local blocks (aitechinspire.com,
// "Snapshot: key facts from the report").
//
//   k_dec_file    one work-group per (b,h): summarise (if needed) and file the newly eligible
//                 blocks into the rings, counting evictions.
//   k_dec_attend  one work-group per (b,h, new token): probe logits, top-P addresses, the ring
//                 views in probe order (cut at M), rerank by <q, summary>, top-R (+ forced
//                 target), then one softmax over the selected remote blocks and the local window.
#include "mdr_address.h"
#include "mdr_internal.h"

#include <type_traits>

namespace mdr {
namespace {

constexpr float kLog2eDec = 1.4426950408889634f;

template <typename T, int D>
__global__ __launch_bounds__(256) void k_dec_file(const T* __restrict__ K, const float* __restrict__ cb,
                                                  const float* __restrict__ bias, DecState d, int target,
                                                  Shape s) {
  __shared__ AddressLds<T, D> sm;
  __shared__ int summ_s, filed_s;
  const int bh = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    summ_s = d.summarized[bh];
    filed_s = d.filed[bh];
  }
  __syncthreads();
  const int summ = summ_s, filed = filed_s;  // uniform
  for (int i = filed; i < target; ++i) {
    if (i >= summ) block_address<T, D>(K, cb, bias, d.ksum, d.addr, i, bh, sm, s);
    __syncthreads();
    if (tid == 0) {
      const int a = d.addr[(size_t)bh * s.nb + i];
      int32_t* rec = d.ring + ((size_t)bh * s.A + a) * (s.cap + 1);
      const int n = rec[0];
      rec[1 + n % s.cap] = i;
      rec[0] = n + 1;
      if (n >= s.cap) d.overflow[bh] += 1;
    }
  }
  if (tid == 0) {
    d.summarized[bh] = max(summ, target);
    d.filed[bh] = max(filed, target);
  }
}

// Every ring record to (0 filed, empty slots).
__global__ __launch_bounds__(256) void k_ring_reset(int32_t* ring, long long records, int cap) {
  const long long n = records * (cap + 1);
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n; x += (long long)gridDim.x * 256)
    ring[x] = x % (cap + 1) == 0 ? 0 : -1;
}

// (value, index) as one 64-bit key ordered by value descending, then index ascending.
__device__ inline uint64_t dec_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ inline int dec_key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// Insert x into top[0..n) (sorted, best first) of capacity K; returns the new length.
__device__ inline int dec_insert(uint64_t* top, int n, int K, uint64_t x) {
  if (n == K && x <= top[K - 1]) return n;
  int pos = n < K ? n : K - 1;
  while (pos > 0 && top[pos - 1] < x) {
    top[pos] = top[pos - 1];
    --pos;
  }
  top[pos] = x;
  return n < K ? n + 1 : n;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_dec_attend(const T* __restrict__ Qn, const T* __restrict__ K,
                                                    const T* __restrict__ V, const float* __restrict__ cb,
                                                    const float* __restrict__ bias, DecState d,
                                                    const int32_t* __restrict__ force, int pos, int n_new,
                                                    T* __restrict__ out, int32_t* __restrict__ sel_out,
                                                    Shape s) {
  constexpr int LPC = 256 / kMaxCodesTotal;  // lanes per code logit
  constexpr int DPL = D / LPC;
  constexpr int KG = 16;      // key groups in the weighted sum of V
  constexpr int DL = D / 16;  // dims per lane there (16 lanes cover a row)
  constexpr int VK = 16;      // keys per lane whose V rows are requested before the softmax
  constexpr int RECMAX = kMaxProbes * 17;
  __shared__ float qs[D];
  __shared__ float mu[kMaxCodesTotal];
  __shared__ int probes[kMaxProbes];
  __shared__ int pstart[kMaxProbes + 1];
  __shared__ int rec[RECMAX];  // the probed addresses' ring records (when capacity <= 16)
  __shared__ int cand[kDecMaxCand];
  __shared__ float rho[kDecMaxCand];
  __shared__ int selb[kMaxRemote];
  __shared__ int nsel_s;
  __shared__ float sc[kDecMaxKeys];
  __shared__ float part[KG][D];
  __shared__ float wred[4];
  // thread 0's selection lists (LDS rather than scratch)
  __shared__ int tcode[kMaxSubspaces][kMaxProbes];
  __shared__ float tval[kMaxSubspaces][kMaxProbes];
  __shared__ uint64_t best[kMaxProbes];
  __shared__ uint64_t vkey[256];
  const int ti = blockIdx.x, bh = blockIdx.y, h = bh % s.H;
  const int t = pos + ti, j = t / s.blk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int GC = s.G * s.C;
  const size_t qrow = (size_t)bh * n_new + ti;
  // the query row and this lane's codebook slice (code cc, dims [pl·DPL, (pl+1)·DPL)) together
  const int cc = tid / LPC, pl = tid % LPC;
  float w[DPL];
  {
    const float* wr = cb + ((size_t)h * GC + (cc < GC ? cc : 0)) * D + pl * DPL;
#pragma unroll
    for (int x = 0; x < DPL; ++x) w[x] = wr[x];
  }
  const float bv = (bias && cc < GC) ? bias[h * GC + cc] : 0.f;
  if (tid < D) qs[tid] = (float)Qn[qrow * D + tid];
  __syncthreads();
  // ---- probe logits mu[g, c] = <codebook[h, g, c], q> + bias: four adjacent lanes per code
  {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc = fmaf(w[x], qs[pl * DPL + x], acc);
#pragma unroll
    for (int x = 1; x < LPC; x <<= 1) acc += __shfl_xor(acc, x);
    if (pl == 0 && cc < GC) mu[cc] = acc + bv;
  }
  __syncthreads();
  // ---- top-P addresses by (sum_g mu[g, c_g] desc, address asc).  Only the top-min(P, C) codes of
  // a subspace can take part, and only rank vectors with prod (k_g + 1) <= P (each is beaten by
  // prod (k_g + 1) - 1 others).  Wave g ranks subspace g's codes (a code's rank = the number of
  // codes with a larger key); one thread per rank vector scores it; a vector's rank among the
  // scored ones places it.  Keys are distinct, so every rank is.
  const int PG = s.P < s.C ? s.P : s.C;
  if (tid < s.P) probes[tid] = -1;  // filled below (there are always at least P candidates)
  if (wave < s.G) {
    const int g = wave;
    const uint64_t key = lane < s.C ? dec_key(mu[g * s.C + lane], lane) : 0;
    int rank = 0;
    for (int o = 0; o < s.C; ++o) {
      const uint64_t ok = ((uint64_t)(uint32_t)__shfl((int)(key >> 32), o) << 32) | (uint32_t)__shfl((int)key, o);
      rank += ok > key;
    }
    if (lane < s.C && rank < PG) {
      tcode[g][rank] = lane;
      tval[g][rank] = mu[g * s.C + lane];
    }
  }
  __syncthreads();
  int nvec = 1;
  for (int g = 0; g < s.G; ++g) nvec *= PG;
  if (nvec <= 256) {
    uint64_t key = 0;
    if (tid < nvec) {
      int rem = tid, prod = 1;
      int rk[kMaxSubspaces];
      for (int g = s.G - 1; g >= 0; --g) {
        rk[g] = rem % PG;
        rem /= PG;
        prod *= rk[g] + 1;
      }
      if (prod <= s.P) {
        float sig = 0.f;
        int a = 0;
        for (int g = 0; g < s.G; ++g) {
          sig += tval[g][rk[g]];
          a = a * s.C + tcode[g][rk[g]];
        }
        key = dec_key(sig, a);
      }
    }
    vkey[tid] = key;
    __syncthreads();
    if (key != 0) {
      int rank = 0;
      for (int o = 0; o < nvec; ++o) rank += vkey[o] > key;
      if (rank < s.P) probes[rank] = dec_key_index(key);
    }
  } else if (tid == 0) {  // large rank spaces: depth-first over the vectors with prod <= P
    int nb = 0;
    int rk[kMaxSubspaces], prod[kMaxSubspaces + 1];
    int g = 0;
    rk[0] = -1;
    prod[0] = 1;
    while (g >= 0) {
      ++rk[g];
      if (rk[g] >= PG || prod[g] * (rk[g] + 1) > s.P) {
        --g;
        continue;
      }
      prod[g + 1] = prod[g] * (rk[g] + 1);
      if (g + 1 < s.G) {
        ++g;
        rk[g] = -1;
        continue;
      }
      float sig = 0.f;
      int a = 0;
      for (int q = 0; q < s.G; ++q) {
        sig += tval[q][rk[q]];
        a = a * s.C + tcode[q][rk[q]];
      }
      nb = dec_insert(best, nb, s.P, dec_key(sig, a));
    }
    for (int p = 0; p < s.P; ++p) probes[p] = dec_key_index(best[p]);
  }
  __syncthreads();
  // ---- the probed rings (count, then slots) in one read each; views in probe rank order, newest
  // first, cut at M
  const int RL = s.cap + 1;
  const bool rec_lds = s.P * RL <= RECMAX;  // uniform
  auto ring_of = [&](int p) -> const int32_t* { return d.ring + ((size_t)bh * s.A + max(probes[p], 0)) * RL; };
  if (rec_lds)
    for (int x = tid; x < s.P * RL; x += 256) rec[x] = probes[x / RL] < 0 ? 0 : ring_of(x / RL)[x % RL];
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int p = 0; p < s.P; ++p) {
      pstart[p] = run;
      const int n = probes[p] < 0 ? 0 : rec_lds ? rec[p * RL] : ring_of(p)[0];
      run = min(s.M, run + min(n, s.cap));
    }
    pstart[s.P] = run;
  }
  __syncthreads();
  const int ncand = pstart[s.P];
  for (int x = tid; x < s.P * s.cap; x += 256) {
    const int p = x / s.cap, e = x % s.cap;
    const int k = pstart[p] + e;
    if (k < pstart[p + 1]) {
      const int32_t* r = rec_lds ? rec + p * RL : ring_of(p);
      const int n = r[0];
      cand[k] = r[1 + (n - 1 - e) % s.cap];
    }
  }
  __syncthreads();
  // ---- rerank scores <q, summary>: four adjacent lanes per candidate, lane ql taking dims
  // 16c + 4ql + e in that order, then xor 1 and xor 2 (the prefill probe's order)
  {
    const int ql = tid & 3;
    const float* ks = d.ksum + (size_t)bh * s.nb * D;
    for (int k = tid >> 2; k < ncand; k += 64) {
      const float* kr = ks + (size_t)cand[k] * D + 4 * ql;
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const float4 kv = *(const float4*)(kr + 16 * c);
        a = fmaf(kv.x, qs[16 * c + 4 * ql], a);
        a = fmaf(kv.y, qs[16 * c + 4 * ql + 1], a);
        a = fmaf(kv.z, qs[16 * c + 4 * ql + 2], a);
        a = fmaf(kv.w, qs[16 * c + 4 * ql + 3], a);
      }
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      if (ql == 0) rho[k] = a;
    }
  }
  __syncthreads();
  // ---- top-R by (score desc, block asc): a candidate's rank is the number of candidates with a
  // larger key (blocks are distinct, so ranks are); then the forced target under the same budget
  for (int k = tid; k < ncand; k += 256) {
    const uint64_t key = dec_key(rho[k], cand[k]);
    int rank = 0;
    for (int o = 0; o < ncand; ++o) rank += dec_key(rho[o], cand[o]) > key;
    if (rank < s.R) selb[rank] = cand[k];
  }
  __syncthreads();
  if (tid == 0) {
    int nr = min(ncand, s.R);
    if (force && s.R > 0) {
      const int f = force[qrow];
      if (f >= 0 && f <= j - s.L) {
        bool present = false;
        for (int r = 0; r < nr; ++r) present |= selb[r] == f;
        if (!present) {
          if (nr < s.R)
            selb[nr++] = f;
          else
            selb[s.R - 1] = f;
        }
      }
    }
    nsel_s = nr;
    if (sel_out)
      for (int r = 0; r < s.R; ++r) sel_out[qrow * s.R + r] = r < nr ? selb[r] : -1;
  }
  __syncthreads();
  // ---- one softmax over the selected remote blocks and the local window (causal up to t)
  const int nsel = nsel_s;
  const int nrk = nsel * s.blk;
  const int lo = max(0, j - s.L + 1) * s.blk;
  const int nkeys = nrk + (t - lo + 1);
  const float c = s.scale * kLog2eDec;
  const size_t rowbase = (size_t)bh * s.S;
  auto key_token = [&](int k) -> int { return k < nrk ? selb[k / s.blk] * s.blk + k % s.blk : lo + (k - nrk); };
  // V rows of this lane's first VK keys (group kg = tid / 16 takes keys kg, kg + 16, ...) are requested
  // together with the K rows of the scores
  const int kg = tid >> 4, l = tid & 15;
  float vv[VK][DL];
#pragma unroll
  for (int u = 0; u < VK; ++u) {
    const int k = kg + u * KG;
    const T* vr = V + (rowbase + key_token(k < nkeys ? k : 0)) * D + l * DL;
#pragma unroll
    for (int x = 0; x < DL; ++x) vv[u][x] = to_f(vr[x]);
  }
  float mx = -INFINITY;
  for (int k = tid; k < nkeys; k += 256) {
    const T* kr = K + (rowbase + key_token(k)) * D;
    float a = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += Vec16<T>::n) {
      const typename Vec16<T>::type v = *(const typename Vec16<T>::type*)(kr + c0);
#pragma unroll
      for (int e = 0; e < Vec16<T>::n; ++e) a = fmaf(to_f(v[e]), qs[c0 + e], a);
    }
    sc[k] = a;
    mx = fmaxf(mx, a);
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
  if (lane == 0) wred[wave] = mx;
  __syncthreads();
  mx = c * fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  __syncthreads();
  float sum = 0.f;
  for (int k = tid; k < nkeys; k += 256) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sc[k], c, -mx));
    sc[k] = p;
    sum += p;
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) sum += __shfl_xor(sum, x);
  if (lane == 0) wred[wave] = sum;
  __syncthreads();
  const float total = (wred[0] + wred[1]) + (wred[2] + wred[3]);
  // o[d] = sum_k p_k V[k][d]: lane l of group kg holds dims [l·D/16, (l+1)·D/16) for keys kg, kg + 16,
  // ...; the group partials are then added in group order
  {
    float acc[DL];
#pragma unroll
    for (int x = 0; x < DL; ++x) acc[x] = 0.f;
#pragma unroll
    for (int u = 0; u < VK; ++u) {
      const int k = kg + u * KG;
      const float p = k < nkeys ? sc[k] : 0.f;
#pragma unroll
      for (int x = 0; x < DL; ++x) acc[x] = fmaf(p, vv[u][x], acc[x]);
    }
    for (int k = kg + VK * KG; k < nkeys; k += KG) {
      const T* vr = V + (rowbase + key_token(k)) * D + l * DL;
      const float p = sc[k];
#pragma unroll
      for (int x = 0; x < DL; ++x) acc[x] = fmaf(p, to_f(vr[x]), acc[x]);
    }
#pragma unroll
    for (int x = 0; x < DL; ++x) part[kg][l * DL + x] = acc[x];
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < KG; ++g) o += part[g][tid];
    out[qrow * D + tid] = (T)(o / total);
  }
}

template <typename T>
hipError_t dec_file_t(const Shape& s, const void* k, const float* cb, const float* bias, const DecState& d,
                      int target, hipStream_t st) {
  dim3 grid(s.B * s.H);
  switch (s.D) {
    case 32: hipLaunchKernelGGL((k_dec_file<T, 32>), grid, dim3(256), 0, st, (const T*)k, cb, bias, d, target, s); break;
    case 64: hipLaunchKernelGGL((k_dec_file<T, 64>), grid, dim3(256), 0, st, (const T*)k, cb, bias, d, target, s); break;
    case 128: hipLaunchKernelGGL((k_dec_file<T, 128>), grid, dim3(256), 0, st, (const T*)k, cb, bias, d, target, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dec_attend_t(const Shape& s, const void* q, const void* k, const void* v, const float* cb,
                        const float* bias, const DecState& d, const int32_t* force, int pos, int n_new, void* out,
                        int32_t* sel, hipStream_t st) {
  dim3 grid(n_new, s.B * s.H);
#define MDR_DEC(DD)                                                                                              \
  hipLaunchKernelGGL((k_dec_attend<T, DD>), grid, dim3(256), 0, st, (const T*)q, (const T*)k, (const T*)v, cb, \
                     bias, d, force, pos, n_new, (T*)out, sel, s)
  switch (s.D) {
    case 32: MDR_DEC(32); break;
    case 64: MDR_DEC(64); break;
    case 128: MDR_DEC(128); break;
    default: return hipErrorInvalidValue;
  }
#undef MDR_DEC
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_reset(int32_t* ring, long long records, int cap, hipStream_t st) {
  long long blocks = (records * (cap + 1) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_ring_reset, dim3((unsigned)blocks), dim3(256), 0, st, ring, records, cap);
  return hipGetLastError();
}

hipError_t launch_decode_file(const Shape& s, const void* k_cache, const float* codebook, const float* bias,
                              const DecState& d, int target, hipStream_t st) {
  if (s.dtype == MDR_BF16) return dec_file_t<bf16>(s, k_cache, codebook, bias, d, target, st);
  return dec_file_t<float>(s, k_cache, codebook, bias, d, target, st);
}

hipError_t launch_decode_attend(const Shape& s, const void* q_new, const void* k_cache, const void* v_cache,
                                const float* codebook, const float* bias, const DecState& d,
                                const int32_t* force, int pos, int n_new, void* out, int32_t* sel,
                                hipStream_t st) {
  if (s.dtype == MDR_BF16)
    return dec_attend_t<bf16>(s, q_new, k_cache, v_cache, codebook, bias, d, force, pos, n_new, out, sel, st);
  return dec_attend_t<float>(s, q_new, k_cache, v_cache, codebook, bias, d, force, pos, n_new, out, sel, st);
}

}  // namespace mdr
