// Routing kernels of Monodratic routed sparse causal attention on gfx950:
//   k_address        block key summaries and product addresses
//   k_post           causal posting lists (histogram, wavefront scan, stable scatter) + overflow
//   k_probe_rerank   per query token: probe scores, top-P addresses, candidate views,
//                    rerank against the block summaries, top-R selection (+ forced target)
//   k_probe_fixed    the same with the routing sizes fixed at compile time; it also builds the
//                    posting lists in LDS
// Both count the selected pairs per (token range, remote block) for the binning of the attention.
//
// The method (remio.ai, "Monodratic claims learned routing can make sparse causal attention
// more selective", section "Monodratic turns sparse attention into a retrieval decision";
// aitechinspire.com write-up, "Snapshot: key facts from the report"): after RoPE each source
// block receives a product address that combines the decisions of several learned code
// components; the address points to a bounded posting list; a query probes addresses,
// collects candidates, reranks them and keeps a fixed number of remote blocks.  A block may
// never be visible to a query placed before it.
#include "mdr_internal.h"
#include "mdr_address.h"

#include <float.h>

#include <type_traits>

namespace mdr {

namespace {

// ---------------------------------------------------------------------------------------------
// Block key summaries and product addresses: one work-group of 256 threads per (b,h) and NB adjacent
// blocks (blocks i0 + NB x .. of blockIdx.x = x, up to iend); the arithmetic is block_address()
// (mdr_address.h), shared with the decode path, and gives every block the same bits whatever NB.  The
// work-group also clears the pair counters' columns of its blocks when asked.
template <typename T, int D, int BLK, int NB>
__global__ __launch_bounds__(256) void k_address(const T* __restrict__ K, const float* __restrict__ cb,
                                                 const float* __restrict__ bias, float* __restrict__ ksum,
                                                 int32_t* __restrict__ addr, int32_t* __restrict__ pair_zero,
                                                 int32_t* __restrict__ alt, float* __restrict__ amargin, int i0,
                                                 int iend, Shape s) {
  __shared__ AddressLds<T, D, NB> sm;
  const int i = i0 + blockIdx.x * NB;
  const int nv = min(NB, iend - i);
  const int bh = blockIdx.y;
  if (pair_zero)
    for (int b = 0; b < nv; ++b) clear_pair_counts(pair_zero, s, bh, i + b, threadIdx.x, 256);
  block_address<T, D, BLK, NB>(K, cb, bias, ksum, addr, i, bh, sm, s, alt, amargin, nv);
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
  __shared__ int ads[kMaxBlocks];  // this (b,h)'s addresses, read from global memory once
  __shared__ int part[4];
  __shared__ int total;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int A = s.A;
  const int n_elig = s.nb > s.L ? s.nb - s.L : 0;
  const int32_t* ad = addr + (size_t)bh * s.nb;
  for (int a = tid; a < A; a += 256) hist[a] = 0;
  for (int i = tid; i < n_elig; i += 256) ads[i] = ad[i];
  __syncthreads();
  for (int i = tid; i < n_elig; i += 256) {
    const int a = ads[i];
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
  int tot_over = 0, tot = 0;
  block_exclusive_scan<256>(over, part, &tot_over);
  int run = block_exclusive_scan<256>(sum, part, &tot);
  if (tid == 0) {
    overflow[bh] = tot_over;
    off[(size_t)bh * (A + 1) + A] = tot;
    total = tot;
  }
  for (int a = a0; a < a1; ++a) {
    const int v = hist[a];
    off[(size_t)bh * (A + 1) + a] = run;
    hist[a] = run;  // becomes the scatter cursor of address a
    run += v;
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
      int a = i < n_elig ? ads[i] : -1;
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
// Redirect lists of one (b,h), for the overflow policy that redirects.  The block at position k of
// list a leaves the primary view when the block y at position k + capacity becomes eligible (query
// block y + L) and then arrives in the redirect list of its alternate address.  A block evicts at
// most one other, so arrivals are indexed by the evicting block y and ordered by it; a stable
// counting sort by alternate address (one ballot per address bit, as in k_post) keeps that order
// within each list.  overflow = the drop policy's overflow minus the redirected blocks that fill
// spare slots of their lists at the last query block.
__global__ __launch_bounds__(256) void k_post_redirect(const int32_t* __restrict__ addr,
                                                       const int32_t* __restrict__ alt,
                                                       const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ idx, int32_t* __restrict__ roff,
                                                       int32_t* __restrict__ ridx, int32_t* __restrict__ rtime,
                                                       int32_t* __restrict__ overflow, Shape s) {
  extern __shared__ int rsm[];
  const int A = s.A, ne = s.ne;
  int* hist = rsm;         // [A] arrivals per address, then the scatter cursors
  int* key = hist + A;     // [ne] alternate address of the block evicted by block y (-1: none)
  int* evb = key + ne;     // [ne] the block evicted by block y
  __shared__ int part[4];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int32_t* offp = off + (size_t)bh * (A + 1);
  const int32_t* idxp = idx + (size_t)bh * s.nb;
  const int32_t* ad = addr + (size_t)bh * s.nb;
  const int32_t* al = alt + (size_t)bh * s.nb;
  for (int a = tid; a < A; a += 256) hist[a] = 0;
  for (int y = tid; y < ne; y += 256) key[y] = -1;
  __syncthreads();
  const int total = min(offp[A], ne);
  for (int q = tid; q < total; q += 256) {
    const int y = idxp[q];
    if (y < 0 || y >= ne) continue;
    const int a = ad[y];
    if (a < 0 || a >= A || q - s.cap < offp[a]) continue;
    const int x = idxp[q - s.cap];
    const int b = (x >= 0 && x < ne) ? al[x] : -1;
    if (b >= 0 && b < A) {
      key[y] = b;
      evb[y] = x;
      atomicAdd(&hist[b], 1);
    }
  }
  __syncthreads();
  const int seg = (A + 255) / 256;
  const int a0 = min(A, tid * seg), a1 = min(A, a0 + seg);
  int sum = 0, over = 0, shown = 0;
  for (int a = a0; a < a1; ++a) {
    const int np = offp[a + 1] - offp[a];
    sum += hist[a];
    over += max(0, np - s.cap);
    shown += min(max(0, s.cap - np), hist[a]);
  }
  int tot_over = 0, tot_shown = 0, tot = 0;
  block_exclusive_scan<256>(over, part, &tot_over);
  block_exclusive_scan<256>(shown, part, &tot_shown);
  int run = block_exclusive_scan<256>(sum, part, &tot);
  int32_t* ro = roff + (size_t)bh * (A + 1);
  if (tid == 0) {
    overflow[bh] = tot_over - tot_shown;
    ro[A] = tot;
  }
  for (int a = a0; a < a1; ++a) {
    const int v = hist[a];
    ro[a] = run;
    hist[a] = run;
    run += v;
  }
  __syncthreads();
  int32_t* oi = ridx + (size_t)bh * s.nb;
  int32_t* ot = rtime + (size_t)bh * s.nb;
  if (tid < kWave) {
    const int lane = tid;
    int nbits = 0;
    while ((1 << nbits) < A) ++nbits;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < ne; c0 += kWave) {
      const int y = c0 + lane;
      int k = y < ne ? key[y] : -1;
      const bool valid = k >= 0;
      if (!valid) k = 0;
      unsigned long long same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (k >> b) & 1;
        const unsigned long long m1 = __ballot(bit);
        same &= bit ? m1 : ~m1;
      }
      if (valid) {
        const int rank = __popcll(same & lt);
        const int count = __popcll(same);
        const int cur = hist[k];
        oi[cur + rank] = evb[y];
        ot[cur + rank] = y + s.L;
        __builtin_amdgcn_wave_barrier();
        if (rank == count - 1) hist[k] = cur + count;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int i = tot + tid; i < s.nb; i += 256) {
    oi[i] = -1;
    ot[i] = -1;
  }
}

// ---------------------------------------------------------------------------------------------
// Probe + rerank.  A work-group of kProbeThreads lanes handles as many consecutive query tokens of
// one (b,h), one token per lane for the ranking steps (per-lane scratch lives in LDS, laid out
// [slot][lane] so lanes never conflict):
//   mu[g,c]   = <codebook[h,g,c], q_t> + bias[h,g,c], for all tokens of the work-group at once on
//               MFMA (fp32 16x16x4; tokens as rows, codes as columns, subspaces padded to 16 codes)
//   probes    = top-P addresses by sigma(a) = sum_g mu[g, c_g(a)] (summed in subspace order), ties to
//               the smaller address.  With the codes of each subspace ranked by (mu desc, code asc),
//               an address whose subspace ranks are (k_0, .., k_{G-1}) is beaten by every address
//               with ranks k'_g <= k_g, i.e. by prod_g (k_g + 1) - 1 others, so only rank vectors
//               with prod_g (k_g + 1) <= P are scored.
//   candidates= for each probe in rank order, the newest `capacity` CSR entries <= j - L,
//               newest first, until M candidates
//   selection = top-R candidates by <q_t, summary_i>, ties to the smaller block
// Optionally the selected (token, slot) pairs are counted per (token range, remote block) for the
// binning of the attention.
template <typename T, int D>
__global__ __launch_bounds__(kProbeThreads) void k_probe_rerank(
    const T* __restrict__ Q, const float* __restrict__ cb, const float* __restrict__ bias,
    const float* __restrict__ ksum, const int32_t* __restrict__ off, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ force, int32_t* __restrict__ sel, int32_t* __restrict__ ncand,
    int32_t* __restrict__ phist, ProbeExtra ex, Shape s) {
  constexpr int NT = kProbeThreads;
  extern __shared__ __align__(16) float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.y, h = bh % s.H;
  const int tbase = blockIdx.x * NT;
  const int t = tbase + tid;
  const int C = s.C, G = s.G, P = s.P, R = s.R, A = s.A;
  const int CP = (C + 15) & ~15;
  const int MST = G * CP + 4;
  // with diagnostics one more address and candidate are ranked, for the margins at the boundaries: the
  // P + 1 best addresses come from the min(P + 1, C) best codes per subspace and the rank vectors with
  // prod (k_g + 1) <= P + 1
  const bool diag = ex.probes || ex.sel_score || ex.pmargin || ex.smargin;
  const int Pl = diag ? P + 1 : P;                   // rank-vector bound and address list length
  const int KPl = min(Pl, A);
  const int Rl = diag ? R + 1 : R;                   // candidate list length
  const int Pg = min(Pl, C);
  const int PgM = min(P + 1, C);                     // LDS is laid out for the diagnostics sizes
  float* mu = smem;                                  // [NT][MST]
  int* tcode = (int*)(mu + NT * MST);                // [G*PgM][NT]
  float* tpv = (float*)(tcode + G * PgM * NT);       // [P+1][NT]
  int* tpa = (int*)(tpv + (P + 1) * NT);             // [P+1][NT]
  float* trv = (float*)(tpa + (P + 1) * NT);         // [R+1][NT]
  int* tri = (int*)(trv + (R + 1) * NT);             // [R+1][NT]
  int* csr = tri + (R + 1) * NT;                     // off [A+1], idx [ne] when staged
  const int32_t* offp = off + (size_t)bh * (A + 1);
  const int32_t* idxp = idx + (size_t)bh * s.nb;
  if (s.csr_lds) {
    for (int k = tid; k <= A; k += NT) csr[k] = offp[k];
    for (int k = tid; k < s.ne; k += NT) csr[A + 1 + k] = idxp[k];
    offp = csr;
    idxp = csr + A + 1;
  }

  // ---- mu on MFMA.  Lane l supplies Q[token 16tt + l%16][d] and W[code 16ct + l%16][d] for
  // d = (l/16)(D/4) + kk (a fixed permutation of the contraction index) and receives
  // mu[token 16tt + 4(l/16) + k][code 16ct + l%16].
  {
    const int r16 = lane & 15, s4 = lane >> 4;
    float qa[4][D / 4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (wave * 64 + tt * 16 >= NT) break;
      int tq = tbase + wave * 64 + tt * 16 + r16;
      tq = tq < s.S ? tq : s.S - 1;
      const T* qp = Q + ((size_t)bh * s.S + tq) * D + s4 * (D / 4);
      constexpr int VEC = Vec16<T>::n;
#pragma unroll
      for (int c = 0; c < D / 4 / VEC; ++c) {
        typename Vec16<T>::type v = *(const typename Vec16<T>::type*)(qp + c * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) qa[tt][c * VEC + e] = to_f(v[e]);
      }
    }
    const float* cbh = cb + (size_t)h * G * C * D;
    for (int g = 0; g < G; ++g) {
      for (int ct = 0; ct < CP / 16; ++ct) {
        const int code = ct * 16 + r16;
        float wb[D / 4];
        if (code < C) {
          const float4* wp = (const float4*)(cbh + ((size_t)g * C + code) * D + s4 * (D / 4));
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            const float4 v = wp[c];
            wb[4 * c] = v.x;
            wb[4 * c + 1] = v.y;
            wb[4 * c + 2] = v.z;
            wb[4 * c + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < D / 4; ++c) wb[c] = 0.f;
        }
        const float bv = (bias && code < C) ? bias[(h * G + g) * C + code] : 0.f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (wave * 64 + tt * 16 >= NT) break;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < D / 4; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[tt][kk], wb[kk], acc, 0, 0, 0);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            mu[(wave * 64 + tt * 16 + 4 * s4 + k) * MST + g * CP + code] = acc[k] + bv;
        }
      }
    }
  }
  __syncthreads();
  const bool active = t < s.S;
  int nr = 0;
  if (active) {  // no barriers inside
  const int j = t / s.blk;
  const int cutoff = j - s.L;
  const float* mrow = mu + tid * MST;

  // ---- top-min(P, C) codes of every subspace, by (mu desc, code asc)
  for (int g = 0; g < G; ++g) {
    float pv = FLT_MAX;
    int pc = -1;
    for (int p = 0; p < Pg; ++p) {
      int bc = -1;
      float bv = -FLT_MAX;
      for (int c = 0; c < C; ++c) {
        const float v = mrow[g * CP + c];
        const bool after = (v < pv) || (v == pv && c > pc);
        if (after && (bc < 0 || v > bv)) {
          bc = c;
          bv = v;
        }
      }
      tcode[(g * Pg + p) * NT + tid] = bc;
      pv = bv;
      pc = bc;
    }
  }
  // ---- score the rank vectors with prod (k_g + 1) <= Pl, keep the top-Pl addresses
  int ncomb = 1;
  for (int g = 0; g < G; ++g) ncomb *= Pg;
  int np = 0;
  for (int kc = 0; kc < ncomb; ++kc) {
    int rk[kMaxSubspaces];
    int rem = kc, prod = 1;
#pragma unroll
    for (int g = kMaxSubspaces - 1; g >= 0; --g) {
      if (g < G) {
        rk[g] = rem % Pg;
        rem /= Pg;
        prod *= rk[g] + 1;
      }
    }
    if (prod > Pl) continue;
    int c0 = tcode[rk[0] * NT + tid];
    float sig = mrow[c0];
    int a = c0;
#pragma unroll
    for (int g = 1; g < kMaxSubspaces; ++g) {
      if (g < G) {
        const int cg = tcode[(g * Pg + rk[g]) * NT + tid];
        sig += mrow[g * CP + cg];
        a = a * C + cg;
      }
    }
    int pos;
    if (np == KPl) {
      const float wv = tpv[(KPl - 1) * NT + tid];
      const int wa = tpa[(KPl - 1) * NT + tid];
      if (!(sig > wv || (sig == wv && a < wa))) continue;
      pos = KPl - 1;
    } else {
      pos = np++;
    }
    while (pos > 0) {
      const float pvv = tpv[(pos - 1) * NT + tid];
      const int pa = tpa[(pos - 1) * NT + tid];
      if (!(sig > pvv || (sig == pvv && a < pa))) break;
      tpv[pos * NT + tid] = pvv;
      tpa[pos * NT + tid] = pa;
      --pos;
    }
    tpv[pos * NT + tid] = sig;
    tpa[pos * NT + tid] = a;
  }

  // ---- candidates in probe rank order (each probe's view: its newest `capacity` eligible
  // primaries, then, under the redirect policy, the newest arrivals of its redirect list while slots
  // remain), cut at M; rerank by <q_t, summary>.  Dropped candidates: per probe, the eligible
  // blocks the list holds beyond its capacity.
  int nc = 0, ndr = 0;
  if (cutoff >= 0) {
    float qv[D];
    if (R > 0) {
      const T* qp = Q + ((size_t)bh * s.S + t) * D;
      constexpr int VEC = Vec16<T>::n;
#pragma unroll
      for (int c = 0; c < D / VEC; ++c) {
        typename Vec16<T>::type v = *(const typename Vec16<T>::type*)(qp + c * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) qv[c * VEC + e] = to_f(v[e]);
      }
    }
    const float* ksh = ksum + (size_t)bh * s.nb * D;
    const int32_t* roffp = ex.roff ? ex.roff + (size_t)bh * (A + 1) : nullptr;
    const int32_t* ridxp = ex.roff ? ex.ridx + (size_t)bh * s.nb : nullptr;
    const int32_t* rtimep = ex.roff ? ex.rtime + (size_t)bh * s.nb : nullptr;
    auto consider = [&](int i) {
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
      if (nr == Rl) {
        const float wv = trv[(Rl - 1) * NT + tid];
        const int wi = tri[(Rl - 1) * NT + tid];
        if (!(rho > wv || (rho == wv && i < wi))) return;
        pos = Rl - 1;
      } else {
        pos = nr++;
      }
      while (pos > 0) {
        const float pvv = trv[(pos - 1) * NT + tid];
        const int pi = tri[(pos - 1) * NT + tid];
        if (!(rho > pvv || (rho == pvv && i < pi))) break;
        trv[pos * NT + tid] = pvv;
        tri[pos * NT + tid] = pi;
        --pos;
      }
      trv[pos * NT + tid] = rho;
      tri[pos * NT + tid] = i;
    };
    for (int p = 0; p < min(np, P); ++p) {
      const int a = tpa[p * NT + tid];
      const int lo = offp[a], hi = offp[a + 1];
      int l0 = lo, l1 = hi;  // first entry > cutoff
      while (l0 < l1) {
        const int mid = (l0 + l1) >> 1;
        if (idxp[mid] <= cutoff)
          l0 = mid + 1;
        else
          l1 = mid;
      }
      const int nprim = l0 - lo, tp = min(s.cap, nprim);
      const int take = min(tp, s.M - nc);  // with R = 0 the candidates are counted, not scored
      if (R > 0)
        for (int e = 0; e < take; ++e) consider(idxp[l0 - 1 - e]);
      else
        nc += take;
      int narr = 0;
      if (roffp) {
        const int rlo = roffp[a];
        int r0 = rlo, r1 = roffp[a + 1];  // first arrival after query block j
        while (r0 < r1) {
          const int mid = (r0 + r1) >> 1;
          if (rtimep[mid] <= j)
            r0 = mid + 1;
          else
            r1 = mid;
        }
        narr = r0 - rlo;
        const int taker = min(min(s.cap - tp, narr), s.M - nc);
        if (R > 0)
          for (int e = 0; e < taker; ++e) consider(ridxp[r0 - 1 - e]);
        else
          nc += taker;
      }
      // held: the primaries not redirected away (every block has an alternate when C > 1) plus arrivals
      ndr += max(0, (roffp && C > 1 ? tp : nprim) + narr - s.cap);
    }
  }
  const int nrank = nr;  // ranked candidates kept (up to Rl)
  nr = min(nr, R);
  int fslot = -1;        // the slot a forced block took
  if (force && R > 0) {
    const int f = force[(size_t)bh * s.S + t];
    if (f >= 0 && f <= cutoff) {
      bool present = false;
      for (int r = 0; r < nr; ++r) present |= (tri[r * NT + tid] == f);
      if (!present) {  // the forced block goes to its slot once the diagnostics have read the ranking
        fslot = nr < R ? nr : R - 1;
        if (nr < R) ++nr;
      }
    }
  }
  const size_t tt = (size_t)bh * s.S + t;
  if (diag) {
    if (ex.probes)
      for (int p = 0; p < P; ++p) ex.probes[tt * P + p] = tpa[p * NT + tid];
    float pm = INFINITY;
    for (int p = 0; p + 1 < np; ++p) pm = fminf(pm, tpv[p * NT + tid] - tpv[(p + 1) * NT + tid]);
    if (ex.pmargin) ex.pmargin[tt] = pm;
    float sm = INFINITY;
    for (int r = 0; r + 1 < nrank && r < R; ++r) sm = fminf(sm, trv[r * NT + tid] - trv[(r + 1) * NT + tid]);
    if (ex.smargin) ex.smargin[tt] = R > 0 ? sm : INFINITY;
    if (ex.sel_score)
      for (int r = 0; r < R; ++r)
        ex.sel_score[tt * R + r] = r >= nr ? -INFINITY : r == fslot ? NAN : trv[r * NT + tid];
  }
  if (fslot >= 0) tri[fslot * NT + tid] = force[(size_t)bh * s.S + t];
  int32_t* srow = sel + tt * R;
  for (int r = 0; r < R; ++r) srow[r] = r < nr ? tri[r * NT + tid] : -1;
  if (ncand) ncand[tt] = nc;
  if (ex.ndrop) ex.ndrop[tt] = ndr;
  }  // active
  if (!phist) return;  // uniform
  // ---- count the selected pairs of this work-group's token range per remote block (LDS histogram in the
  // place of mu when it fits)
  PairCounter<NT> pc{s.ne <= NT * MST ? (int*)mu : nullptr, phist + pair_counts_row(s, bh, tbase),
                     s.ne};
  pc.begin();
  for (int r = 0; r < nr; ++r) pc.add(tri[r * NT + tid]);
  pc.end();
}

// ---------------------------------------------------------------------------------------------
// The same probe + rerank with the routing sizes fixed at compile time (G subspaces of C codes,
// P probes, R remote blocks): every per-token list lives in registers, rank vectors are
// enumerated at compile time, and the top-P / top-R lists are kept sorted by an unrolled
// insertion network.  Semantics are identical to k_probe_rerank.
// (value, index) ranked by value descending then index ascending, as one unsigned 64-bit key: the
// high word is the float's bits made order-preserving, the low word the complemented index.  A
// larger key is a better entry, so every comparison is a single 64-bit compare.
__device__ inline uint64_t rank_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ inline float key_value(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}
__device__ inline int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// Keep top[0..K) sorted (best first) while inserting x; empty slots hold 0, below every real key.
template <int K>
__device__ inline void insert_key(uint64_t (&top)[K], uint64_t x) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool better = x > top[k];
    const uint64_t t = top[k];
    top[k] = better ? x : t;
    x = better ? t : x;
  }
}

// The same ranks with 32-bit keys: the value's order-preserving bits with the low B bits given to the
// complemented index.  One unsigned compare then ranks (value desc, index asc) exactly as long as no
// two ranked values agree above those B bits.  top[0..K) is kept sorted (best first, empty slots 0)
// by a median-of-three network: the new rank k is the median of the old ranks k and k-1 and x.
constexpr int key_bits(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}
__device__ inline uint32_t order_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // ~u if negative, else the sign bit set
}
template <int B>
__device__ inline uint32_t packed_key(float v, int idx) {
  constexpr uint32_t mask = (1u << B) - 1u;
  return (order_bits(v) & ~mask) | (mask - (uint32_t)idx);
}
template <int B>
__device__ inline int packed_index(uint32_t k) {
  constexpr uint32_t mask = (1u << B) - 1u;
  return (int)(mask - (k & mask));
}
__device__ inline uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <int K>
__device__ inline void insert_packed(uint32_t (&top)[K], uint32_t x) {
#pragma unroll
  for (int k = K - 1; k >= 1; --k) top[k] = med3_u32(top[k], x, top[k - 1]);
  top[0] = max(top[0], x);
}
// The first K-1 packed ranks are the exact ones when no two neighbours among the K kept keys share
// their value bits (so that every one of them is alone in its group of equal truncated values).
template <int K, int B>
__device__ inline bool packed_exact(const uint32_t (&top)[K]) {
  bool ok = true;
#pragma unroll
  for (int k = 0; k + 1 < K; ++k) ok &= top[k + 1] == 0u || ((top[k] ^ top[k + 1]) >> B) != 0u;
  return ok;
}

template <int G, int PG>
struct RankSpace {
  static constexpr int count() {
    int n = 1;
    for (int g = 0; g < G; ++g) n *= PG;
    return n;
  }
};

// Posting lists of one (b,h) built in LDS from its block addresses ads[0..ne) (the filed blocks),
// with the semantics of k_post: counts per address, exclusive offsets, then a stable scatter by
// wave 0 (per 64-block chunk a lane's slot is the number of earlier lanes with the same address,
// found with one ballot per address bit, plus that address's running cursor), so each list holds
// its blocks in ascending order.  cur [A] is scratch.  Ends with a barrier.  When `publish`, the
// work-group also writes the CSR (with -1 beyond the filed entries) and the overflow count.
template <int NT>
__device__ void build_posting_csr(const int* ads, int* cur, int* offl, int* idxl, const Shape& s, int bh,
                                  bool publish, const FusedPost& fp) {
  const int tid = threadIdx.x;
  const int A = s.A, ne = s.ne;
  for (int a = tid; a <= A; a += NT) offl[a] = 0;
  lds_barrier();
  for (int i = tid; i < ne; i += NT) {
    const int a = ads[i];
    if (a >= 0 && a < A) atomicAdd(&offl[a], 1);
  }
  lds_barrier();
  // thread tid owns the contiguous address segment [a0, a1)
  __shared__ int part[NT / 64];
  const int seg = (A + NT - 1) / NT;
  const int a0 = min(A, tid * seg), a1 = min(A, a0 + seg);
  int sum = 0, over = 0;
  for (int a = a0; a < a1; ++a) {
    const int n = offl[a];
    sum += n;
    over += max(0, n - s.cap);
  }
  int tot = 0, tot_over = 0;
  int run = block_exclusive_scan<NT>(sum, part, &tot);
  if (publish) block_exclusive_scan<NT>(over, part, &tot_over);
  for (int a = a0; a < a1; ++a) {
    const int n = offl[a];
    offl[a] = run;
    cur[a] = run;
    run += n;
  }
  if (tid == 0) offl[A] = tot;
  lds_barrier();
  if (tid < 64) {
    const int lane = tid;
    int nbits = 0;
    while ((1 << nbits) < A) ++nbits;
    const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < ne; c0 += 64) {
      const int i = c0 + lane;
      int a = i < ne ? ads[i] : -1;
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
        const int c = cur[a];
        idxl[c + rank] = i;
        __builtin_amdgcn_wave_barrier();
        if (rank == count - 1) cur[a] = c + count;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  lds_barrier();
  if (publish) {
    int32_t* og = fp.off + (size_t)bh * (A + 1);
    int32_t* ig = fp.idx + (size_t)bh * s.nb;
    for (int a = tid; a <= A; a += NT) og[a] = offl[a];
    for (int i = tid; i < s.nb; i += NT) ig[i] = i < tot ? idxl[i] : -1;
    if (tid == 0) fp.overflow[bh] = tot_over;
  }
}

// The same lists with the filing spread over the work-group's waves: wave w takes a contiguous run of
// 64-block chunks, so its blocks come after those of waves < w.  Each wave first counts its blocks per
// address (a row of `wcur` [NT/64][A] per wave); the scan over addresses turns the rows into each
// wave's first slot per address (after the blocks of the earlier waves), and every wave then files its
// chunks in order with the ballot ranks, as above.  The result is identical; the chain of dependent
// chunk steps is NT/64 times shorter.
template <int NT>
__device__ void build_posting_csr_waves(const int* ads, int* wcur, int* offl, int* idxl, const Shape& s, int bh,
                                        bool publish, const FusedPost& fp) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int A = s.A, ne = s.ne;
  const int nch = (ne + 63) / 64, cpw = (nch + NW - 1) / NW;
  const int c0 = min(nch, wave * cpw), c1 = min(nch, c0 + cpw);
  int* cw = wcur + wave * A;  // this wave's counts, then its cursors
  for (int a = tid; a < NW * A; a += NT) wcur[a] = 0;
  lds_barrier();
  for (int c = c0; c < c1; ++c) {
    const int i = c * 64 + lane;
    const int a = i < ne ? ads[i] : -1;
    if (a >= 0 && a < A) atomicAdd(&cw[a], 1);
  }
  lds_barrier();
  // thread tid owns the contiguous address segment [a0, a1)
  __shared__ int part[NT / 64];
  const int seg = (A + NT - 1) / NT;
  const int a0 = min(A, tid * seg), a1 = min(A, a0 + seg);
  int sum = 0, over = 0;
  for (int a = a0; a < a1; ++a) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n += wcur[w * A + a];
    sum += n;
    over += max(0, n - s.cap);
  }
  int tot = 0, tot_over = 0;
  int run = block_exclusive_scan<NT>(sum, part, &tot);
  if (publish) block_exclusive_scan<NT>(over, part, &tot_over);
  for (int a = a0; a < a1; ++a) {
    offl[a] = run;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int n = wcur[w * A + a];
      wcur[w * A + a] = run;
      run += n;
    }
  }
  if (tid == 0) offl[A] = tot;
  lds_barrier();
  int nbits = 0;
  while ((1 << nbits) < A) ++nbits;
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int c = c0; c < c1; ++c) {
    const int i = c * 64 + lane;
    int a = i < ne ? ads[i] : -1;
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
      const int cp = cw[a];
      idxl[cp + rank] = i;
      __builtin_amdgcn_wave_barrier();
      if (rank == count - 1) cw[a] = cp + count;
    }
    __builtin_amdgcn_wave_barrier();
  }
  lds_barrier();
  if (publish) {
    int32_t* og = fp.off + (size_t)bh * (A + 1);
    int32_t* ig = fp.idx + (size_t)bh * s.nb;
    for (int a = tid; a <= A; a += NT) og[a] = offl[a];
    for (int i = tid; i < s.nb; i += NT) ig[i] = i < tot ? idxl[i] : -1;
    if (tid == 0) fp.overflow[bh] = tot_over;
  }
}

// Lane layout of the MFMA operands below: lane l = 16 s4 + r16 holds D/4 dims of one row (a token
// of Q or a code of the codebook).  bf16: dims 32kk + 8 s4 + e (the k-slots of v_mfma_f32_16x16x32_bf16);
// fp32: dims s4 (D/4) + x (one k-step of v_mfma_f32_16x16x4f32 per x).
template <bool BF, int D>
__device__ inline int operand_dim(int s4, int x) {
  return BF ? 32 * (x >> 3) + 8 * s4 + (x & 7) : s4 * (D / 4) + x;
}

// Small bf16 shapes keep four waves per SIMD, so that four 256-token work-groups share a CU.
constexpr int probe_min_waves(int bytes, int D, int C) { return bytes == 2 && D <= 64 && C <= 16 ? 4 : 1; }

constexpr int cpow(int b, int e) { return e == 0 ? 1 : b * cpow(b, e - 1); }

template <typename T, int D, int G, int C, int P, int R, bool FUSED, bool DIAG, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(probe_min_waves((int)sizeof(T), D, C)))) void k_probe_fixed(
    const T* __restrict__ Q, const float* __restrict__ cb, const float* __restrict__ bias,
    const float* __restrict__ ksum, const int32_t* __restrict__ off, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ force, int32_t* __restrict__ sel, int32_t* __restrict__ ncand,
    int32_t* __restrict__ phist, FusedPost fp, ProbeExtra ex, Shape s) {
  static_assert(NT % 64 == 0 && NT <= kProbeFixedThreads, "whole waves of 64 tokens");
  constexpr bool BF = std::is_same<T, bf16>::value;
  constexpr int CP = (C + 15) & ~15;
  constexpr int MST = G * CP + 1;  // odd stride: each lane's row starts in its own bank
  constexpr int PG = P < C ? P : C;
  constexpr int DQ = D / 4;        // operand dims per lane
  extern __shared__ __align__(16) float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, s4 = lane >> 4;
  const int bh = blockIdx.y, h = bh % s.H;
  const int tbase = blockIdx.x * NT;
  const int t = tbase + tid;
  const int A = s.A;
  constexpr int RK = R > 0 ? R : 1;
  // the mu rows, later the candidate list and then (diagnostics) the scores or (routing) the top-R keys
  float* mu = smem;  // [NT][MST]
  int* csr = (int*)(smem + max(NT * MST, DIAG ? NT * s.M * 2 : NT * (s.M + 2 * RK)));  // off [A+1], idx [ne]
  // ---- the addresses (or the CSR) of this (b,h), first 8 per lane
  const int32_t* og = off + (size_t)bh * (A + 1);
  const int32_t* ig = idx + (size_t)bh * s.nb;
  const int32_t* ag = FUSED ? fp.addr + (size_t)bh * s.nb : nullptr;
  const int ncsr = A + 1 + s.ne;
  const int nread = FUSED ? s.ne : ncsr;  // addresses of the filed blocks, or the CSR itself
  int cv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = u * NT + tid;
    if (FUSED)
      cv[u] = k < nread ? ag[k] : 0;
    else
      cv[u] = k < nread ? (k <= A ? og[k] : ig[k - A - 1]) : 0;
  }
  // ---- the posting-list CSR into LDS (this kernel is only used when it fits): read as is, or
  // built here from the addresses (FUSED), in the mu region, before the logits need it
  int* stage = FUSED ? (int*)mu : csr;  // addresses [ne] and list cursors [A] | the CSR
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = u * NT + tid;
    if (k < nread) stage[k] = cv[u];
  }
  for (int k0 = 8 * NT; k0 < nread; k0 += 8 * NT) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u * NT + tid;
      if (FUSED)
        v[u] = k < nread ? ag[k] : 0;
      else
        v[u] = k < nread ? (k <= A ? og[k] : ig[k - A - 1]) : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u * NT + tid;
      if (k < nread) stage[k] = v[u];
    }
  }
  // the codebook rows and biases of this lane's codes and the query rows of its four 16-token tiles
  // are requested next, so that they arrive while the lists are built
  const float* cbh = cb + (size_t)h * G * C * D;
  float wv[G][CP / 16][DQ];
  float bv[G][CP / 16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int ct = 0; ct < CP / 16; ++ct) {
      const int code = ct * 16 + r16;
      const float* wr = cbh + ((size_t)g * C + (code < C ? code : 0)) * D;
#pragma unroll
      for (int x = 0; x < DQ; x += 4) {
        const float4 v = *(const float4*)(wr + operand_dim<BF, D>(s4, x));
        wv[g][ct][x] = code < C ? v.x : 0.f;
        wv[g][ct][x + 1] = code < C ? v.y : 0.f;
        wv[g][ct][x + 2] = code < C ? v.z : 0.f;
        wv[g][ct][x + 3] = code < C ? v.w : 0.f;
      }
      bv[g][ct] = (bias && code < C) ? bias[(h * G + g) * C + code] : 0.f;
    }
  constexpr int QV = DQ * (int)sizeof(T) / 16;  // 16-byte pieces of a lane's query slice
  uint4 qraw[4][QV];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    int tq = tbase + wave * 64 + tt * 16 + r16;
    tq = tq < s.S ? tq : s.S - 1;
    const T* qp = Q + ((size_t)bh * s.S + tq) * D;
#pragma unroll
    for (int c = 0; c < QV; ++c) qraw[tt][c] = *(const uint4*)(qp + operand_dim<BF, D>(s4, c * (16 / (int)sizeof(T))));
  }
  int fv = -1;
  if (force && R > 0 && t < s.S) fv = force[(size_t)bh * s.S + t];
  if constexpr (FUSED) {
    // one cursor row per wave when they fit beside the addresses, else one wave files every chunk
    if ((long long)s.ne + (NT / 64) * A <= (long long)NT * MST)
      build_posting_csr_waves<NT>(stage, stage + s.ne, csr, csr + A + 1, s, bh, blockIdx.x == 0, fp);
    else
      build_posting_csr<NT>(stage, stage + s.ne, csr, csr + A + 1, s, bh, blockIdx.x == 0, fp);
  }
  const int* offp = csr;
  const int* idxp = csr + A + 1;
  // ---- mu on MFMA: lane l receives mu[token 16tt + 4(l/16) + k][code 16ct + l%16].  fp32 inputs use
  // v_mfma_f32_16x16x4_f32.  For bf16 inputs every fp32 codebook value is split exactly into three
  // bf16 parts (w = hi + mid + lo, 8 significand bits each) and mu accumulates q*hi + q*mid + q*lo on
  // v_mfma_f32_16x16x32_bf16; q is exact in bf16, so every product is exact and only the fp32
  // accumulation rounds, as in an fp32 dot product.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int ct = 0; ct < CP / 16; ++ct) {
      if constexpr (BF) {
        bf16x8 wh[D / 32], wm[D / 32], wl[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float w = wv[g][ct][8 * kk + e];
            const bf16 hi = (bf16)w;
            const float r1 = w - (float)hi;
            const bf16 mi = (bf16)r1;
            wh[kk][e] = hi;
            wm[kk][e] = mi;
            wl[kk][e] = (bf16)(r1 - (float)mi);
          }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const bf16x8 qa = *(const bf16x8*)&qraw[tt][kk];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, wh[kk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, wm[kk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, wl[kk], acc, 0, 0, 0);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k)
            mu[(wave * 64 + tt * 16 + 4 * s4 + k) * MST + g * CP + ct * 16 + r16] = acc[k] + bv[g][ct];
        }
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const float* qa = (const float*)&qraw[tt][0];
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int x = 0; x < DQ; ++x) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[x], wv[g][ct][x], acc, 0, 0, 0);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            mu[(wave * 64 + tt * 16 + 4 * s4 + k) * MST + g * CP + ct * 16 + r16] = acc[k] + bv[g][ct];
        }
      }
    }
  lds_barrier();
  const bool active = t < s.S;
  const int j = t / s.blk;
  const int cutoff = j - s.L;
  const float* mrow = mu + tid * MST;

  // ---- top-PG codes of every subspace by (mu desc, code asc): packed 32-bit keys, one more kept
  // than used to see the boundary; a token whose packed ranks might differ from the exact ones
  // ranks that subspace again with 64-bit keys.  mu is read back from LDS for the kept codes.
  constexpr int CB = key_bits(C);
  constexpr int KG = PG < C ? PG + 1 : PG;
  int tcode[G][PG];
  float tval[G][PG];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t top[KG];
#pragma unroll
    for (int p = 0; p < KG; ++p) top[p] = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) insert_packed<KG>(top, packed_key<CB>(mrow[g * CP + c], c));
    if (packed_exact<KG, CB>(top)) {
#pragma unroll
      for (int p = 0; p < PG; ++p) tcode[g][p] = packed_index<CB>(top[p]);
    } else {
      uint64_t top64[PG];
#pragma unroll
      for (int p = 0; p < PG; ++p) top64[p] = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) insert_key<PG>(top64, rank_key(mrow[g * CP + c], c));
#pragma unroll
      for (int p = 0; p < PG; ++p) tcode[g][p] = key_index(top64[p]);
    }
#pragma unroll
    for (int p = 0; p < PG; ++p) tval[g][p] = mrow[g * CP + tcode[g][p]];
  }
  // ---- rank vectors with prod (k_g + 1) <= P, top-P addresses by (sigma desc, address asc); packed
  // keys when the address takes few bits, with the same boundary check and 64-bit fallback
  constexpr int NCOMB = RankSpace<G, PG>::count();
  constexpr int AB = G * CB;
  constexpr bool PACK_A = AB <= 12;
  constexpr int KP = P + 1;
  auto combo = [&](int kc, float& sig, int& a) -> bool {
    int rem = kc, prod = 1;
    int rk[G];
#pragma unroll
    for (int g = G - 1; g >= 0; --g) {
      rk[g] = rem % PG;
      rem /= PG;
      prod *= rk[g] + 1;
    }
    sig = tval[0][rk[0]];
    a = tcode[0][rk[0]];
#pragma unroll
    for (int g = 1; g < G; ++g) {
      sig += tval[g][rk[g]];
      a = a * C + tcode[g][rk[g]];
    }
    return prod <= P;
  };
  auto exact_addresses = [&](int (&out)[P]) {
    uint64_t tpk[P];
#pragma unroll
    for (int p = 0; p < P; ++p) tpk[p] = 0;
#pragma unroll
    for (int kc = 0; kc < NCOMB; ++kc) {
      float sig;
      int a;
      if (combo(kc, sig, a)) insert_key<P>(tpk, rank_key(sig, a));
    }
#pragma unroll
    for (int p = 0; p < P; ++p) out[p] = key_index(tpk[p]);
  };
  int tpa[P];
  float pmarg = INFINITY;  // diagnostics: smallest gap between neighbouring scores of the P + 1 best addresses
  if constexpr (DIAG) {
    // exact (value desc, index asc) ranks over every code and rank vector that can reach the P + 1 best
    // addresses: min(P + 1, C) codes per subspace, rank vectors with prod (k_g + 1) <= P + 1
    constexpr int PX = P + 1 < C ? P + 1 : C;
    constexpr int NCX = RankSpace<G, PX>::count();
    constexpr int KX = P + 1 < cpow(C, G) ? P + 1 : cpow(C, G);
    int xcode[G][PX];
    float xval[G][PX];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint64_t t64[PX];
#pragma unroll
      for (int p = 0; p < PX; ++p) t64[p] = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) insert_key<PX>(t64, rank_key(mrow[g * CP + c], c));
#pragma unroll
      for (int p = 0; p < PX; ++p) {
        xcode[g][p] = key_index(t64[p]);
        xval[g][p] = mrow[g * CP + xcode[g][p]];
      }
    }
    uint64_t tpk[KX];
#pragma unroll
    for (int p = 0; p < KX; ++p) tpk[p] = 0;
#pragma unroll
    for (int kc = 0; kc < NCX; ++kc) {
      int rem = kc, prod = 1;
      int rk[G];
#pragma unroll
      for (int g = G - 1; g >= 0; --g) {
        rk[g] = rem % PX;
        rem /= PX;
        prod *= rk[g] + 1;
      }
      float sig = xval[0][rk[0]];
      int a = xcode[0][rk[0]];
#pragma unroll
      for (int g = 1; g < G; ++g) {
        sig += xval[g][rk[g]];
        a = a * C + xcode[g][rk[g]];
      }
      if (prod <= P + 1) insert_key<KX>(tpk, rank_key(sig, a));
    }
#pragma unroll
    for (int p = 0; p < P; ++p) tpa[p] = key_index(tpk[p]);
#pragma unroll
    for (int p = 0; p + 1 < KX; ++p) pmarg = fminf(pmarg, key_value(tpk[p]) - key_value(tpk[p + 1]));
  } else if constexpr (PACK_A) {
    uint32_t tpk[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) tpk[p] = 0;
#pragma unroll
    for (int kc = 0; kc < NCOMB; ++kc) {
      float sig;
      int a;
      if (combo(kc, sig, a)) insert_packed<KP>(tpk, packed_key<AB>(sig, a));
    }
    if (packed_exact<KP, AB>(tpk)) {
#pragma unroll
      for (int p = 0; p < P; ++p) tpa[p] = packed_index<AB>(tpk[p]);
    } else {
      exact_addresses(tpa);
    }
  } else {
    exact_addresses(tpa);
  }
  // ---- candidate ranges: probe p contributes the `take[p]` newest entries <= cutoff of its list,
  // ending at CSR position lim[p] (exclusive), then (redirect policy) the `rtake[p]` newest arrivals
  // of its redirect list up to query block j, ending at rlim[p], until M candidates.  Dropped
  // candidates: per probe, the eligible blocks the list holds beyond its capacity.
  int lim[P], take[P], rlim[P], rtake[P];
  int nc = 0, ndr = 0;
  const int32_t* roffp = ex.roff ? ex.roff + (size_t)bh * (A + 1) : nullptr;
  const int32_t* ridxp = ex.roff ? ex.ridx + (size_t)bh * s.nb : nullptr;
  const int32_t* rtimep = ex.roff ? ex.rtime + (size_t)bh * s.nb : nullptr;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    take[p] = 0;
    lim[p] = 0;
    rtake[p] = 0;
    rlim[p] = 0;
    if (active && cutoff >= 0) {
      const int a = tpa[p];
      const int lo = offp[a], hi = offp[a + 1];
      int l0 = lo, l1 = hi;  // first entry > cutoff
      while (l0 < l1) {
        const int mid = (l0 + l1) >> 1;
        if (idxp[mid] <= cutoff)
          l0 = mid + 1;
        else
          l1 = mid;
      }
      const int nprim = l0 - lo, tp = min(s.cap, nprim);
      const int tk = R > 0 ? min(tp, s.M - nc) : 0;
      take[p] = tk > 0 ? tk : 0;
      lim[p] = l0;
      nc += take[p];
      int narr = 0;
      if (roffp) {
        const int rlo = roffp[a];
        int r0 = rlo, r1 = roffp[a + 1];  // first arrival after query block j
        while (r0 < r1) {
          const int mid = (r0 + r1) >> 1;
          if (rtimep[mid] <= j)
            r0 = mid + 1;
          else
            r1 = mid;
        }
        narr = r0 - rlo;
        const int tr = R > 0 ? min(min(s.cap - tp, narr), s.M - nc) : 0;
        rtake[p] = tr > 0 ? tr : 0;
        rlim[p] = r0;
        nc += rtake[p];
      }
      // held: the primaries not redirected away (every block has an alternate when C > 1) plus arrivals
      ndr += max(0, (roffp && C > 1 ? tp : nprim) + narr - s.cap);
    }
  }
  // ---- the work-group's candidates as one list (token-major) in LDS, in the place of mu
  __shared__ int scan_tmp[NT / 64];
  int total;
  const int base = block_exclusive_scan<NT>(nc, scan_tmp, &total);
  int* clist = (int*)smem;                          // [total] (local token << 16) | block
  float* rho = smem + NT * s.M;                     // [total] scores (diagnostics)
  uint64_t* topk = (uint64_t*)(smem + NT * s.M);    // [NT][RK] each token's top-R keys (routing)
  {
    int k = base;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      for (int e = 0; e < take[p]; ++e) clist[k++] = (tid << 16) | idxp[lim[p] - 1 - e];
      for (int e = 0; e < rtake[p]; ++e) clist[k++] = (tid << 16) | ridxp[rlim[p] - 1 - e];
    }
  }
  lds_barrier();
  // ---- rerank scores: LPT adjacent lanes share a token (token wave*64 + (64/LPT)m + lane/LPT,
  // m = 0..LPT-1); lane o = lane%LPT takes dims 4*LPT*c + 4o + e, so the group reads 16*LPT contiguous
  // bytes of a summary per load.  Several candidates are in flight at a time; the partial dots are
  // added in a fixed order (xor 1, 2, ...).  The query slices are read again (from L2) rather than
  // kept live through the selection above, the next token's while the current one is scored.  The
  // routing variant ranks each score into the token's top-R right away (the group's lanes hold the same
  // list) and leaves only the R keys in LDS; the diagnostics variant, which needs every candidate's
  // score, stores them all.
  {
    constexpr int LPT = 4;
    constexpr int NC4 = D / (4 * LPT);   // float4 per candidate per lane
    constexpr int UB = 16 / NC4;         // candidates in flight
    const float* ksh = ksum + (size_t)bh * s.nb * D;
    const int grp = lane / LPT, lo = lane % LPT;
    using QP = typename std::conditional<BF, uint2, uint4>::type;  // 4 query values
    auto q_slice = [&](int m, QP (&raw)[NC4]) {
      int tq = tbase + wave * 64 + (64 / LPT) * m + grp;
      tq = tq < s.S ? tq : s.S - 1;
      const T* qp = Q + ((size_t)bh * s.S + tq) * D + 4 * lo;
#pragma unroll
      for (int c = 0; c < NC4; ++c) raw[c] = *(const QP*)(qp + 4 * LPT * c);
    };
    QP qnext[NC4];
    q_slice(0, qnext);
    for (int m = 0; m < LPT; ++m) {
      const int src = (64 / LPT) * m + grp;
      const int b0 = __shfl(base, src), n0 = __shfl(nc, src);
      float qf[4 * NC4];
#pragma unroll
      for (int c = 0; c < NC4; ++c) {
        if constexpr (BF) {
          const bf16x4 qb = *(const bf16x4*)&qnext[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[4 * c + e] = (float)qb[e];
        } else {
          const float4 q4 = *(const float4*)&qnext[c];
          qf[4 * c] = q4.x;
          qf[4 * c + 1] = q4.y;
          qf[4 * c + 2] = q4.z;
          qf[4 * c + 3] = q4.w;
        }
      }
      if (m + 1 < LPT) q_slice(m + 1, qnext);
      uint64_t tk[RK];
#pragma unroll
      for (int r = 0; r < RK; ++r) tk[r] = 0;
      for (int k0 = 0; k0 < n0; k0 += UB) {
        float4 kv[UB][NC4];
        int iu[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int i = clist[b0 + (k0 + u < n0 ? k0 + u : k0)] & 0xffff;
          iu[u] = i;
          const float* kr = ksh + (size_t)i * D + 4 * lo;
#pragma unroll
          for (int c = 0; c < NC4; ++c) kv[u][c] = *(const float4*)(kr + 4 * LPT * c);
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          float a = 0.f;
#pragma unroll
          for (int c = 0; c < NC4; ++c) {
            a = fmaf(kv[u][c].x, qf[4 * c], a);
            a = fmaf(kv[u][c].y, qf[4 * c + 1], a);
            a = fmaf(kv[u][c].z, qf[4 * c + 2], a);
            a = fmaf(kv[u][c].w, qf[4 * c + 3], a);
          }
#pragma unroll
          for (int x = 1; x < LPT; x <<= 1) a += __shfl_xor(a, x);
          if constexpr (DIAG) {
            if (lo == 0 && k0 + u < n0) rho[b0 + k0 + u] = a;
          } else {
            if (k0 + u < n0) insert_key<RK>(tk, rank_key(a, iu[u]));
          }
        }
      }
      if constexpr (!DIAG) {
        if (lo == 0)
#pragma unroll
          for (int r = 0; r < RK; ++r) topk[(wave * 64 + src) * RK + r] = tk[r];
      }
    }
  }
  lds_barrier();
  // ---- top-R of the token's candidates by (score desc, block asc): ranked here from the scores
  // (diagnostics), or as ranked in the rerank (the order of insertion does not change a top list under
  // this total order)
  constexpr int RKX = DIAG ? RK + 1 : RK;  // diagnostics: one more, for the margin at the boundary
  int tri[RK];
  int nr = 0;
  if (active) {
    uint64_t trk[RKX];
    if constexpr (DIAG) {
#pragma unroll
      for (int r = 0; r < RKX; ++r) trk[r] = 0;
      for (int k = base; k < base + nc; ++k) insert_key<RKX>(trk, rank_key(rho[k], clist[k] & 0xffff));
    } else {
#pragma unroll
      for (int r = 0; r < RK; ++r) trk[r] = topk[tid * RK + r];
    }
#pragma unroll
    for (int r = 0; r < RK; ++r) tri[r] = key_index(trk[r]);
    nr = nc < R ? nc : R;
    int fslot = -1;  // the slot a forced block took
    if (force && R > 0) {
      const int f = fv;
      if (f >= 0 && f <= cutoff) {
        bool present = false;
#pragma unroll
        for (int r = 0; r < RK; ++r) present |= (r < nr && tri[r] == f);
        if (!present) {
          const int slot = nr < R ? nr : R - 1;
#pragma unroll
          for (int r = 0; r < RK; ++r)
            if (r == slot) tri[r] = f;
          nr = nr < R ? nr + 1 : R;
          fslot = slot;
        }
      }
    }
    int32_t* srow = sel + ((size_t)bh * s.S + t) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) srow[r] = r < nr ? tri[r] : -1;
    if (ncand) ncand[(size_t)bh * s.S + t] = nc;
    if (ex.ndrop) ex.ndrop[(size_t)bh * s.S + t] = ndr;
    if constexpr (DIAG) {
      const size_t tt = (size_t)bh * s.S + t;
      if (ex.probes)
#pragma unroll
        for (int p = 0; p < P; ++p) ex.probes[tt * P + p] = tpa[p];
      if (ex.pmargin) ex.pmargin[tt] = pmarg;
      float smarg = INFINITY;
#pragma unroll
      for (int r = 0; r + 1 < RKX; ++r)
        if (r + 1 < nc && r < R) smarg = fminf(smarg, key_value(trk[r]) - key_value(trk[r + 1]));
      if (ex.smargin) ex.smargin[tt] = R > 0 ? smarg : INFINITY;
      if (ex.sel_score)
#pragma unroll
        for (int r = 0; r < R; ++r)
          ex.sel_score[tt * R + r] = r >= nr ? -INFINITY : r == fslot ? NAN : key_value(trk[r]);
    }
  }
  if (!phist) return;  // uniform
  // ---- count the selected pairs of this work-group's token range per remote block (LDS histogram in the
  // place of mu when it fits)
  PairCounter<NT> pc{s.ne <= NT * MST ? (int*)mu : nullptr, phist + pair_counts_row(s, bh, tbase),
                     s.ne};
  pc.begin();
  if (active) {
#pragma unroll
    for (int r = 0; r < RK; ++r)
      if (r < nr) pc.add(tri[r]);
  }
  pc.end();
}

// Two blocks per work-group when a thread's key rows of both fit in a few registers (at most four
// 16-byte reads per block), else one.
template <typename T, int D, int BLK>
constexpr int address_blocks_per_group() {
  return (BLK + AddressLds<T, D>::RG - 1) / AddressLds<T, D>::RG <= 4 ? 2 : 1;
}

template <typename T, int D, int BLK>
hipError_t address_launch_b(const Shape& s, int n, const void* k, const float* cb, const float* bias, float* ksum,
                            int32_t* addr, int32_t* cnt, int32_t* alt, float* am, int i0, hipStream_t st) {
  constexpr int NB = address_blocks_per_group<T, D, BLK>();
  const dim3 grid((n + NB - 1) / NB, s.B * s.H);
  hipLaunchKernelGGL((k_address<T, D, BLK, NB>), grid, dim3(256), 0, st, (const T*)k, cb, bias, ksum, addr, cnt, alt,
                     am, i0, i0 + n, s);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t address_launch_d(const Shape& s, int n, const void* k, const float* cb, const float* bias, float* ksum,
                            int32_t* addr, int32_t* cnt, int32_t* alt, float* am, int i0, hipStream_t st) {
  switch (s.blk) {
    case 32: return address_launch_b<T, D, 32>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
    case 64: return address_launch_b<T, D, 64>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
    default: return address_launch_b<T, D, 128>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
  }
}

template <typename T>
hipError_t address_dispatch(const Shape& s, const void* k, const float* cb, const float* bias, float* ksum,
                            int32_t* addr, int32_t* cnt, int32_t* alt, float* am, int i0, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  switch (s.D) {
    case 32: return address_launch_d<T, 32>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
    case 64: return address_launch_d<T, 64>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
    case 128: return address_launch_d<T, 128>(s, n, k, cb, bias, ksum, addr, cnt, alt, am, i0, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, int G, int C, int P, int R, bool FUSED, bool DIAG, int NT>
hipError_t probe_fixed_launch_nt(const Shape& s, const void* q, const float* cb, const float* bias, const float* ksum,
                                 const int32_t* off, const int32_t* idx, const int32_t* force, int32_t* sel,
                                 int32_t* ncand, int32_t* phist, const FusedPost& fp,
                                 const ProbeExtra& ex, hipStream_t st) {
  dim3 grid((s.S + NT - 1) / NT, s.B * s.H);
  const size_t lds = probe_lds_bytes(s, NT, DIAG);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_probe_fixed<T, D, G, C, P, R, FUSED, DIAG, NT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_probe_fixed<T, D, G, C, P, R, FUSED, DIAG, NT>), grid, dim3(NT), lds, st, (const T*)q, cb,
                     bias, ksum, off, idx, force, sel, ncand, phist, fp, ex, s);
  return hipGetLastError();
}

// The routing path's probe (lists built in the kernel, no diagnostics) also comes with 128- and 64-token
// work-groups, for shapes whose LDS holds more waves of the smaller groups and for grids that 256-token
// groups would leave short of two per CU; the others keep 256.
template <typename T, int D, int G, int C, int P, int R, bool FUSED, bool DIAG>
hipError_t probe_fixed_launch_t(const Shape& s, const void* q, const float* cb, const float* bias, const float* ksum,
                                const int32_t* off, const int32_t* idx, const int32_t* force, int32_t* sel,
                                int32_t* ncand, int32_t* phist, const FusedPost& fp,
                                const ProbeExtra& ex, hipStream_t st) {
  if constexpr (FUSED && !DIAG) {
    const int nt = probe_fixed_tokens(s);
    if (nt == 64)
      return probe_fixed_launch_nt<T, D, G, C, P, R, FUSED, DIAG, 64>(s, q, cb, bias, ksum, off, idx, force, sel,
                                                                      ncand, phist, fp, ex, st);
    if (nt == 128)
      return probe_fixed_launch_nt<T, D, G, C, P, R, FUSED, DIAG, 128>(s, q, cb, bias, ksum, off, idx, force, sel,
                                                                       ncand, phist, fp, ex, st);
  }
  return probe_fixed_launch_nt<T, D, G, C, P, R, FUSED, DIAG, kProbeFixedThreads>(
      s, q, cb, bias, ksum, off, idx, force, sel, ncand, phist, fp, ex, st);
}

template <typename T, int D, int G, int C, int P, int R>
hipError_t probe_fixed_launch(const Shape& s, const void* q, const float* cb, const float* bias, const float* ksum,
                              const int32_t* off, const int32_t* idx, const int32_t* force, int32_t* sel,
                              int32_t* ncand, int32_t* phist, const FusedPost* fuse,
                              const ProbeExtra& ex, hipStream_t st) {
  const bool diag = ex.probes || ex.sel_score || ex.pmargin || ex.smargin;
  const FusedPost none{nullptr, nullptr, nullptr, nullptr};
  if (fuse)
    return diag ? probe_fixed_launch_t<T, D, G, C, P, R, true, true>(s, q, cb, bias, ksum, off, idx, force, sel,
                                                                     ncand, phist, *fuse, ex, st)
                : probe_fixed_launch_t<T, D, G, C, P, R, true, false>(s, q, cb, bias, ksum, off, idx, force, sel,
                                                                      ncand, phist, *fuse, ex, st);
  return diag ? probe_fixed_launch_t<T, D, G, C, P, R, false, true>(s, q, cb, bias, ksum, off, idx, force, sel, ncand,
                                                                    phist, none, ex, st)
              : probe_fixed_launch_t<T, D, G, C, P, R, false, false>(s, q, cb, bias, ksum, off, idx, force, sel,
                                                                     ncand, phist, none, ex, st);
}

// Shapes with a compile-time specialisation (the five workload families); others use k_probe_rerank.
#define MDR_PROBE_FIXED_SHAPES(X) \
  X(bf16, 64, 2, 16, 4, 2)        \
  X(bf16, 128, 2, 32, 4, 4)       \
  X(bf16, 128, 3, 8, 6, 8)        \
  X(float, 64, 2, 8, 16, 2)       \
  X(float, 32, 2, 4, 2, 2)

template <typename T>
hipError_t probe_dispatch(const Shape& s, const void* q, const float* cb, const float* bias, const float* ksum,
                          const int32_t* off, const int32_t* idx, const int32_t* force, int32_t* sel,
                          int32_t* ncand, int32_t* phist, const FusedPost* fuse,
                          const ProbeExtra& ex, hipStream_t st) {
#define MDR_FIXED(TT, DD, GG, CC, PP, RR)                                                                        \
  if (std::is_same<T, TT>::value && s.D == DD && s.G == GG && s.C == CC && s.P == PP && s.R == RR && s.fixed_probe) \
    return probe_fixed_launch<TT, DD, GG, CC, PP, RR>(s, q, cb, bias, ksum, off, idx, force, sel, ncand, phist,  \
                                                      fuse, ex, st);
  MDR_PROBE_FIXED_SHAPES(MDR_FIXED)
#undef MDR_FIXED
  if (fuse) return hipErrorInvalidValue;  // only the specialised probe builds the lists itself
  dim3 grid((s.S + kProbeThreads - 1) / kProbeThreads, s.B * s.H);
  const size_t lds = probe_lds_bytes(s, kProbeThreads);
  const void* fn = nullptr;
  switch (s.D) {
    case 32: fn = (const void*)k_probe_rerank<T, 32>; break;
    case 64: fn = (const void*)k_probe_rerank<T, 64>; break;
    case 128: fn = (const void*)k_probe_rerank<T, 128>; break;
    default: return hipErrorInvalidValue;
  }
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  switch (s.D) {
    case 32:
      hipLaunchKernelGGL((k_probe_rerank<T, 32>), grid, dim3(kProbeThreads), lds, st, (const T*)q, cb, bias, ksum,
                         off, idx, force, sel, ncand, phist, ex, s);
      break;
    case 64:
      hipLaunchKernelGGL((k_probe_rerank<T, 64>), grid, dim3(kProbeThreads), lds, st, (const T*)q, cb, bias, ksum,
                         off, idx, force, sel, ncand, phist, ex, s);
      break;
    default:
      hipLaunchKernelGGL((k_probe_rerank<T, 128>), grid, dim3(kProbeThreads), lds, st, (const T*)q, cb, bias,
                         ksum, off, idx, force, sel, ncand, phist, ex, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_address(const Shape& s, const void* k, const float* codebook, const float* bias, float* ksum,
                          int32_t* addr, int32_t* pair_zero, hipStream_t st, int i0, int n, int32_t* alt,
                          float* amargin) {
  if (n < 0) n = s.nb - i0;
  if (s.dtype == MDR_BF16)
    return address_dispatch<bf16>(s, k, codebook, bias, ksum, addr, pair_zero, alt, amargin, i0, n, st);
  return address_dispatch<float>(s, k, codebook, bias, ksum, addr, pair_zero, alt, amargin, i0, n, st);
}

bool probe_fixed_shape(const Shape& s) {
  if (!s.csr_lds) return false;
  const bool bf = s.dtype == MDR_BF16;
#define MDR_MATCH(TT, DD, GG, CC, PP, RR)                                                                  \
  if ((std::is_same<TT, bf16>::value == bf) && s.D == DD && s.G == GG && s.C == CC && s.P == PP && s.R == RR) \
    return true;
  MDR_PROBE_FIXED_SHAPES(MDR_MATCH)
#undef MDR_MATCH
  return false;
}

size_t probe_lds_bytes(const Shape& s, int nt, bool diag) {
  const int CP = (s.C + 15) & ~15;
  if (s.fixed_probe) {
    // mu rows during the logits, then the work-group's candidate list (block ids) and either the
    // candidates' scores (diagnostics) or each token's top-R keys (two words each)
    const size_t mu_w = (size_t)nt * (s.G * CP + 1);
    const size_t pairs_w = diag ? (size_t)nt * s.M * 2 : (size_t)nt * (s.M + 2 * (s.R > 0 ? s.R : 1));
    return ((mu_w > pairs_w ? mu_w : pairs_w) + (s.csr_lds ? (size_t)(s.A + 1 + s.ne) : 0)) * 4;
  }
  const int Pg = s.P + 1 < s.C ? s.P + 1 : s.C;  // laid out for the diagnostics sizes (P + 1, R + 1)
  const size_t words = (size_t)kProbeThreads * (s.G * CP + 4) +
                       (size_t)kProbeThreads * (s.G * Pg + 2 * (s.P + 1) + 2 * (s.R + 1)) +
                       (s.csr_lds ? (size_t)(s.A + 1 + s.ne) : 0);
  return words * 4;
}

hipError_t launch_post(const Shape& s, const int32_t* addr, int32_t* off, int32_t* idx, int32_t* overflow,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_post, dim3(s.B * s.H), dim3(256), 0, st, addr, off, idx, overflow, s);
  return hipGetLastError();
}

hipError_t launch_probe_rerank(const Shape& s, const void* q, const float* codebook, const float* bias,
                               const float* ksum, const int32_t* off, const int32_t* idx, const int32_t* force,
                               int32_t* sel, int32_t* ncand, int32_t* phist, hipStream_t st,
                               const FusedPost* fuse, const ProbeExtra& ex) {
  if (fuse && ex.roff) return hipErrorInvalidValue;  // redirect lists need the whole CSR first
  if (s.dtype == MDR_BF16)
    return probe_dispatch<bf16>(s, q, codebook, bias, ksum, off, idx, force, sel, ncand, phist, fuse, ex, st);
  return probe_dispatch<float>(s, q, codebook, bias, ksum, off, idx, force, sel, ncand, phist, fuse, ex, st);
}

hipError_t launch_post_redirect(const Shape& s, const int32_t* addr, const int32_t* alt, const int32_t* off,
                                const int32_t* idx, int32_t* roff, int32_t* ridx, int32_t* rtime,
                                int32_t* overflow, hipStream_t st) {
  const size_t lds = ((size_t)s.A + 2 * (size_t)s.ne) * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_post_redirect, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_post_redirect, dim3(s.B * s.H), dim3(256), lds, st, addr, alt, off, idx, roff, ridx, rtime,
                     overflow, s);
  return hipGetLastError();
}

bool probe_fuses_post(const Shape& s) { return probe_fuses_post_nt(s, kProbeFixedThreads); }

bool probe_fuses_post_nt(const Shape& s, int nt) {
  // the fixed probe stages the addresses and list cursors in its mu region
  const int CP = (s.C + 15) & ~15;
  return s.fixed_probe && (long long)s.ne + s.A <= (long long)nt * (s.G * CP + 1);
}

int probe_fixed_tokens(const Shape& s) {
  // first the size whose work-groups keep the most waves resident as far as the LDS goes (160 KiB per
  // CU, allocated in 512-byte granules with room for the kernel's few static words; counted up to
  // four waves per SIMD, ties to the larger size, which builds the lists fewer times)...
  auto lds_waves = [&](int nt) {
    const size_t wg = (probe_lds_bytes(s, nt, false) + 64 + 511) / 512 * 512;
    const long long w = (long long)(160 * 1024 / wg) * (nt / 64);
    return w < 16 ? w : 16;
  };
  int nt = kProbeFixedThreads;
  for (int c = kProbeFixedThreads / 2; c >= 64 && probe_fuses_post_nt(s, c); c /= 2)
    if (lds_waves(c) > lds_waves(nt)) nt = c;
  // ...then smaller ones while the grid would give fewer than two work-groups per CU
  while (nt > 64 && (long long)s.B * s.H * ((s.S + nt - 1) / nt) < 2LL * kCUs && probe_fuses_post_nt(s, nt / 2))
    nt /= 2;
  return nt;
}

}  // namespace mdr
