// Binning of the selected (token, slot) pairs by remote block, for the selected-set attention.
//
// Routing is per query token, so the remote blocks of neighbouring tokens differ (aitechinspire.com
// write-up, "Snapshot: key facts from the report": each query probes, reranks and keeps a fixed number
// of remote blocks).  The attention reads each selected block's K/V once and applies it to every pair
// that chose it, so the pairs are first grouped by block -- a counting sort in space linear in the
// sequence:
//   counts   per (b,h), token range g (tbin tokens) and remote block i, the number of valid pairs: the
//            probe kernels count their own selections; k_pair_count counts a selection passed in, one
//            work-group per range writing its whole row (so the counters need no clearing first)
//   scatter  k_pair_scatter, one work-group per (range, b,h): the totals over all ranges give each
//            block's list offset (poff), the counts of the earlier ranges this range's first slot per
//            block; its pairs then go to their block's part of the list for this range.  For the
//            backward the waves file them in ascending pair id (t R + r) with ballot ranks, so every
//            list is in ascending token order whatever the timing; for the forward, whose partials
//            depend on each pair's own query only, each takes the next slot by an LDS atomic.  The
//            lists are stored as the remote work items: each block's list cut into records of
//            kItemPairs pair ids.
#include "mdr_internal.h"

namespace mdr {

namespace {

constexpr int kCountThreads = 1024;

// The scatter work-group takes its range's pairs kSubPairs at a time: their blocks (or -1) are staged in
// LDS by all threads at once, then the waves that file pairs count and file them from LDS.  Those waves'
// count and cursor rows share the LDS with two rows of per-block values and the staged blocks.
constexpr int kScatterThreads = 1024;
constexpr int kSubPairs = 4096;
constexpr int kScatterLdsInts = 37 * 1024;  // 148 KiB
__host__ __device__ inline int scatter_waves(int ne) {
  const int w = (kScatterLdsInts - kSubPairs) / ne - 3;
  return w > kScatterThreads / 64 ? kScatterThreads / 64 : w;
}

__global__ __launch_bounds__(kCountThreads) void k_pair_count(const int32_t* __restrict__ sel,
                                                              int32_t* __restrict__ phist, Shape s) {
  extern __shared__ int cnt[];  // [ne]
  const int g = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < s.ne; i += kCountThreads) cnt[i] = 0;
  __syncthreads();
  const int tfirst = g * s.tbin, tlast = min(s.S, tfirst + s.tbin);
  for (int t = tfirst + tid; t < tlast; t += kCountThreads) {
    const int j = t / s.blk;
    const int32_t* row = sel + ((size_t)bh * s.S + t) * s.R;
    for (int r = 0; r < s.R; ++r)
      if (sel_entry_valid(row, r, j, s.L)) atomicAdd(&cnt[row[r]], 1);
  }
  __syncthreads();
  int32_t* dst = phist + pair_counts_row(s, bh, tfirst);
  for (int i = tid; i < s.ne; i += kCountThreads) dst[i] = cnt[i];
}

// STABLE: the waves file their pairs with ballot ranks, so every list is in ascending pair id (the
// backward's sums over a block's pairs then run in a fixed order).  Otherwise (the forward) each pair
// takes the next slot of its block within the range's part of the list by an LDS atomic: the order
// inside a range's part varies from call to call, but the forward computes every pair's partial from
// its own query alone, so its results do not depend on it.
template <bool STABLE>
__global__ __launch_bounds__(kScatterThreads) void k_pair_scatter(const int32_t* __restrict__ sel,
                                                              const int32_t* __restrict__ phist,
                                                              int32_t* __restrict__ poff, int32_t* __restrict__ ioff,
                                                              int32_t* __restrict__ items, Shape s) {
  extern __shared__ int sm[];
  __shared__ int scan_tmp[2 * (kScatterThreads / 64)];
  const int ne = s.ne, g = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwf = scatter_waves(ne);
  int* base = sm;            // [ne] the next free slot per block of this range
  int* start = base + ne;    // [ne] pairs per block, then each block's list offset
  int* istart = start + ne;  // [ne] each block's first work item
  int* wc = istart + ne;     // [nwf][ne] per-wave counts, then per-wave cursors
  int* keys = wc + nwf * ne; // [kSubPairs] the blocks of the piece's pairs (-1: entry not used)
  // this range's tokens, kSubPairs / R at a time (all of a token's pairs in one piece); the first piece's
  // entries are requested before the counts, so the two reads overlap
  const int tfirst = g * s.tbin, tlast = min(s.S, tfirst + s.tbin);
  const int tps = kSubPairs / s.R;  // tokens per piece
  const int32_t* selh = sel + (size_t)bh * s.S * s.R;
  int v[kSubPairs / kScatterThreads];
  auto load_piece = [&](int t0) __attribute__((always_inline)) {  // contiguous: pair p is selh[t0 R + p]
    const int np = min(tps, tlast - t0) * s.R;
#pragma unroll
    for (int u = 0; u < kSubPairs / kScatterThreads; ++u) {
      const int x = u * kScatterThreads + tid;
      v[u] = x < np ? selh[(size_t)t0 * s.R + x] : -1;
    }
  };
  load_piece(tfirst);
  const int32_t* ph = phist + pair_counts_row(s, bh, 0);
  for (int i = tid; i < ne; i += kScatterThreads) {
    int v[kMaxBinRanges];  // every range's count requested at once
#pragma unroll
    for (int gg = 0; gg < kMaxBinRanges; ++gg) v[gg] = gg < s.ng ? ph[(size_t)gg * ne + i] : 0;
    int tot = 0, pre = 0;
#pragma unroll
    for (int gg = 0; gg < kMaxBinRanges; ++gg) {
      tot += v[gg];
      pre += gg < g ? v[gg] : 0;
    }
    start[i] = tot;
    base[i] = pre;
  }
  __syncthreads();
  // block offsets and work items: thread tid owns the contiguous block segment [a0, a1)
  const int seg = (ne + kScatterThreads - 1) / kScatterThreads;
  const int a0 = min(ne, tid * seg), a1 = min(ne, a0 + seg);
  int sum = 0, isum = 0;
  for (int a = a0; a < a1; ++a) {
    sum += start[a];
    isum += (start[a] + kItemPairs - 1) / kItemPairs;
  }
  int total, itot, irun;
  int run = block_exclusive_scan2<kScatterThreads>(sum, isum, scan_tmp, &total, &itot, &irun);
  int32_t* po = poff + (size_t)bh * (ne + 1);
  int32_t* io = ioff + (size_t)bh * (ne + 1);
  int32_t* it = items + item_record(s, bh, 0);
  for (int a = a0; a < a1; ++a) {
    const int tot = start[a];
    const int ni = (tot + kItemPairs - 1) / kItemPairs;
    if (g == 0) {
      po[a] = run;
      io[a] = irun;
    }
    if (a % s.ng == g)
      for (int k = 0; k < ni; ++k) it[(size_t)(irun + k) * kItemInts] = a | (min(kItemPairs, tot - k * kItemPairs) << 16);
    istart[a] = irun;
    irun += ni;
    base[a] += run;
    start[a] = run;
    run += tot;
  }
  if (g == 0 && tid == 0) {
    po[ne] = total;
    io[ne] = itot;
  }
  for (int k = itot + g * kScatterThreads + tid; k < s.max_items; k += kScatterThreads * s.ng)
    it[(size_t)k * kItemInts] = -1;
  // within a piece, pair p (pair id (t0 + p / R) R + p % R) goes to wave p / share
  int nbits = 0;
  while ((1 << nbits) < ne) ++nbits;
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  // a token's entries are used when eligible (0 <= i <= j - L) and not repeated by an earlier entry.
  // When R divides 64 the R entries of a token sit in adjacent lanes of one wave (entry x of the piece
  // is in lane x % 64), so each lane tests its own entry against the earlier ones by lane shuffles
  // before the keys are staged; otherwise the thread that owns a token rewrites its staged row.
  const bool lane_rows = 64 % s.R == 0;  // then R is a power of two, as the block size always is
  const int rsh = __builtin_ctz(s.R), bsh = __builtin_ctz(s.blk);
  // unstable filing of pair pid into block i: the next free slot of the range's part of i's list
  auto file = [&](int i, int pid) __attribute__((always_inline)) {
    const int pos = atomicAdd(&base[i], 1) - start[i];
    if (pos >= 0 && istart[i] + pos / kItemPairs < s.max_items) items[item_pair_slot(s, bh, istart[i], pos)] = pid;
  };
  for (int t0 = tfirst; t0 < tlast; t0 += tps) {
    const int nt = min(tps, tlast - t0), np = nt * s.R;
    const int share = ((np + nwf - 1) / nwf + 63) & ~63;
    if (t0 != tfirst) load_piece(t0);  // the piece's entries, all requested at once
    if (lane_rows) {
#pragma unroll
      for (int u = 0; u < kSubPairs / kScatterThreads; ++u) {
        const int x = u * kScatterThreads + tid, r = x & (s.R - 1);
        const int e = v[u];
        bool ok = e >= 0 && e <= ((t0 + (x >> rsh)) >> bsh) - s.L;
        for (int q = 1; q < s.R; ++q) {
          const int prev = __shfl(e, lane - q < 0 ? 0 : lane - q);
          ok = ok && !(q <= r && prev == e);
        }
        v[u] = ok ? e : -1;
      }
    }
    __syncthreads();  // the previous piece is filed: its keys and the counts are free
    if (!STABLE && lane_rows) {  // the entries were tested in registers: file them from there
#pragma unroll
      for (int u = 0; u < kSubPairs / kScatterThreads; ++u)
        if (v[u] >= 0) file(v[u], t0 * s.R + u * kScatterThreads + tid);
      continue;
    }
#pragma unroll
    for (int u = 0; u < kSubPairs / kScatterThreads; ++u) keys[u * kScatterThreads + tid] = v[u];
    if (STABLE)
      for (int x = tid; x < nwf * ne; x += kScatterThreads) wc[x] = 0;
    __syncthreads();
    if (!lane_rows) {
      for (int u = tid; u < nt; u += kScatterThreads) {
        int* row = keys + u * s.R;
        const int cutoff = (t0 + u) / s.blk - s.L;
        for (int r = s.R - 1; r >= 0; --r) {
          const int e = row[r];
          bool ok = e >= 0 && e <= cutoff;
          for (int q = 0; q < r; ++q) ok = ok && row[q] != e;
          row[r] = ok ? e : -1;
        }
      }
      __syncthreads();
    }
    if (!STABLE) {
      for (int p = tid; p < np; p += kScatterThreads)
        if (keys[p] >= 0) file(keys[p], t0 * s.R + p);
      continue;
    }
    const int pw0 = min(np, wave * share), pw1 = min(np, pw0 + share);
    if (wave < nwf)
      for (int p = pw0 + lane; p < pw1; p += 64) {
        const int i = keys[p];
        if (i >= 0) atomicAdd(&wc[wave * ne + i], 1);
      }
    __syncthreads();
    for (int i = tid; i < ne; i += kScatterThreads) {
      int c = base[i];
      for (int w = 0; w < nwf; ++w) {
        const int n = wc[w * ne + i];
        wc[w * ne + i] = c;
        c += n;
      }
      base[i] = c;  // the next piece starts after this one
    }
    __syncthreads();
    if (wave < nwf) {
      int* cw = wc + wave * ne;
      for (int c0 = pw0; c0 < pw1; c0 += 64) {
        const int p = c0 + lane;
        int i = p < pw1 ? keys[p] : -1;
        const bool valid = i >= 0;
        if (!valid) i = 0;
        unsigned long long same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = (i >> b) & 1;
          const unsigned long long m1 = __ballot(bit);
          same &= bit ? m1 : ~m1;
        }
        if (valid) {
          const int rank = __popcll(same & lt);
          const int count = __popcll(same);
          const int cur = cw[i];
          const int pos = cur + rank - start[i];  // the pair's place in block i's list
          if (pos >= 0 && istart[i] + pos / kItemPairs < s.max_items)
            items[item_pair_slot(s, bh, istart[i], pos)] = t0 * s.R + p;
          __builtin_amdgcn_wave_barrier();
          if (rank == count - 1) cw[i] = cur + count;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

}  // namespace

size_t pair_scatter_lds_bytes(const Shape& s) {
  if (s.ne <= 0) return 0;
  if (scatter_waves(s.ne) < 1) return (size_t)1 << 30;  // never: ne <= 8192 leaves room for two waves
  return ((size_t)(3 + scatter_waves(s.ne)) * s.ne + kSubPairs) * 4;
}

hipError_t launch_pair_count(const Shape& s, const int32_t* sel, int32_t* phist, hipStream_t st) {
  if (s.R <= 0 || s.ne <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pair_count, dim3(s.ng, s.B * s.H), dim3(kCountThreads), (size_t)s.ne * 4, st, sel, phist, s);
  return hipGetLastError();
}

hipError_t launch_pair_scatter(const Shape& s, const int32_t* sel, const int32_t* phist, int32_t* poff,
                               int32_t* ioff, int32_t* items, hipStream_t st, bool stable) {
  if (s.R <= 0 || s.ne <= 0) return hipSuccess;
  const size_t lds = pair_scatter_lds_bytes(s);
  const void* fn = stable ? (const void*)k_pair_scatter<true> : (const void*)k_pair_scatter<false>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (stable)
    hipLaunchKernelGGL(k_pair_scatter<true>, dim3(s.ng, s.B * s.H), dim3(kScatterThreads), lds, st, sel, phist, poff,
                       ioff, items, s);
  else
    hipLaunchKernelGGL(k_pair_scatter<false>, dim3(s.ng, s.B * s.H), dim3(kScatterThreads), lds, st, sel, phist, poff,
                       ioff, items, s);
  return hipGetLastError();
}

}  // namespace mdr
