// Selected-set attention of Monodratic routed sparse causal attention on gfx950.
//
// The method runs exact causal softmax over the tokens of the selected remote blocks and the
// guaranteed local blocks, with no approximation after selection (aitechinspire.com write-up,
// "Snapshot: key facts from the report" and "What's the core idea?"; remio.ai, "Monodratic
// claims learned routing can make sparse causal attention more selective", section "Monodratic
// turns sparse attention into a retrieval decision").  Selecting whole blocks keeps data
// movement regular (same article, section "Why learned product-hash routing matters now").
//
// Routing is per query token, so the remote blocks of neighbouring tokens differ.  Reading
// each token's remote blocks separately would move every block many times, so the remote part
// is regrouped by block:
//   pairs          each selected (token, slot) pair is appended to the cell (remote block i, query
//                  block j) -- by the probe kernel, or by k_pair_bin when a selection is passed in;
//                  only the work-group owning query block j writes a cell, so no counter is hot
//   k_attn_remote  one work-group per selected block (split when blocks are heavy): the block's
//                  K/V is staged in LDS once, its pair ids go to an LDS list during the cell scan,
//                  its pairs are walked 128 at a time (16 per wave), the pairs' queries are
//                  gathered, S^T = K Q^T and O^T = V^T P^T run on MFMA, and each pair's softmax
//                  partial (max, sum, normalised output) is stored
//   k_attn_local   one work-group per query block: the L local blocks through LDS on MFMA with
//                  the causal mask on the diagonal block and an online softmax, then the
//                  remote partials of each token are merged in slot order and O is written.
//
// MFMA lane layouts (gfx950, 64 lanes): for v_mfma_f32_16x16x32_bf16 lane l supplies
// A[l%16][8(l/16)+e] and B[8(l/16)+e][l%16], e = 0..7, and receives C[4(l/16)+k][l%16],
// k = 0..3; for v_mfma_f32_16x16x4_f32 lane l supplies A[l%16][l/16] and B[l/16][l%16].
// Scores are computed transposed (keys as rows, queries as columns) so each lane keeps one
// query (l%16) through the softmax and the PV product.
#include "mdr_internal.h"
#include "mdr_tiles.h"

#include <math.h>

#include <type_traits>

namespace mdr {

namespace {

using namespace tiles;

// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fill(int32_t* p, long long n, int32_t value) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = value;
}

__global__ __launch_bounds__(256) void k_pair_bin(const int32_t* __restrict__ sel, int32_t* __restrict__ cellcnt,
                                                  int32_t* __restrict__ bins, Shape s) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (t >= s.S) return;
  const int j = t / s.blk;
  const int32_t* row = sel + ((size_t)bh * s.S + t) * s.R;
  for (int r = 0; r < s.R; ++r)
    if (sel_entry_valid(row, r, j, s.L)) record_pair(cellcnt, bins, s, bh, row[r], j, t, r);
}

// One work-group per (remote block i, split): the pairs of block i are the concatenation of its
// cells (i, j), j = i + L .. nb - 1.  The work-group scans the cell counts into LDS, stages the
// block's K/V in LDS once, and walks its pairs kRemoteWaves * 16 at a time (iteration c goes to
// split c % splits): each wave gathers 16 pairs' queries, S^T = K Q^T and O^T = V^T P^T run on
// MFMA, and every pair's softmax partial is stored at [token][slot].  The next iteration's pair
// ids and query rows are loaded before the current one is computed.
//
// Each cell's dense slots are read together with its count, so the first pair ids of every cell
// are known when the scan ends: they are written to an LDS pair list in pair order and a pair's id
// is then one LDS read.  Pairs past a cell's dense slots, or past the list's capacity, take the
// other route (the cell by binary search over the prefix, then the id from the cell's row).
constexpr int kRemoteWaves = 8;

// Capacity of the remote kernel's LDS pair list: what is left of the LDS once the work-groups
// that the K/V tile and the cell prefix allow (at most four: 32 waves per CU) have their share,
// at most 2048 and a multiple of 64.  Host and device compute it from the same values.
__host__ __device__ inline int remote_pair_cap(size_t kv_bytes, int ne) {
  const size_t lim = 159 * 1024;  // 160 KiB less a margin for the static scratch
  const size_t base = kv_bytes + (size_t)(ne + 1) * 4;
  if (base >= lim) return 0;
  size_t nwg = lim / base;
  if (nwg > 4) nwg = 4;
  size_t cap = (lim / nwg - base) / 4;
  if (cap > 2048) cap = 2048;
  return (int)(cap & ~(size_t)63);
}

template <typename T, int D, int BLK>
__global__ __launch_bounds__(kRemoteWaves * 64) void k_attn_remote(const T* __restrict__ Q, const T* __restrict__ K,
                                                                   const T* __restrict__ V,
                                                                   const int32_t* __restrict__ cellcnt,
                                                                   const int32_t* __restrict__ bins,
                                                                   T* __restrict__ part_o, float* __restrict__ part_ml,
                                                                   Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = kRemoteWaves * 64;
  constexpr int PER_IT = kRemoteWaves * 16;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vx = Ks + TL::K_ELEMS;
  int* pre = (int*)(Vx + TL::V_ELEMS);  // [ne + 1] exclusive prefix of the cell counts
  int* plist = pre + s.ne + 1;           // [pcap] pair ids in pair order (-2: read from the cell row)
  const int pcap = remote_pair_cap(TL::LDS_BYTES, s.ne);
  __shared__ int scan_tmp[kRemoteWaves];
  const int i = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncell = s.ne - i;
  const long long row0 = (long long)bh * s.cells_per_bh + cell_row(i, s.ne);
  const size_t rowbase = (size_t)bh * s.S;
  // the block's K/V is requested before the cell counts are scanned
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + (rowbase + (size_t)i * BLK) * D, V + (rowbase + (size_t)i * BLK) * D, tid);
  int run = 0;
  for (int c0 = 0; c0 < ncell; c0 += NTHR) {
    const int c = c0 + tid;
    int v = 0;
    int4 dense = make_int4(-1, -1, -1, -1);
    if (c < ncell) {  // the count and the dense slots in one round trip
      v = cellcnt[row0 + c];
      dense = *(const int4*)(bins + (row0 + c) * kCellDense);
      v = min(v, BLK);
    }
    int tot;
    const int ex = block_exclusive_scan<NTHR>(v, scan_tmp, &tot);
    if (c < ncell) {
      const int b0 = run + ex;
      pre[c] = b0;
      const int n = min(v, pcap - b0);  // entries of this cell that fall inside the list
      for (int p = 0; p < n; ++p)
        plist[b0 + p] = p == 0 ? dense.x : p == 1 ? dense.y : p == 2 ? dense.z : p == 3 ? dense.w : -2;
    }
    run += tot;
  }
  if (tid == 0) pre[ncell] = run;
  const int total = run;
  const int nit = (total + PER_IT - 1) / PER_IT;
  if ((int)blockIdx.z >= nit) return;  // uniform for the work-group
  kv.store(Ks, Vx, tid);
  __syncthreads();
  const float c = s.scale * kLog2e;
  // pair id of this lane's slot in iteration it (-1 when past the end)
  auto pair_at = [&](int it) __attribute__((always_inline)) -> int {
    const int pidx = it * PER_IT + wave * 16 + (lane & 15);
    if (pidx >= total) return -1;
    if (pidx < pcap) {
      const int p = plist[pidx];
      if (p != -2) return p;
    }
    int lo = 0, hi = ncell - 1;  // the cell whose range holds pidx
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= pidx)
        lo = mid;
      else
        hi = mid - 1;
    }
    return cell_pair(bins, s, row0 + lo, pidx - pre[lo]);
  };
  int it = blockIdx.z;
  if (it * PER_IT + wave * 16 >= total) return;  // this wave has no pairs at all (no barriers below)
  // software pipeline over this wave's iterations: the next pair id is requested before the current
  // tile is scored and its query row right after, so neither read waits on the other's round trip
  int cur = pair_at(it);
  QFrag<T, D> qf;
  load_q<T, D>(qf, Q + (rowbase + (cur < 0 ? 0 : cur / s.R)) * D, lane);
  for (; it < nit; it += gridDim.z) {
    const int nx = it + (int)gridDim.z;
    const bool more = nx < nit && nx * PER_IT + wave * 16 < total;  // uniform per wave
    const int nxt = more ? pair_at(nx) : -1;
    // softmax in base 2 with the scale folded in: p = 2^(c s - c max s), c = scale * log2(e) > 0
    f32x4 p[TL::NT];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < TL::NT; ++n) {
      p[n] = score_tile<T, D, BLK>(qf, Ks, n, lane);
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = fmaxf(mx, p[n][k]);
    }
    mx = c * wave_max16(mx);
    float sum = 0.f;
#pragma unroll
    for (int n = 0; n < TL::NT; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p[n][k] = fast_exp2(fmaf(p[n][k], c, -mx));
        sum += p[n][k];
      }
    sum = wave_sum16(sum);
    f32x4 o[TL::ND];
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    pv_block<T, D, BLK>(o, p, Vx, lane);
    if (more) load_q<T, D>(qf, Q + (rowbase + (nxt < 0 ? 0 : nxt / s.R)) * D, lane);
    if (cur >= 0) {
      const int t = cur / s.R, r = cur % s.R;
      const size_t pr = (rowbase + t) * s.R + r;
      const float inv = 1.f / sum;
#pragma unroll
      for (int dt = 0; dt < TL::ND; ++dt) store4<T>(part_o + pr * D + 16 * dt + 4 * (lane >> 4), o[dt], inv);
      if ((lane >> 4) == 0) *(float2*)(part_ml + 2 * pr) = make_float2(mx, sum);
    }
    if (!more) break;
    cur = nxt;
  }
}

// One work-group per query block: local blocks + merge of the remote partials.  Every read that
// does not depend on another is issued at the start: the query rows, the first local block of K/V
// (held in registers until the LDS takes it; each later block is read while the previous one is
// scored), the selection row and the first RS = min(R, 2) remote partials (their addresses do not
// depend on the selection; unused ones are ignored).  RS is a template argument so that these
// reads form one straight-line block the compiler need not wait on early.

// bf16 tiles with D <= 64 are held to four waves per SIMD (four 256-thread work-groups per CU).
constexpr int local_min_waves(int bytes, int D) { return bytes == 2 && D <= 64 ? 4 : 1; }

template <typename T, int D, int BLK, int RS>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(local_min_waves((int)sizeof(T), D)))) void k_attn_local(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const int32_t* __restrict__ sel,
    const T* __restrict__ part_o, const float* __restrict__ part_ml, T* __restrict__ out,
    float* __restrict__ lse, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = BLK * 4;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vx = Ks + TL::K_ELEMS;
  const int wg = xcd_chunked(blockIdx.x, gridDim.x);  // query blocks of one head in order per XCD
  const int j = wg % s.nb, bh = wg / s.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave * 16 + (lane & 15);
  const int t = j * BLK + qi;
  const int c4 = 4 * (lane >> 4);
  const size_t rowbase = (size_t)bh * s.S;
  const int j0 = max(0, j - s.L + 1);
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + (rowbase + (size_t)j0 * BLK) * D, V + (rowbase + (size_t)j0 * BLK) * D, tid);
  QFrag<T, D> qf;
  load_q<T, D>(qf, Q + (rowbase + t) * D, lane);
  // reads complete in issue order: keep the K/V and query reads ahead of the partials, which are
  // needed last
  __builtin_amdgcn_sched_barrier(0);
  const int32_t* row = sel + (rowbase + t) * s.R;
  constexpr int RA = RS > 0 ? RS : 1;
  int sr[RA];
  float2 pml[RA];
  Raw4<T> praw[RA][TL::ND];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const size_t pr = (rowbase + t) * s.R + r;
    sr[r] = row[r];
    pml[r] = *(const float2*)(part_ml + 2 * pr);
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) praw[r][dt] = *(const Raw4<T>*)(part_o + pr * D + 16 * dt + c4);
  }
  const float c = s.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4 o[TL::ND];
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one local block: stage it, score it, fold it into the running (m, l, o); only the diagonal
  // block (jj == j) needs the causal mask
  auto block_step = [&](auto diag_tag, int jj) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    if (jj != j0) __syncthreads();  // the previous block is no longer read
    kv.store(Ks, Vx, tid);
    __syncthreads();
    if (jj < j) {  // the next block's read overlaps this block's softmax
      const size_t nx = (rowbase + (size_t)(jj + 1) * BLK) * D;
      kv.load(K + nx, V + nx, tid);
    }
    f32x4 p[TL::NT];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < TL::NT; ++n) {
      p[n] = score_tile<T, D, BLK>(qf, Ks, n, lane);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (DIAG && 16 * n + c4 + k > qi) p[n][k] = -INFINITY;
        mx = fmaxf(mx, p[n][k]);
      }
    }
    // base-2 softmax with the scale folded in (c = scale * log2(e) > 0); m is kept in scaled units
    const float mnew = fmaxf(m, c * wave_max16(mx));
    const float alpha = fast_exp2(m - mnew);
    float sum = 0.f;
#pragma unroll
    for (int n = 0; n < TL::NT; ++n)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p[n][k] = fast_exp2(fmaf(p[n][k], c, -mnew));
        sum += p[n][k];
      }
    sum = wave_sum16(sum);
    l = l * alpha + sum;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) o[dt] *= alpha;
    pv_block<T, D, BLK>(o, p, Vx, lane);
  };
  if (s.L == 2 && j >= 1) {
    // the common window, written out without a loop so that the compiler tracks every read in
    // flight precisely (a loop header merges that state and forces early waits)
    block_step(std::false_type{}, j - 1);
    block_step(std::true_type{}, j);
  } else {
    for (int jj = j0; jj < j; ++jj) block_step(std::false_type{}, jj);
    block_step(std::true_type{}, j);
  }
  // merge the remote partials in slot order: entry r counts when 0 <= sel <= j - L and it does not
  // repeat an earlier entry of the row
  auto merge = [&](float2 ml, const Raw4<T> (&po)[TL::ND]) __attribute__((always_inline)) {
    const float mnew = fmaxf(m, ml.x);
    const float a = fast_exp2(m - mnew);
    const float b = fast_exp2(ml.x - mnew) * ml.y;
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) o[dt] = o[dt] * a + unpack4<T>(po[dt]) * b;
    l = l * a + b;
    m = mnew;
  };
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    bool ok = sr[r] >= 0 && sr[r] <= j - s.L;
#pragma unroll
    for (int p = 0; p < r; ++p) ok = ok && sr[p] != sr[r];
    if (ok) merge(pml[r], praw[r]);
  }
  for (int r = RS; r < s.R; ++r) {
    if (!sel_entry_valid(row, r, j, s.L)) continue;
    const size_t pr = (rowbase + t) * s.R + r;
    Raw4<T> po[TL::ND];
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) po[dt] = *(const Raw4<T>*)(part_o + pr * D + 16 * dt + c4);
    merge(*(const float2*)(part_ml + 2 * pr), po);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) store4<T>(out + (rowbase + t) * D + 16 * dt + c4, o[dt], inv);
  if (lse && c4 == 0) lse[rowbase + t] = m + log2f(l);
}

template <typename T, int D, int BLK, int RS>
hipError_t launch_local(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                        const Buffers& b, hipStream_t st) {
  const size_t lds = Tile<T, D, BLK>::LDS_BYTES;
  hipError_t e;
  if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_attn_local<T, D, BLK, RS>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  hipLaunchKernelGGL((k_attn_local<T, D, BLK, RS>), dim3(s.nb * s.B * s.H), dim3(BLK * 4), lds, st, (const T*)q,
                     (const T*)k, (const T*)v, sel, (const T*)b.part_o, b.part_ml, (T*)out, b.lse, s);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t attend_impl(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                       const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  const bool remote = s.R > 0 && s.ne > 0;
  hipError_t e;
  if ((e = mark_event(ev, 0, st)) != hipSuccess) return e;
  if (remote) {
    const size_t rl = remote_lds_bytes(s);
    if (rl > 65536 && (e = hipFuncSetAttribute((const void*)k_attn_remote<T, D, BLK>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)rl)) != hipSuccess)
      return e;
    hipLaunchKernelGGL((k_attn_remote<T, D, BLK>), dim3(s.ne, s.B * s.H, s.split), dim3(kRemoteWaves * 64), rl, st,
                       (const T*)q,
                       (const T*)k, (const T*)v, b.cellcnt, b.bins, (T*)b.part_o, b.part_ml, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark_event(ev, 1, st)) != hipSuccess) return e;
  return s.R >= 2   ? launch_local<T, D, BLK, 2>(s, q, k, v, sel, out, b, st)
         : s.R == 1 ? launch_local<T, D, BLK, 1>(s, q, k, v, sel, out, b, st)
                    : launch_local<T, D, BLK, 0>(s, q, k, v, sel, out, b, st);
}

template <typename T, int D>
size_t remote_lds_d(const Shape& s) {
  switch (s.blk) {
    case 32: return Tile<T, D, 32>::LDS_BYTES;
    case 64: return Tile<T, D, 64>::LDS_BYTES;
    default: return Tile<T, D, 128>::LDS_BYTES;
  }
}

template <typename T>
size_t remote_lds_t(const Shape& s) {
  switch (s.D) {
    case 32: return remote_lds_d<T, 32>(s);
    case 64: return remote_lds_d<T, 64>(s);
    default: return remote_lds_d<T, 128>(s);
  }
}

template <typename T, int D>
hipError_t attend_blk(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                      const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  switch (s.blk) {
    case 32: return attend_impl<T, D, 32>(s, q, k, v, sel, out, b, st, ev);
    case 64: return attend_impl<T, D, 64>(s, q, k, v, sel, out, b, st, ev);
    case 128: return attend_impl<T, D, 128>(s, q, k, v, sel, out, b, st, ev);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t attend_d(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                    const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  switch (s.D) {
    case 32: return attend_blk<T, 32>(s, q, k, v, sel, out, b, st, ev);
    case 64: return attend_blk<T, 64>(s, q, k, v, sel, out, b, st, ev);
    case 128: return attend_blk<T, 128>(s, q, k, v, sel, out, b, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fill(int32_t* p, long long n, int32_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

hipError_t launch_pair_bin(const Shape& s, const int32_t* sel, int32_t* cellcnt, int32_t* bins, hipStream_t st) {
  hipLaunchKernelGGL(k_pair_bin, dim3((s.S + 255) / 256, s.B * s.H), dim3(256), 0, st, sel, cellcnt, bins, s);
  return hipGetLastError();
}

size_t remote_lds_bytes(const Shape& s) {
  const size_t kv = s.dtype == MDR_BF16 ? remote_lds_t<bf16>(s) : remote_lds_t<float>(s);
  return kv + (size_t)(s.ne + 1) * 4 + (size_t)remote_pair_cap(kv, s.ne) * 4;
}

hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                         const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  if (s.dtype == MDR_BF16) return attend_d<bf16>(s, q, k, v, sel, out, b, st, ev);
  return attend_d<float>(s, q, k, v, sel, out, b, st, ev);
}

}  // namespace mdr
