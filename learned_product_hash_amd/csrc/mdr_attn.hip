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
//   pairs          the selected (token, slot) pairs are binned by remote block (mdr_pairs.hip): each
//                  block's list by token range, cut into work items of kItemPairs pair ids (a pair's
//                  partial depends on its own query alone, not on its place in the list)
//   k_attn_remote  one work-group per work item: the block's K/V is staged in LDS, the item's pairs
//                  go 16 per wave, their queries are gathered, S^T = K Q^T and O^T = V^T P^T run on
//                  MFMA, and each pair's softmax partial (normalised output, log2 normaliser) is
//                  stored at [token][slot].  The items of one (b,h) run on one XCD when the heads
//                  divide evenly, so that head's query rows and partials share that XCD's L2
//   k_attn_remote_scan  short sequences (at most kScanMaxTokens tokens, R <= 2): the same partials,
//                  one work-group per (b,h, block), which finds the block's pairs in the selection
//                  itself, so no binning pass runs
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

// One wave's 16 (token, slot) pairs against the block staged in Ks / Vx: lane l's query is pair
// l % 16 (qf, read from that pair's token row), pid its pair id t R + r (< 0: no pair, nothing is
// stored).  Each pair's partial -- the output row normalised by its own sum and the log2 normaliser --
// goes to [token][slot].  A pair's products depend on its own query column alone, so the partial does
// not depend on which other pairs share the wave.
template <typename T, int D, int BLK>
__device__ __forceinline__ void remote_partials(const QFrag<T, D>& qf, const T* Ks, const T* Vx, int pid, int bh,
                                                const Shape& s, T* __restrict__ part_o,
                                                float* __restrict__ part_lse, int lane) {
  using TL = Tile<T, D, BLK>;
  // softmax in base 2 with the scale folded in: p = 2^(c s - c max s), c = scale * log2(e) > 0
  const float c = s.scale * kLog2e;
  f32x4 p[TL::NT];
  float mx = -INFINITY;
#pragma unroll
  for (int nn = 0; nn < TL::NT; ++nn) {
    p[nn] = score_tile<T, D, BLK>(qf, Ks, nn, lane);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mx = fmaxf(mx, p[nn][kk]);
  }
  mx = c * wave_max16(mx);
  float sum = 0.f;
#pragma unroll
  for (int nn = 0; nn < TL::NT; ++nn)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      p[nn][kk] = fast_exp2(fmaf(p[nn][kk], c, -mx));
      sum += p[nn][kk];
    }
  sum = wave_sum16(sum);
  f32x4 o[TL::ND];
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  pv_block<T, D, BLK>(o, p, Vx, lane);
  if (pid >= 0) {
    const size_t pr = partial_index(s, bh, pid);  // the pair (token, slot)
    const float inv = 1.f / sum;
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) store4<T>(part_o + pr * D + 16 * dt + 4 * (lane >> 4), o[dt], inv);
    if ((lane >> 4) == 0) part_lse[pr] = mx + log2f(sum);
  }
}

// One work-group per remote work item: kItemPairs pairs (or fewer) of one block's pair list, 16 per
// wave.  The item record (block and pair ids in one read), then the block's K/V and the pairs' query
// rows: two dependent reads ahead of the products.
constexpr int kRemoteWaves = kItemPairs / 16;

template <typename T, int D, int BLK>
__global__ __launch_bounds__(kRemoteWaves * 64) void k_attn_remote(const T* __restrict__ Q, const T* __restrict__ K,
                                                                   const T* __restrict__ V,
                                                                   const int32_t* __restrict__ items,
                                                                   T* __restrict__ part_o, float* __restrict__ part_lse,
                                                                   Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = kRemoteWaves * 64;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vx = Ks + TL::K_ELEMS;
  // work item k of (b,h) (its items on one XCD when pinned)
  int bh, k;
  remote_work_of(s, blockIdx.x, &bh, &k);
  if (bh >= s.B * s.H) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = wave * 16 + (lane & 15);
  const int32_t* rec = items + item_record(s, bh, k);
  const int hdr = rec[0];
  int pid = rec[kItemHead + e];
  if (hdr < 0) return;  // past the last item (uniform for the work-group)
  const int i = hdr & 0xffff, n = hdr >> 16;
  if (e >= n || (unsigned)pid >= (unsigned)(s.S * s.R)) pid = -1;  // only ids of this (b,h) are ever gathered
  const size_t rowbase = (size_t)bh * s.S;
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + block_row(s, bh, i) * D, V + block_row(s, bh, i) * D, tid);
  QFrag<T, D> qf;
  load_q<T, D>(qf, Q + (rowbase + (pid < 0 ? 0 : pid / s.R)) * D, lane);
  kv.store(Ks, Vx, tid);
  __syncthreads();
  if (wave * 16 >= n) return;  // no pairs for this wave (no barriers below)
  remote_partials<T, D, BLK>(qf, Ks, Vx, pid, bh, s, part_o, part_lse, lane);
}

// Short sequences (remote_scans): one work-group per (b,h, eligible block i) finds the pairs that
// selected block i itself, from the selection rows of the tokens that can see it (query blocks i + L
// and later), so that no binning pass runs before it.  Thread tid reads the rows of tokens
// t0 + c NTHR + tid; a token contributes its first entry equal to i (a repeat of an earlier entry of
// the row is not a pair).  The pair ids are compacted into LDS in ascending token order (per-wave
// ballot counts, one scan), then go 16 per wave, kItemPairs at a time, through remote_partials: the
// same partials, bit for bit, as the binned kernel's.
template <typename T, int D, int BLK, int R>
__global__ __launch_bounds__(kRemoteWaves * 64) void k_attn_remote_scan(const T* __restrict__ Q,
                                                                        const T* __restrict__ K,
                                                                        const T* __restrict__ V,
                                                                        const int32_t* __restrict__ sel,
                                                                        T* __restrict__ part_o,
                                                                        float* __restrict__ part_lse, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = kRemoteWaves * 64;
  constexpr int ROWS = kScanMaxTokens / NTHR;  // selection rows per thread
  constexpr int NC = ROWS * kRemoteWaves;      // wave counts, (row, wave)-major = ascending tokens
  static_assert(NC == 2 * 64, "the count scan takes two counts per lane of one wave");
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vx = Ks + TL::K_ELEMS;
  int32_t* cnt = (int32_t*)(Vx + TL::V_ELEMS);  // NC counts, then their exclusive scan; [NC] = total
  uint16_t* list = (uint16_t*)(cnt + NC + 4);   // the block's pair ids (below S R <= 2 kScanMaxTokens)
  int bh, i;
  remote_block_of(s, blockIdx.x, gridDim.x, &bh, &i);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t rowbase = (size_t)bh * s.S;
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + block_row(s, bh, i) * D, V + block_row(s, bh, i) * D, tid);
  const int t0 = (i + s.L) * BLK;
  int e[ROWS][R];
#pragma unroll
  for (int c = 0; c < ROWS; ++c) {
    const int t = t0 + c * NTHR + tid;
#pragma unroll
    for (int r = 0; r < R; ++r) e[c][r] = t < s.S ? sel[(rowbase + t) * R + r] : -1;
  }
  // 2 bits per row: 1 + the slot of the token's pair with block i, 0 for none
  unsigned hits = 0;
  unsigned long long bal[ROWS];
#pragma unroll
  for (int c = 0; c < ROWS; ++c) {
    int h = 0;
#pragma unroll
    for (int r = R - 1; r >= 0; --r)
      if (e[c][r] == i) h = r + 1;
    hits |= (unsigned)h << (2 * c);
    bal[c] = __ballot(h != 0);
    if (lane == 0) cnt[c * kRemoteWaves + wave] = __popcll(bal[c]);
  }
  kv.store(Ks, Vx, tid);
  __syncthreads();
  if (wave == 0) {
    const int a = cnt[2 * lane], b = cnt[2 * lane + 1];
    int x = a + b;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    cnt[2 * lane] = x - a - b;
    cnt[2 * lane + 1] = x - b;
    if (lane == 63) cnt[NC] = x;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int c = 0; c < ROWS; ++c) {
    const int h = (hits >> (2 * c)) & 3;
    if (h)
      list[cnt[c * kRemoteWaves + wave] + __popcll(bal[c] & below)] = (uint16_t)((t0 + c * NTHR + tid) * R + h - 1);
  }
  __syncthreads();
  const int n = cnt[NC];
#pragma unroll 1
  for (int base = wave * 16; base < n; base += kItemPairs) {  // no barriers in this loop
    const int e = base + (lane & 15);
    const int pid = e < n ? (int)list[e] : -1;
    QFrag<T, D> qf;
    load_q<T, D>(qf, Q + (rowbase + (pid < 0 ? 0 : pid / R)) * D, lane);
    // the tiles are read again in every round: an offset the compiler cannot see through keeps it from
    // holding the whole block's operands in registers across rounds
    int off = 0;
    asm volatile("" : "+s"(off));
    remote_partials<T, D, BLK>(qf, Ks + off, Vx + off, pid, bh, s, part_o, part_lse, lane);
  }
}

// LDS of k_attn_remote_scan: the block's K/V, the wave counts and the pair list (16-bit pair ids: every
// pair id t R + r is below kScanMaxTokens R <= 65536), sized for the most pairs a block can have, one
// per token that can see it: S - L blk.
static_assert(kScanMaxTokens * 2 <= 65536, "16-bit pair ids");
template <typename T, int D, int BLK>
size_t scan_lds_bytes(const Shape& s) {
  const size_t most = s.S > s.L * BLK ? (size_t)(s.S - s.L * BLK) : 0;
  return Tile<T, D, BLK>::LDS_BYTES + (size_t)(kScanMaxTokens / (kRemoteWaves * 64) * kRemoteWaves + 4) * 4 +
         (most * 2 + 15) / 16 * 16;
}

// One work-group per query block: local blocks + merge of the remote partials.  The selection row,
// the first local block of K/V (held in registers until the LDS takes it; each later block is read
// while the previous one is scored) and the query rows are read at the start; with the last (diagonal)
// block, the partials of the row's first RS = min(R, 2) entries are requested, only for the entries
// the token uses, so that no unused partial row is fetched (and their registers are live only
// through that block).  RS is a template argument so that these reads form one straight-line block
// the compiler need not wait on early.

// bf16 tiles are held to four waves per SIMD with D <= 64 (four 256-thread work-groups per CU) and to
// two with D = 128 (left free, that shape took one wave per SIMD).
constexpr int local_min_waves(int bytes, int D) { return bytes == 2 ? (D <= 64 ? 4 : 2) : 1; }

template <typename T, int D, int BLK, int RS, bool TAIL>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(local_min_waves((int)sizeof(T), D)))) void k_attn_local(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const int32_t* __restrict__ sel,
    const T* __restrict__ part_o, const float* __restrict__ part_lse, T* __restrict__ out,
    float* __restrict__ lse, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = BLK * 4;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vx = Ks + TL::K_ELEMS;
  int j, bh;
  query_block_of(s, blockIdx.x, gridDim.x, &bh, &j);  // query blocks of one head in order per XCD
  // walked from the last query block down: the remote kernel just before ends with the highest
  // blocks' items, so their K/V, the top tokens' query rows and partials are then still in the L2
  j = s.nb - 1 - j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave * 16 + (lane & 15);
  const int t = j * BLK + qi;
  const int c4 = 4 * (lane >> 4);
  const size_t rowbase = (size_t)bh * s.S;
  const int j0 = max(0, j - s.L + 1);
  const int32_t* row = sel + (rowbase + t) * s.R;
  constexpr int RA = RS > 0 ? RS : 1;
  int sr[RA];
#pragma unroll
  for (int r = 0; r < RS; ++r) sr[r] = row[r];
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + (rowbase + (size_t)j0 * BLK) * D, V + (rowbase + (size_t)j0 * BLK) * D, tid);
  QFrag<T, D> qf;
  load_q<T, D>(qf, Q + (rowbase + t) * D, lane);
  // the first RS partials are requested with the diagonal block, only those of used entries: entry r
  // counts when 0 <= sel <= j - L and it does not repeat an earlier entry of the row
  bool use[RA];
  float plse[RA];
  Raw4<T> praw[RA][TL::ND];
  auto request_partials = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      bool ok = sr[r] >= 0 && sr[r] <= j - s.L;
#pragma unroll
      for (int p = 0; p < r; ++p) ok = ok && sr[p] != sr[r];
      use[r] = ok;
      const size_t pr = (rowbase + t) * s.R + r;
      plse[r] = ok ? part_lse[pr] : 0.f;
#pragma unroll
      for (int dt = 0; dt < TL::ND; ++dt)
        praw[r][dt] = ok ? *(const Raw4<T>*)(part_o + pr * D + 16 * dt + c4) : Raw4<T>{};
    }
  };
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
    if (jj == j) request_partials();
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
  // merge the remote partials in slot order (the used entries above, then for R > RS the rest of the
  // row).  A partial with normalised output o_r and log2 normaliser lse_r carries the weight 2^lse_r.
  auto merge = [&](float lr, const Raw4<T> (&po)[TL::ND]) __attribute__((always_inline)) {
    const float mnew = fmaxf(m, lr);
    const float a = fast_exp2(m - mnew);
    const float b = fast_exp2(lr - mnew);
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) o[dt] = o[dt] * a + unpack4<T>(po[dt]) * b;
    l = l * a + b;
    m = mnew;
  };
#pragma unroll
  for (int r = 0; r < RS; ++r)
    if (use[r]) merge(plse[r], praw[r]);
  if constexpr (TAIL) {
    // slots RS .. R-1 (R > RS): the whole row is read at once, then the used slots' partials two at a
    // time, both requested before either is merged
    int sx[kMaxRemote];
#pragma unroll
    for (int r = 0; r < kMaxRemote; ++r) sx[r] = r < s.R ? row[r] : -1;
    auto used = [&](int r) -> bool {
      bool ok = sx[r] >= 0 && sx[r] <= j - s.L;
#pragma unroll
      for (int p = 0; p < kMaxRemote; ++p) ok = ok && (p >= r || sx[p] != sx[r]);
      return ok;
    };
#pragma unroll
    for (int r = RS; r < kMaxRemote; r += 2) {
      if (r >= s.R) break;
      const bool u0 = used(r), u1 = r + 1 < s.R && used(r + 1);
      const size_t pr = (rowbase + t) * s.R + r;
      Raw4<T> pa[TL::ND], pb[TL::ND];
      float la = 0.f, lb = 0.f;
      if (u0) {
#pragma unroll
        for (int dt = 0; dt < TL::ND; ++dt) pa[dt] = *(const Raw4<T>*)(part_o + pr * D + 16 * dt + c4);
        la = part_lse[pr];
      }
      if (u1) {
#pragma unroll
        for (int dt = 0; dt < TL::ND; ++dt) pb[dt] = *(const Raw4<T>*)(part_o + (pr + 1) * D + 16 * dt + c4);
        lb = part_lse[pr + 1];
      }
      if (u0) merge(la, pa);
      if (u1) merge(lb, pb);
    }
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) store4<T>(out + (rowbase + t) * D + 16 * dt + c4, o[dt], inv);
  if (lse && c4 == 0) lse[rowbase + t] = m + log2f(l);
}

template <typename T, int D, int BLK, int RS, bool TAIL = false>
hipError_t launch_local(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                        const Buffers& b, hipStream_t st) {
  const size_t lds = Tile<T, D, BLK>::LDS_BYTES;
  hipError_t e;
  if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_attn_local<T, D, BLK, RS, TAIL>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  hipLaunchKernelGGL((k_attn_local<T, D, BLK, RS, TAIL>), dim3(s.nb * s.B * s.H), dim3(BLK * 4), lds, st, (const T*)q,
                     (const T*)k, (const T*)v, sel, (const T*)b.part_o, b.part_lse, (T*)out, b.lse, s);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t attend_impl(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                       const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  const bool remote = s.R > 0 && s.ne > 0;
  hipError_t e;
  if ((e = mark_event(ev, 0, st)) != hipSuccess) return e;
  if (remote && remote_scans(s)) {
    const size_t rl = scan_lds_bytes<T, D, BLK>(s);
    const void* kfn = s.R == 2 ? (const void*)k_attn_remote_scan<T, D, BLK, 2> : (const void*)k_attn_remote_scan<T, D, BLK, 1>;
    if (rl > 65536 && (e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rl)) != hipSuccess)
      return e;
    const unsigned grid = (unsigned)(s.B * s.H * s.ne);
    if (s.R == 2)
      hipLaunchKernelGGL((k_attn_remote_scan<T, D, BLK, 2>), dim3(grid), dim3(kRemoteWaves * 64), rl, st, (const T*)q,
                         (const T*)k, (const T*)v, sel, (T*)b.part_o, b.part_lse, s);
    else
      hipLaunchKernelGGL((k_attn_remote_scan<T, D, BLK, 1>), dim3(grid), dim3(kRemoteWaves * 64), rl, st, (const T*)q,
                         (const T*)k, (const T*)v, sel, (T*)b.part_o, b.part_lse, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (remote) {
    const size_t rl = remote_lds_bytes(s);
    if (rl > 65536 && (e = hipFuncSetAttribute((const void*)k_attn_remote<T, D, BLK>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)rl)) != hipSuccess)
      return e;
    hipLaunchKernelGGL((k_attn_remote<T, D, BLK>), dim3((unsigned)remote_grid(s)), dim3(kRemoteWaves * 64),
                       rl, st, (const T*)q, (const T*)k, (const T*)v, b.items, (T*)b.part_o, b.part_lse, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark_event(ev, 1, st)) != hipSuccess) return e;
  return s.R > 2    ? launch_local<T, D, BLK, 2, true>(s, q, k, v, sel, out, b, st)
         : s.R == 2 ? launch_local<T, D, BLK, 2>(s, q, k, v, sel, out, b, st)
         : s.R == 1 ? launch_local<T, D, BLK, 1>(s, q, k, v, sel, out, b, st)
                    : launch_local<T, D, BLK, 0>(s, q, k, v, sel, out, b, st);
}

template <typename T, int D>
size_t scan_lds_d(const Shape& s) {
  return s.blk == 32   ? scan_lds_bytes<T, D, 32>(s)
         : s.blk == 64 ? scan_lds_bytes<T, D, 64>(s)
                       : scan_lds_bytes<T, D, 128>(s);
}

template <typename T>
size_t scan_lds_t(const Shape& s) {
  return s.D == 32 ? scan_lds_d<T, 32>(s) : s.D == 64 ? scan_lds_d<T, 64>(s) : scan_lds_d<T, 128>(s);
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

bool remote_scans(const Shape& s) {
  if (s.R < 1 || s.R > 2 || s.ne <= 0 || s.S > kScanMaxTokens) return false;
  return (s.dtype == MDR_BF16 ? scan_lds_t<bf16>(s) : scan_lds_t<float>(s)) <= 160 * 1024;
}

size_t remote_lds_bytes(const Shape& s) {
  return s.dtype == MDR_BF16 ? remote_lds_t<bf16>(s) : remote_lds_t<float>(s);
}

hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, void* out,
                         const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  if (s.dtype == MDR_BF16) return attend_d<bf16>(s, q, k, v, sel, out, b, st, ev);
  return attend_d<float>(s, q, k, v, sel, out, b, st, ev);
}

}  // namespace mdr
