// Internal declarations shared by the HIP sources of the routed-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mdr.h"

namespace mdr {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kItemPairs = 128;     // (token, slot) pairs of one remote work item: 8 waves of 16
// A remote work item is one record of kItemInts ints: [0] = block | (pairs << 16) (-1 past the last item),
// [kItemHead + e] = the pair id t*R + r of its e-th pair, in list order (ascending token).
constexpr int kItemHead = 4;
constexpr int kItemInts = kItemHead + kItemPairs;
constexpr int kMaxBinRanges = 16;   // token ranges per (b,h) of the pair binning
constexpr int kMaxProbes = 16;
constexpr int kMaxRemote = 16;
constexpr int kMaxSubspaces = 4;
constexpr int kMaxCodesTotal = 64;  // subspaces * codes
constexpr int kMaxAddresses = 4096;
constexpr int kMaxBlocks = 8192;

// Every size of one call, resolved once on the host.
struct Shape {
  int B, H, S, D, W, blk, nb, G, C, A, cap, P, M, R, L, dtype;
  float scale;      // softmax scale (1/sqrt(D) unless given)
  float rope_base;  // mixer only
  int ne;           // blocks that some query block can see: nb - L (or 0)
  int ng;           // token ranges of the pair binning per (b,h): tokens [g tbin, (g + 1) tbin)
  int tbin;         // tokens per range, a multiple of 256 (every probe work-group lies in one range)
  int max_items;    // remote work items per (b,h), an upper bound: ne + ceil(S R / kItemPairs)
  int pin;          // remote work of (b,h) runs on XCD bh % 8 (when B H is a multiple of 8)
  int csr_lds;      // probe stage stages the posting-list CSR in LDS
  int fixed_probe;  // probe stage uses its compile-time specialisation for these sizes
  int policy;       // mdr_overflow_policy
};

constexpr int kProbeThreads = 128;  // query tokens per probe work-group (one per lane)
constexpr int kProbeFixedThreads = 256;  // the same for the compile-time specialised probe

// Device buffers of one call (workspace regions or caller-provided outputs).
struct Buffers {
  float* ksum;
  int32_t* addr;
  int32_t* off;
  int32_t* idx;
  int32_t* overflow;
  int32_t* sel;
  int32_t* ncand;
  int32_t* phist;      // [B,H,ng,ne] pairs of token range g that selected block i
  int32_t* poff;       // [B,H,ne+1] pairs selecting blocks < i (block i's list has poff[i+1] - poff[i] pairs)
  int32_t* ioff;       // [B,H,ne+1] work items of blocks < i (block i's list is in items ioff[i] .. ioff[i+1])
  int32_t* items;      // [B,H,max_items,kItemInts] remote work items: each block's pair list in pieces
  void* part_o;        // [B,H,S,R,D] remote partial outputs (normalised), io dtype
  float* part_lse;     // [B,H,S,R] remote partial: log2 of its softmax normaliser (scaled exponent units)
  void* mq;            // mixer: Q, K, V, O in [B,H,S,D]
  void* mk;
  void* mv;
  void* mo;
  void* mwt;           // mixer: Wq, Wk, Wv transposed ([H*D][W] each), then Wo transposed ([W][H*D])
  float* lse;          // [B,H,S] optional output of the attention: log2 of each token's softmax
                       // normaliser sum_s 2^(scale log2(e) q.k_s) (nullptr: not written)
  float* dvec;         // [B,H,S] backward: D_t = dO_t . O_t
  int32_t* alt;        // [B,H,nb] alternate address of each block (redirect policy)
  int32_t* roff;       // [B,H,A+1] redirect lists: per address, blocks redirected into it
  int32_t* ridx;       // [B,H,nb]  (block ids, in arrival order; -1 beyond the last)
  int32_t* rtime;      // [B,H,nb]  (the query block at which each arrives; -1 beyond the last)
  int32_t* ndrop;      // [B,H,S] optional: candidates the probed lists held but did not return
  float* amargin;      // [B,H,nb] optional: each block's smallest code-logit margin
  int32_t* probes;     // optional probe diagnostics (see ProbeExtra)
  float* sel_score;
  float* pmargin;
  float* smargin;
};

// Redirect lists and the optional per-token outputs of the probe stage beyond the selection (all null
// under the drop policy without diagnostics).
struct ProbeExtra {
  const int32_t* roff;
  const int32_t* ridx;
  const int32_t* rtime;
  int32_t* ndrop;
  int32_t* probes = nullptr;    // [B,H,S,P] the probed addresses in rank order
  float* sel_score = nullptr;   // [B,H,S,R] rerank score of each selected block
  float* pmargin = nullptr;     // [B,H,S] smallest neighbour gap of the P + 1 best address scores
  float* smargin = nullptr;     // [B,H,S] smallest neighbour gap of the R + 1 best candidate scores
};

// Streaming-decode state (one region of a caller-owned buffer each).
struct DecState {
  int32_t* ring;        // [B,H,A,cap+1]: blocks filed under the address so far, then cap slots;
                        // the n-th block filed sits in slot n % cap
  int32_t* overflow;    // [B,H] blocks evicted so far
  int32_t* summarized;  // [B,H] blocks whose summary and address are in ksum / addr
  int32_t* filed;       // [B,H] blocks filed so far (blocks 0 .. filed - 1)
  int32_t* addr;        // [B,H,nb]
  float* ksum;          // [B,H,nb,D]
};
constexpr int kDecMaxKeys = 4096;  // (R + L) * block keys per decoded token
constexpr int kDecMaxCand = 1024;  // candidates per decoded token

// Selection entry r of a token in query block j is used iff it is an eligible block
// (0 <= i <= j - L) not repeated by an earlier entry of the same token.
__device__ inline bool sel_entry_valid(const int32_t* row, int r, int j, int L) {
  const int i = row[r];
  if (i < 0 || i > j - L) return false;
  for (int p = 0; p < r; ++p)
    if (row[p] == i) return false;
  return true;
}

// Work-groups are handed to the 8 XCDs of the chip in turn (linear id mod 8), and each XCD has its
// own L2.  xcd_chunked(id, n) renumbers the n work-groups of a 1-D grid so that each XCD receives a
// contiguous run of logical indices, in order: neighbours that share data (adjacent query blocks
// reading the same K/V block) then run on the same XCD at about the same time.  A bijection on
// [0, n) for any n.
constexpr int kXcds = 8;
constexpr int kCUs = 256;  // compute units of the chip (32 per XCD)
__host__ __device__ inline int xcd_chunked(int id, int n) {
  const int x = id % kXcds, k = id / kXcds;
  const int q = n / kXcds, r = n % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// ---- index arithmetic shared by the kernels and the host self-check (mdr_selfcheck_indices), which
// runs these same functions over every launch index of a configuration and checks each result
// against the buffer it addresses.

// The remote kernel's work-group id -> (b,h, work item).  Pinned: ids cycle over the XCDs, so
// (b,h) = id % 8 + 8 (id / 8 / max_items) keeps every item of one (b,h) on one XCD.  bh >= B H: no work.
__host__ __device__ inline void remote_work_of(const Shape& s, long long id, int* bh, int* k) {
  if (s.pin) {
    const long long m = id / kXcds;
    *bh = (int)(id % kXcds + kXcds * (m / s.max_items));
    *k = (int)(m % s.max_items);
  } else {
    *bh = (int)(id / s.max_items);
    *k = (int)(id % s.max_items);
  }
}
// Short sequences: the remote attention kernel finds each block's pairs itself, with no binning
// pass before it (remote_scans), when a block's candidate tokens fit one scan: S <= kScanMaxTokens.
constexpr int kScanMaxTokens = 8192;
// The scanning remote kernel's work-group id -> (b,h, eligible block i), the blocks of one head in
// order per XCD.  A bijection onto B H ne for n = B H ne.
__host__ __device__ inline void remote_block_of(const Shape& s, int id, int n, int* bh, int* i) {
  const int wg = xcd_chunked(id, n);
  *i = wg % s.ne;
  *bh = wg / s.ne;
}
__host__ __device__ inline long long remote_grid(const Shape& s) {
  const long long bh = (long long)s.B * s.H;
  return (s.pin ? (bh + kXcds - 1) / kXcds * kXcds : bh) * s.max_items;
}
// First int of work item k's record of (b,h); pair slot of the pos-th pair of a block whose first item
// is istart.
__host__ __device__ inline size_t item_record(const Shape& s, int bh, int k) {
  return ((size_t)bh * s.max_items + k) * kItemInts;
}
__host__ __device__ inline size_t item_pair_slot(const Shape& s, int bh, int istart, int pos) {
  return item_record(s, bh, istart + pos / kItemPairs) + kItemHead + pos % kItemPairs;
}
// Row of pair counts of the token range holding token t0, of (b,h).
__host__ __device__ inline size_t pair_counts_row(const Shape& s, int bh, int t0) {
  return ((size_t)bh * s.ng + t0 / s.tbin) * s.ne;
}
// First key row of block i of (b,h); the (token, slot) pair pid's partial (times D for its output row).
__host__ __device__ inline size_t block_row(const Shape& s, int bh, int i) {
  return (size_t)bh * s.S + (size_t)i * s.blk;
}
__host__ __device__ inline size_t partial_index(const Shape& s, int bh, int pid) {
  return (size_t)bh * s.S * s.R + pid;
}
// The query-block kernels' work-group id -> ((b,h), query block j), query blocks of one head in order
// per XCD.
__host__ __device__ inline void query_block_of(const Shape& s, int id, int n, int* bh, int* j) {
  const int wg = xcd_chunked(id, n);
  *j = wg % s.nb;
  *bh = wg / s.nb;
}

// Pair binning.  The counters phist are cleared column by column: the work-group that summarises block
// i clears entry i of every token range of its (b,h).
__device__ inline void clear_pair_counts(int32_t* phist, const Shape& s, int bh, int i, int tid, int nthreads) {
  if (i >= s.ne) return;
  int32_t* col = phist + pair_counts_row(s, bh, 0) + i;
  for (int g = tid; g < s.ng; g += nthreads) col[(size_t)g * s.ne] = 0;
}

// Adds the pairs a work-group of NT threads selected to the counters of its token range: each thread
// passes its pairs' blocks to add(); an LDS histogram (cnt, ne ints, or nullptr when the blocks do not
// fit: then every pair is one device-scope atomic) collects them, then each non-empty block is one
// device-scope atomic add.  Every thread of the work-group must call begin() and end().
template <int NT>
struct PairCounter {
  int* cnt;
  int32_t* dst;  // phist row of this (b,h, range)
  int ne;
  __device__ void begin() {  // cnt may alias LDS the work-group used before: every such use is done first
    __syncthreads();
    if (cnt)
      for (int i = threadIdx.x; i < ne; i += NT) cnt[i] = 0;
    __syncthreads();
  }
  __device__ void add(int i) {
    if (cnt)
      atomicAdd(&cnt[i], 1);
    else
      atomicAdd(&dst[i], 1);
  }
  __device__ void end() {
    __syncthreads();
    if (cnt)
      for (int i = threadIdx.x; i < ne; i += NT) {
        const int c = cnt[i];
        if (c) atomicAdd(&dst[i], c);
      }
  }
};

// Work-group barrier that orders LDS accesses only: global loads still in flight stay in flight
// across it (the fences are restricted to the local address space).  Used where a barrier
// protects LDS data only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive scan of one int per thread over a work-group of NT threads (NT a multiple of 64).
// tmp holds NT/64 ints.  Returns the exclusive prefix; *total receives the sum.
template <int NT>
__device__ inline int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  lds_barrier();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int tw = tmp[w];
    before += (w < wave) ? tw : 0;
    sum += tw;
  }
  lds_barrier();
  *total = sum;
  return before + x - v;
}

// Two exclusive scans at once (a and b per thread, NT a multiple of 64), with the barriers of one.
// tmp holds 2 NT/64 ints.  Returns a's exclusive prefix, *b_before b's; *total_a, *total_b the sums.
template <int NT>
__device__ inline int block_exclusive_scan2(int a, int b, int* tmp, int* total_a, int* total_b, int* b_before) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = a, y = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int xa = __shfl_up(x, o), yb = __shfl_up(y, o);
    if (lane >= o) {
      x += xa;
      y += yb;
    }
  }
  if (lane == 63) {
    tmp[wave] = x;
    tmp[NW + wave] = y;
  }
  lds_barrier();
  int ba = 0, sa = 0, bb = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int ta = tmp[w], tb = tmp[NW + w];
    ba += (w < wave) ? ta : 0;
    bb += (w < wave) ? tb : 0;
    sa += ta;
    sb += tb;
  }
  lds_barrier();
  *total_a = sa;
  *total_b = sb;
  *b_before = bb + y - b;
  return ba + x - a;
}

// Profiling events: entry i of an optional event array is recorded on the stream when present
// (a null array or a null entry records nothing).
inline hipError_t mark_event(hipEvent_t* ev, int i, hipStream_t st) {
  return ev && ev[i] ? hipEventRecord(ev[i], st) : hipSuccess;
}

// Launchers (return hipGetLastError()).
// pair_zero (optional): the address kernel of block i clears column i of the pair counters.
// Blocks [i0, i0 + n) (n < 0: to the end).
// alt (optional): also the alternate address of each block (runner-up code of its lowest-margin
// subspace).  amargin (optional): each block's smallest top1 - top2 code-logit margin.
hipError_t launch_address(const Shape& s, const void* k, const float* codebook, const float* bias,
                          float* ksum, int32_t* addr, int32_t* pair_zero, hipStream_t st, int i0 = 0, int n = -1,
                          int32_t* alt = nullptr, float* amargin = nullptr);
hipError_t launch_post(const Shape& s, const int32_t* addr, int32_t* off, int32_t* idx,
                       int32_t* overflow, hipStream_t st);
// Posting lists built inside the probe kernel (from the block addresses) instead of read: every
// work-group builds its (b,h)'s CSR in LDS and work-group 0 of each (b,h) also writes it out.
struct FusedPost {
  const int32_t* addr;
  int32_t* off;
  int32_t* idx;
  int32_t* overflow;
};
// phist (optional): the selected pairs are counted per (token range, remote block) for the binning.
hipError_t launch_probe_rerank(const Shape& s, const void* q, const float* codebook, const float* bias,
                               const float* ksum, const int32_t* off, const int32_t* idx,
                               const int32_t* force, int32_t* sel, int32_t* ncand, int32_t* phist,
                               hipStream_t st, const FusedPost* fuse = nullptr,
                               const ProbeExtra& ex = ProbeExtra{nullptr, nullptr, nullptr, nullptr});
// Redirect lists from the posting CSR and the alternates; overwrites overflow with the blocks no
// final view returns.
hipError_t launch_post_redirect(const Shape& s, const int32_t* addr, const int32_t* alt, const int32_t* off,
                                const int32_t* idx, int32_t* roff, int32_t* ridx, int32_t* rtime,
                                int32_t* overflow, hipStream_t st);
// True when launch_probe_rerank accepts `fuse` for this shape (the compile-time specialised probe).
bool probe_fuses_post(const Shape& s);
bool probe_fuses_post_nt(const Shape& s, int nt);
// Query tokens per work-group of the routing path's probe (256, or 128 / 64 on small grids).
int probe_fixed_tokens(const Shape& s);
// LDS of the probe kernel (the generic kernel, or the fixed one with nt threads and, when diag, the
// diagnostics outputs; the default is the largest form).
size_t probe_lds_bytes(const Shape& s, int nt = kProbeFixedThreads, bool diag = true);
// Decode: file blocks [filed, target) of every (b,h) (summarising those not summarised yet), then
// route and attend tokens pos .. pos + n_new - 1 (one query block).
hipError_t launch_ring_reset(int32_t* ring, long long records, int cap, hipStream_t st);
hipError_t launch_decode_file(const Shape& s, const void* k_cache, const float* codebook, const float* bias,
                              const DecState& d, int target, hipStream_t st);
hipError_t launch_decode_attend(const Shape& s, const void* q_new, const void* k_cache, const void* v_cache,
                                const float* codebook, const float* bias, const DecState& d,
                                const int32_t* force, int pos, int n_new, void* out, int32_t* sel,
                                hipStream_t st);
bool probe_fixed_shape(const Shape& s);
hipError_t launch_fill(int32_t* p, long long n, int32_t value, hipStream_t st);
// Pair binning of a selection: launch_pair_count writes every token range's row of counts (the probe
// kernels count their own selections instead, into counters the address kernel clears);
// launch_pair_scatter turns the counts into the per-block lists, cut into the remote work items
// (stable: ascending token within a block, for the backward's fixed summation order; otherwise the
// order within each token range's part of a list is arbitrary, which the forward's results do not
// depend on).
hipError_t launch_pair_count(const Shape& s, const int32_t* sel, int32_t* phist, hipStream_t st);
hipError_t launch_pair_scatter(const Shape& s, const int32_t* sel, const int32_t* phist, int32_t* poff,
                               int32_t* ioff, int32_t* items, hipStream_t st, bool stable);
size_t pair_scatter_lds_bytes(const Shape& s);
size_t remote_lds_bytes(const Shape& s);
// True when the forward's remote attention scans the selection itself (k_attn_remote_scan: S <=
// kScanMaxTokens, R <= 2, its LDS fits): no pair binning runs, and the probe kernels need not count.
bool remote_scans(const Shape& s);
// True when the forward's remote pairs go through the binning (pair counts, scatter, work items).
inline bool pairs_binned(const Shape& s) { return s.R > 0 && s.ne > 0 && !remote_scans(s); }
// The attention of a selection whose pairs are binned (items).  ev (optional, 2 entries):
// recorded before attn_remote and attn_local.
hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v,
                         const int32_t* sel, void* out, const Buffers& b, hipStream_t st,
                         hipEvent_t* ev = nullptr);
// Backward of the attention under a fixed selection (poff / ioff / items must hold the selection's pairs;
// part_o receives the remote dQ shares, dvec the row dots).  ev (optional, 3 entries): recorded before
// the row-dot, key-block and query-block kernels.
hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel,
                                  const void* out, const float* lse, const void* d_out, void* dq, void* dk, void* dv,
                                  const Buffers& b, hipStream_t st, hipEvent_t* ev = nullptr);
hipError_t launch_project_heads(const Shape& s, const void* x, const void* w, void* out, bool rope,
                                hipStream_t st);
// wt (optional): the transposed weights (4 * W * H * D elements, launch_transpose_weights); without it
// the simple tiled product is used.
hipError_t launch_project_out(const Shape& s, const void* o, const void* wo, void* delta, void* wt,
                              hipStream_t st);
// True when launch_project_out with wt takes the tiled product on the transposed Wo.
bool project_out_tiled(const Shape& s);
// The mixer's weights transposed into wt in one launch: matrices first .. first + count - 1 of
// (Wq, Wk, Wv, Wo), matrix z at wt + z W H D (k-contiguous rows for the tiled products).
hipError_t launch_transpose_weights(const Shape& s, const void* wq, const void* wk, const void* wv, const void* wo,
                                    void* wt, int first, int count, hipStream_t st);
// Q, K, V projections with RoPE, block summaries and addresses (and alternates when alt is given)
// fused into one launch, on the weights launch_transpose_weights wrote to wt; pair_zero (optional) as
// for launch_address.  Only when qkv_fuses_address.
bool qkv_fuses_address(const Shape& s);
hipError_t launch_qkv_fused(const Shape& s, const void* x, void* q, void* k, void* v, const float* cb,
                            const float* bias, float* ksum, int32_t* addr, int32_t* alt, int32_t* pair_zero,
                            const void* wt, hipStream_t st, float* amargin = nullptr);

}  // namespace mdr
