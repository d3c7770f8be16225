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
constexpr int kPairsPerChunk = 64;  // (query, slot) pairs one remote work-group handles
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
  long long cells_per_bh;  // (remote block i, query block j) cells with j >= i + L: ne (ne + 1) / 2
  int split;        // remote work-groups per block
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
  int32_t* cellcnt;    // [B,H,cells] pairs per (remote block i, query block j) cell
  int32_t* bins;       // (t*R + r) of the pairs of each cell: a dense [B,H,cells,kCellDense] table of
                       // the first slots, then [B,H,cells,blk] rows (see cell_slot)
  void* part_o;        // [B,H,S,R,D] remote partial outputs (normalised), io dtype
  float* part_ml;      // [B,H,S,R,2] remote partial (max in log2 units, sum)
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
};

// Redirect lists and the dropped-candidate output of the probe stage (all null under the drop
// policy without diagnostics).
struct ProbeExtra {
  const int32_t* roff;
  const int32_t* ridx;
  const int32_t* rtime;
  int32_t* ndrop;
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

// The cells of remote block i are (i, j) for j = i + L .. nb - 1, stored contiguously; a cell
// holds the pairs of query block j that selected block i (at most blk of them).
__host__ __device__ inline long long cell_row(int i, int ne) {
  const long long ii = i;
  return ii * ne - ii * (ii - 1) / 2;
}

// Selection entry r of a token in query block j is used iff it is an eligible block
// (0 <= i <= j - L) not repeated by an earlier entry of the same token.
__device__ inline bool sel_entry_valid(const int32_t* row, int r, int j, int L) {
  const int i = row[r];
  if (i < 0 || i > j - L) return false;
  for (int p = 0; p < r; ++p)
    if (row[p] == i) return false;
  return true;
}

// Where slot pos of a cell's pair list lives.  Cells hold 1.3 pairs on average and a row of a
// block's cells is read front to back, so the first kCellDense slots of every cell sit in a dense
// table ([cells][kCellDense], consecutive cells on shared cache lines) at the start of the bins
// region; slots kCellDense .. blk - 1 sit in full-width rows ([cells][blk]) after it.
constexpr int kCellDense = 4;
__host__ __device__ inline long long cells_total(const Shape& s) { return (long long)s.B * s.H * s.cells_per_bh; }
__device__ inline int32_t* cell_slot(int32_t* bins, const Shape& s, long long cell, int pos) {
  return pos < kCellDense ? bins + cell * kCellDense + pos
                          : bins + cells_total(s) * kCellDense + cell * s.blk + pos;
}
__device__ inline int32_t cell_pair(const int32_t* __restrict__ bins, const Shape& s, long long cell, int pos) {
  return pos < kCellDense ? bins[cell * kCellDense + pos] : bins[cells_total(s) * kCellDense + cell * s.blk + pos];
}

// Append pair (t, r) of query block j to the cell (i, j).  Only the work-group that owns query
// block j touches the cell, so its counter sees at most blk atomic adds.
__device__ inline void record_pair(int32_t* cellcnt, int32_t* bins, const Shape& s, int bh, int i, int j, int t,
                                   int r) {
  const long long cell = (long long)bh * s.cells_per_bh + cell_row(i, s.ne) + (j - i - s.L);
  const int pos = atomicAdd(&cellcnt[cell], 1);
  if (pos < s.blk) *cell_slot(bins, s, cell, pos) = t * s.R + r;
}

// Work-groups are handed to the 8 XCDs of the chip in turn (linear id mod 8), and each XCD has its
// own L2.  xcd_chunked(id, n) renumbers the n work-groups of a 1-D grid so that each XCD receives a
// contiguous run of logical indices, in order: neighbours that share data (adjacent query blocks
// reading the same K/V block) then run on the same XCD at about the same time.  A bijection on
// [0, n) for any n.
constexpr int kXcds = 8;
__device__ inline int xcd_chunked(int id, int n) {
  const int x = id % kXcds, k = id / kXcds;
  const int q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + k;
}

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

// Profiling events: entry i of an optional event array is recorded on the stream when present
// (a null array or a null entry records nothing).
inline hipError_t mark_event(hipEvent_t* ev, int i, hipStream_t st) {
  return ev && ev[i] ? hipEventRecord(ev[i], st) : hipSuccess;
}

// Launchers (return hipGetLastError()).
// cell_zero (optional): the address kernel of block i clears the cell counters of row i.
// Blocks [i0, i0 + n) (n < 0: to the end).
// alt (optional): also the alternate address of each block (runner-up code of its lowest-margin
// subspace).
hipError_t launch_address(const Shape& s, const void* k, const float* codebook, const float* bias,
                          float* ksum, int32_t* addr, int32_t* cell_zero, hipStream_t st, int i0 = 0, int n = -1,
                          int32_t* alt = nullptr);
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
hipError_t launch_probe_rerank(const Shape& s, const void* q, const float* codebook, const float* bias,
                               const float* ksum, const int32_t* off, const int32_t* idx,
                               const int32_t* force, int32_t* sel, int32_t* ncand, int32_t* cellcnt,
                               int32_t* bins, hipStream_t st, const FusedPost* fuse = nullptr,
                               const ProbeExtra& ex = ProbeExtra{nullptr, nullptr, nullptr, nullptr});
// Redirect lists from the posting CSR and the alternates; overwrites overflow with the blocks no
// final view returns.
hipError_t launch_post_redirect(const Shape& s, const int32_t* addr, const int32_t* alt, const int32_t* off,
                                const int32_t* idx, int32_t* roff, int32_t* ridx, int32_t* rtime,
                                int32_t* overflow, hipStream_t st);
// True when launch_probe_rerank accepts `fuse` for this shape (the compile-time specialised probe).
bool probe_fuses_post(const Shape& s);
size_t probe_lds_bytes(const Shape& s);
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
hipError_t launch_pair_bin(const Shape& s, const int32_t* sel, int32_t* cellcnt, int32_t* bins,
                           hipStream_t st);
size_t remote_lds_bytes(const Shape& s);
// ev (optional, 2 entries): recorded before attn_remote and attn_local.
hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v,
                         const int32_t* sel, void* out, const Buffers& b, hipStream_t st,
                         hipEvent_t* ev = nullptr);
// The selection's pairs binned into cells in ascending token order within each cell (the cell
// counters must be zero before the call).
hipError_t launch_pair_bin_ordered(const Shape& s, const int32_t* sel, int32_t* cellcnt, int32_t* bins,
                                   hipStream_t st);
// Backward of the attention under a fixed selection (cellcnt / bins must hold the selection's
// pairs; part_o receives the remote dQ shares, dvec the row dots).  ev (optional, 3 entries):
// recorded before the row-dot, key-block and query-block kernels.
hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel,
                                  const void* out, const float* lse, const void* d_out, void* dq, void* dk, void* dv,
                                  const Buffers& b, hipStream_t st, hipEvent_t* ev = nullptr);
hipError_t launch_project_heads(const Shape& s, const void* x, const void* w, void* out, bool rope,
                                hipStream_t st);
// wt (optional): workspace for the transposed weights (4 * W * H * D elements); without it the
// simple tiled product is used.
hipError_t launch_project_out(const Shape& s, const void* o, const void* wo, void* delta, void* wt,
                              hipStream_t st);
// Q, K, V projections with RoPE, block summaries and addresses (and alternates when alt is given)
// fused into one launch; cell_zero (optional) as for launch_address.  Only when qkv_fuses_address.
bool qkv_fuses_address(const Shape& s);
hipError_t launch_qkv_fused(const Shape& s, const void* x, const void* wq, const void* wk, const void* wv, void* q,
                            void* k, void* v, const float* cb, const float* bias, float* ksum, int32_t* addr,
                            int32_t* alt, int32_t* cell_zero, void* wt, hipStream_t st);

}  // namespace mdr
