// Backward pass of the selected-set attention with the routing held fixed: given Q, K, V, the
// selection, the output O, its per-token base-2 normaliser (lse) and the upstream gradient dO,
// computes dQ, dK, dV.  The router's own gradient is left open by the pages (remio.ai, "The 99.35%
// result does not prove language quality"); the attention after selection is exact softmax
// (aitechinspire.com, "Snapshot: key facts from the report"), whose gradient is
//   P = softmax(scale q k^T) over the selected keys,  D_t = dO_t . O_t,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
//   k_bwd_dot  D_t for every token.
//   k_bwd_kv   one work-group per key block i, one wave per 16 of its keys: the entries that read
//              block i -- the tokens of the local query blocks i .. i + L - 1 (causal on block i)
//              and the remote (token, slot) pairs of its cells -- are staged 32 (or 16) at a time; each
//              wave recomputes S = Q K^T and dP = dO V^T for its keys with the entries as rows,
//              then accumulates dV^T += dO^T P and dK^T += Q^T dS on MFMA (the score layout is
//              the PV operand layout, as in the forward); for remote entries the waves also
//              compute, with the keys as rows, the pair's share of dQ (scale dS K over block i)
//              and store it in the pair's partial slot.  dK, dV are written once, no atomics.
//   k_bwd_q    one work-group per query block: dQ of the local window (recomputed), plus the
//              remote shares in slot order.
#include "mdr_internal.h"
#include "mdr_tiles.h"

namespace mdr {
namespace {

using namespace tiles;

// D_t = sum_d dO[t][d] O[t][d] in fp32: LPT lanes per token, each 16 bytes of the row, added in a
// fixed order (lane partial, then xor 1, 2, ...).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_dot(const T* __restrict__ O, const T* __restrict__ dO,
                                                 float* __restrict__ Dv, long long n) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LPT = D / VEC;
  const long long t = ((long long)blockIdx.x * 256 + threadIdx.x) / LPT;
  const int l = threadIdx.x % LPT;
  float a = 0.f;
  if (t < n) {
    const T* o = O + t * D + l * VEC;
    const T* g = dO + t * D + l * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) a = fmaf((float)o[e], (float)g[e], a);
  }
#pragma unroll
  for (int x = 1; x < LPT; x <<= 1) a += __shfl_xor(a, x);
  if (t < n && l == 0) Dv[t] = a;
}

// Pairs binned into cells in a fixed order (ascending token within each cell), so that the
// gradient sums below always add the same terms in the same order.  One work-group per query block
// j, one thread per token: each eligible block the token selects gets the token's bit in a BLK-bit
// mask in LDS (atomic OR, so the result does not depend on timing), and the token's place in the
// cell (i, j) is the number of set bits below its own.  Cells left empty keep the count zero from
// the fill that precedes this kernel.
template <int BLK>
__global__ __launch_bounds__(BLK) void k_pair_bin_ordered(const int32_t* __restrict__ sel,
                                                          int32_t* __restrict__ cellcnt, int32_t* __restrict__ bins,
                                                          Shape s) {
  constexpr int NWORD = BLK / 32;
  extern __shared__ uint32_t masks[];  // [ne][NWORD]: the tokens of this query block selecting block i
  const int j = blockIdx.x, bh = blockIdx.y;
  if (j < s.L) return;  // no eligible block for the whole query block
  const int tid = threadIdx.x;
  const int t = j * BLK + tid;
  const int32_t* row = sel + ((size_t)bh * s.S + t) * s.R;
  uint32_t used = 0;  // bit r: entry r counts (eligible, first of a repeat)
  for (int r = 0; r < s.R; ++r)
    if (sel_entry_valid(row, r, j, s.L)) used |= 1u << r;
  for (int r = 0; r < s.R; ++r)
    if (used >> r & 1)
      for (int w = 0; w < NWORD; ++w) masks[row[r] * NWORD + w] = 0;
  __syncthreads();
  for (int r = 0; r < s.R; ++r)
    if (used >> r & 1) atomicOr(&masks[row[r] * NWORD + tid / 32], 1u << (tid % 32));
  __syncthreads();
  for (int r = 0; r < s.R; ++r) {
    if (!(used >> r & 1)) continue;
    const int i = row[r];
    const uint32_t* m = masks + i * NWORD;
    int pos = 0, tot = 0;
    for (int w = 0; w < NWORD; ++w) {
      const int c = __popc(m[w]);
      tot += c;
      if (w < tid / 32) pos += c;
    }
    pos += __popc(m[tid / 32] & ((1u << (tid % 32)) - 1u));
    const long long cell = (long long)bh * s.cells_per_bh + cell_row(i, s.ne) + (j - i - s.L);
    bins[cell * BLK + pos] = t * s.R + r;
    if (pos == 0) cellcnt[cell] = tot;
  }
}

template <int BLK>
hipError_t pair_bin_ordered(const Shape& s, const int32_t* sel, int32_t* cellcnt, int32_t* bins, hipStream_t st) {
  const size_t lds = (size_t)s.ne * (BLK / 32) * 4;
  hipError_t e;
  if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_pair_bin_ordered<BLK>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_pair_bin_ordered<BLK>, dim3(s.nb, s.B * s.H), dim3(BLK), lds, st, sel, cellcnt, bins, s);
  return hipGetLastError();
}

// Entries staged per chunk: 32, or 16 where 32 would not fit the 160 KiB of LDS.
template <typename T, int D, int BLK>
constexpr int bwd_ec() {
  return ((2 * BLK + 64) * Tile<T, D, BLK>::KST * (int)sizeof(T) + (4 * BLK + 1) * 4 + 1024 <= 160 * 1024) ? 32 : 16;
}

template <typename T, int D, int BLK>
constexpr size_t bwd_kv_lds() {
  constexpr int EC = bwd_ec<T, D, BLK>();
  return (size_t)(2 * Tile<T, D, BLK>::K_ELEMS + 2 * Tile<T, D, EC>::K_ELEMS) * sizeof(T) + (size_t)(4 * BLK + 1) * 4;
}

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 4) void k_bwd_kv(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, const T* __restrict__ dO,
                                                    const float* __restrict__ lse, const float* __restrict__ Dv,
                                                    const int32_t* __restrict__ cellcnt,
                                                    const int32_t* __restrict__ bins, T* __restrict__ dq_part,
                                                    T* __restrict__ dK, T* __restrict__ dV, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int EC = bwd_ec<T, D, BLK>();
  using TE = Tile<T, D, EC>;
  static_assert(!TL::bf || EC % 32 == 0, "bf16 products take the entries 32 at a time");
  constexpr int NTHR = BLK * 4;
  constexpr int NW = BLK / 16;  // one wave per 16 keys
  constexpr int NCH = D / TL::VEC;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vs = Ks + TL::K_ELEMS;
  T* Qs = Vs + TL::V_ELEMS;   // [EC][KST] the chunk's query rows
  T* dOs = Qs + TE::K_ELEMS;  // [EC][KST] the chunk's output-gradient rows
  int* pre = (int*)(dOs + TE::K_ELEMS);  // [NTHR + 1] exclusive prefix of the counts of a run of cells
  __shared__ int etok[EC], epair[EC];
  __shared__ float else2[EC], edd[EC];
  __shared__ int scan_tmp[NW];
  const int i = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s4 = lane >> 4, r16 = lane & 15;
  const size_t rowbase = (size_t)bh * s.S;
  for (int x = tid; x < BLK * NCH; x += NTHR) {
    const int row = x / NCH, ch = x % NCH;
    const size_t g = (rowbase + (size_t)i * BLK + row) * D + ch * TL::VEC;
    *(uint4*)(Ks + row * TL::KST + ch * TL::VEC) = *(const uint4*)(K + g);
    *(uint4*)(Vs + row * TL::VST + ch * TL::VEC) = *(const uint4*)(V + g);
  }
  __syncthreads();
  // this wave's 16 keys as the MFMA operand held in registers (K for S, V for dP)
  QFrag<T, D> kf, vf;
  load_q<T, D>(kf, Ks + (16 * wave + r16) * TL::KST, lane);
  load_q<T, D>(vf, Vs + (16 * wave + r16) * TL::VST, lane);
  const int key_tok = i * BLK + 16 * wave + r16;  // this lane's key (a column of S)
  const float c = s.scale * kLog2e;
  f32x4 dk[TL::ND], dv[TL::ND];
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // entries: segment -1 = the tokens of the local query blocks i .. i + L - 1; segment g >= 0 = the
  // pairs of the cells g NTHR .. g NTHR + NTHR - 1 of block i (query blocks i + L + cell)
  const int nl = (min(i + s.L, s.nb) - i) * BLK;
  const int ncell = (s.R > 0 && i < s.ne) ? s.ne - i : 0;
  const long long row0 = (long long)bh * s.cells_per_bh + (ncell > 0 ? cell_row(i, s.ne) : 0);
  const int nseg = (ncell + NTHR - 1) / NTHR;
  for (int seg = -1; seg < nseg; ++seg) {
    int n_ent = nl, nc = 0;
    const long long cbase = row0 + (long long)seg * NTHR;
    if (seg >= 0) {
      nc = min(NTHR, ncell - seg * NTHR);
      const int v = tid < nc ? min(cellcnt[cbase + tid], BLK) : 0;
      int tot;
      const int ex = block_exclusive_scan<NTHR>(v, scan_tmp, &tot);
      pre[tid] = ex;
      n_ent = tot;
      __syncthreads();
    }
    for (int e0 = 0; e0 < n_ent; e0 += EC) {
      // ---- stage the chunk: token, pair id, lse, D, then the query and output-gradient rows
      if (tid < EC) {
        const int e = e0 + tid;
        int t = -1, pid = -1;
        if (e < n_ent) {
          if (seg < 0) {
            t = i * BLK + e;
          } else {
            int lo = 0, hi = nc - 1;  // the last cell whose range starts at or before e
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (pre[mid] <= e)
                lo = mid;
              else
                hi = mid - 1;
            }
            pid = bins[(cbase + lo) * BLK + (e - pre[lo])];
            t = pid / s.R;
          }
        }
        etok[tid] = t;
        epair[tid] = pid;
        else2[tid] = t >= 0 ? lse[rowbase + t] : 0.f;
        edd[tid] = t >= 0 ? Dv[rowbase + t] : 0.f;
      }
      __syncthreads();
      for (int x = tid; x < EC * NCH; x += NTHR) {
        const int row = x / NCH, ch = x % NCH;
        const int t = etok[row];
        uint4 qv = make_uint4(0, 0, 0, 0), gv = make_uint4(0, 0, 0, 0);
        if (t >= 0) {
          qv = *(const uint4*)(Q + (rowbase + t) * D + ch * TL::VEC);
          gv = *(const uint4*)(dO + (rowbase + t) * D + ch * TL::VEC);
        }
        *(uint4*)(Qs + row * TL::KST + ch * TL::VEC) = qv;
        *(uint4*)(dOs + row * TL::KST + ch * TL::VEC) = gv;
      }
      __syncthreads();
      // ---- dV, dK of this wave's keys, entries as rows: lane (key r16) holds entries 16rt + 4s4 + k
      {
        f32x4 p[EC / 16], ds[EC / 16];
#pragma unroll
        for (int rt = 0; rt < EC / 16; ++rt) {
          const f32x4 sc = score_tile<T, D, EC>(kf, Qs, rt, lane);
          const f32x4 dp = score_tile<T, D, EC>(vf, dOs, rt, lane);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = 16 * rt + 4 * s4 + k;
            const float pv = etok[e] >= key_tok ? fast_exp2(fmaf(sc[k], c, -else2[e])) : 0.f;
            p[rt][k] = pv;
            ds[rt][k] = pv * (dp[k] - edd[e]);
          }
        }
        pv_block<T, D, EC>(dv, p, dOs, lane);
        pv_block<T, D, EC>(dk, ds, Qs, lane);
      }
      // ---- the remote entries' dQ shares, keys as rows: lane (entry 16g + r16) holds keys 16n + 4s4 + k
      if (seg >= 0) {
        for (int g = wave; g < EC / 16; g += NW) {
          const int e = 16 * g + r16;
          const int pid = epair[e];
          QFrag<T, D> qf, gf;
          load_q<T, D>(qf, Qs + e * TL::KST, lane);
          load_q<T, D>(gf, dOs + e * TL::KST, lane);
          const float le = else2[e], de = edd[e];
          f32x4 dst[TL::NT];
#pragma unroll
          for (int n = 0; n < TL::NT; ++n) {
            const f32x4 sc = score_tile<T, D, BLK>(qf, Ks, n, lane);
            const f32x4 dp = score_tile<T, D, BLK>(gf, Vs, n, lane);
#pragma unroll
            for (int k = 0; k < 4; ++k) dst[n][k] = fast_exp2(fmaf(sc[k], c, -le)) * (dp[k] - de);
          }
          f32x4 dq[TL::ND];
#pragma unroll
          for (int dt = 0; dt < TL::ND; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          pv_block<T, D, BLK>(dq, dst, Ks, lane);
          if (pid >= 0) {
            const size_t pr = rowbase * s.R + pid;  // the pair (token, slot)
#pragma unroll
            for (int dt = 0; dt < TL::ND; ++dt) store4<T>(dq_part + pr * D + 16 * dt + 4 * s4, dq[dt], s.scale);
          }
        }
      }
      __syncthreads();  // the chunk's staging is overwritten next
    }
  }
  // ---- dV^T, dK^T: lane (key r16) holds d = 16dt + 4s4 + k
  const size_t krow = rowbase + key_tok;
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) {
    store4<T>(dV + krow * D + 16 * dt + 4 * s4, dv[dt], 1.f);
    store4<T>(dK + krow * D + 16 * dt + 4 * s4, dk[dt], s.scale);
  }
}

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 4) void k_bwd_q(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, const T* __restrict__ dO,
                                                   const float* __restrict__ lse, const float* __restrict__ Dv,
                                                   const int32_t* __restrict__ sel, const T* __restrict__ dq_part,
                                                   T* __restrict__ dQ, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = BLK * 4;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vs = Ks + TL::K_ELEMS;
  const int j = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave * 16 + (lane & 15);
  const int t = j * BLK + qi;
  const int c4 = 4 * (lane >> 4);
  const size_t rowbase = (size_t)bh * s.S;
  QFrag<T, D> qf, gf;
  load_q<T, D>(qf, Q + (rowbase + t) * D, lane);
  load_q<T, D>(gf, dO + (rowbase + t) * D, lane);
  const float lt = lse[rowbase + t], dt_ = Dv[rowbase + t];
  const float c = s.scale * kLog2e;
  f32x4 dq[TL::ND];
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int j0 = max(0, j - s.L + 1);
  for (int jj = j0; jj <= j; ++jj) {
    if (jj != j0) __syncthreads();
    for (int x = tid; x < BLK * (D / TL::VEC); x += NTHR) {
      const int row = x / (D / TL::VEC), ch = x % (D / TL::VEC);
      *(uint4*)(Ks + row * TL::KST + ch * TL::VEC) = *(const uint4*)(K + (rowbase + (size_t)jj * BLK + row) * D + ch * TL::VEC);
      *(uint4*)(Vs + row * TL::VST + ch * TL::VEC) = *(const uint4*)(V + (rowbase + (size_t)jj * BLK + row) * D + ch * TL::VEC);
    }
    __syncthreads();
    f32x4 ds[TL::NT];
#pragma unroll
    for (int n = 0; n < TL::NT; ++n) {
      const f32x4 sc = score_tile<T, D, BLK>(qf, Ks, n, lane);
      const f32x4 dp = score_tile<T, D, BLK>(gf, Vs, n, lane);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool vis = jj < j || 16 * n + c4 + k <= qi;
        const float pv = vis ? fast_exp2(fmaf(sc[k], c, -lt)) : 0.f;
        ds[n][k] = pv * (dp[k] - dt_);
      }
    }
    pv_block<T, D, BLK>(dq, ds, Ks, lane);
  }
  // the remote shares in slot order (entries used by the forward: 0 <= sel <= j - L, first of a repeat)
  const int32_t* row = sel + (rowbase + t) * s.R;
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) dq[dt] *= s.scale;
  for (int r = 0; r < s.R; ++r) {
    if (!sel_entry_valid(row, r, j, s.L)) continue;
    const size_t pr = (rowbase + t) * s.R + r;
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) {
      const Raw4<T> raw = *(const Raw4<T>*)(dq_part + pr * D + 16 * dt + c4);
      dq[dt] += unpack4<T>(raw);
    }
  }
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) store4<T>(dQ + (rowbase + t) * D + 16 * dt + c4, dq[dt], 1.f);
}

template <typename T, int D, int BLK>
hipError_t bwd_impl(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, const void* o,
                    const float* lse, const void* d_o, void* dq, void* dk, void* dv, const Buffers& b, hipStream_t st,
                    hipEvent_t* ev) {
  const long long n = (long long)s.B * s.H * s.S;
  constexpr int LPT = D * (int)sizeof(T) / 16;
  const long long blocks = (n * LPT + 255) / 256;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_dot<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, (const T*)o, (const T*)d_o,
                     b.dvec, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr size_t kl = bwd_kv_lds<T, D, BLK>();
  if (kl > 65536 && (e = hipFuncSetAttribute((const void*)k_bwd_kv<T, D, BLK>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kl)) != hipSuccess)
    return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_kv<T, D, BLK>), dim3(s.nb, s.B * s.H), dim3(BLK * 4), kl, st, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)d_o, lse, b.dvec, b.cellcnt, b.bins, (T*)b.part_o,
                     (T*)dk, (T*)dv, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t ql = Tile<T, D, BLK>::LDS_BYTES;
  if (ql > 65536 && (e = hipFuncSetAttribute((const void*)k_bwd_q<T, D, BLK>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ql)) != hipSuccess)
    return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_q<T, D, BLK>), dim3(s.nb, s.B * s.H), dim3(BLK * 4), ql, st, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)d_o, lse, b.dvec, sel, (const T*)b.part_o, (T*)dq, s);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_blk(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, const void* o,
                   const float* lse, const void* d_o, void* dq, void* dk, void* dv, const Buffers& b, hipStream_t st,
                   hipEvent_t* ev) {
  switch (s.blk) {
    case 32: return bwd_impl<T, D, 32>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    case 64: return bwd_impl<T, D, 64>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    case 128: return bwd_impl<T, D, 128>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t bwd_d(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, const void* o,
                 const float* lse, const void* d_o, void* dq, void* dk, void* dv, const Buffers& b, hipStream_t st,
                 hipEvent_t* ev) {
  switch (s.D) {
    case 32: return bwd_blk<T, 32>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    case 64: return bwd_blk<T, 64>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    case 128: return bwd_blk<T, 128>(s, q, k, v, sel, o, lse, d_o, dq, dk, dv, b, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_pair_bin_ordered(const Shape& s, const int32_t* sel, int32_t* cellcnt, int32_t* bins,
                                   hipStream_t st) {
  switch (s.blk) {
    case 32: return pair_bin_ordered<32>(s, sel, cellcnt, bins, st);
    case 64: return pair_bin_ordered<64>(s, sel, cellcnt, bins, st);
    case 128: return pair_bin_ordered<128>(s, sel, cellcnt, bins, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel,
                                  const void* out, const float* lse, const void* d_out, void* dq, void* dk, void* dv,
                                  const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  if (s.dtype == MDR_BF16) return bwd_d<bf16>(s, q, k, v, sel, out, lse, d_out, dq, dk, dv, b, st, ev);
  return bwd_d<float>(s, q, k, v, sel, out, lse, d_out, dq, dk, dv, b, st, ev);
}

}  // namespace mdr
