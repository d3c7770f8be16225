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
//              and the remote (token, slot) pairs of its pair list (mdr_pairs.hip: ascending token
//              order, so every sum adds its terms in one fixed order) -- are taken 64 (or fewer) at a time
//              through a pipeline (pair lookup, row reads, products on three chunks at once); each
//              wave recomputes S = Q K^T and dP = dO V^T for its keys with the entries as rows,
//              then accumulates dV^T += dO^T P and dK^T += Q^T dS on MFMA (the score layout is
//              the PV operand layout, as in the forward); for remote entries the waves also
//              compute the pair's share of dQ (scale dS K over block i), from the chunk's dS left
//              in LDS where it fits (else recomputed with the keys as rows), and store it in the
//              pair's partial slot.  dK, dV are written once, no atomics.
//   k_bwd_q    one work-group per query block: dQ of the local window (recomputed), plus the
//              remote shares in slot order.
#include "mdr_internal.h"
#include "mdr_tiles.h"

#include <type_traits>

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

// Sizes of the key-block kernel: the entries of a block (local tokens, then its pair list) are taken
// EC at a time -- 64, or fewer where that would not fit the 160 KiB of LDS.
//
// The remote entries' dQ shares need dS with the keys as the contraction.  For bf16 with D <= 64, where
// one more BLK x EC tile fits without lowering the number of work-groups the LDS allows per CU
// (DS_LDS), each wave leaves its 16 keys' rows of dS^T in that tile (the bf16 values the dK product
// uses), and each share is one product over the block's keys read back from it with transposing
// reads; otherwise each share recomputes S and dP with the keys as rows.  (With D = 128 the kernel is
// at its register limit and the tile's stores made it spill: 2.75 -> 4.0 ms on 128K tokens.)
template <typename T, int D, int BLK>
struct KvCfg {
  using TL = Tile<T, D, BLK>;
  static constexpr int NTHR = BLK * 4;
  static constexpr int NW = BLK / 16;  // one wave per 16 keys
  static constexpr size_t lds(int ec) {
    return (size_t)(2 * BLK + 2 * ec) * TL::KST * sizeof(T) + (size_t)2 * ec * 16;
  }
  static constexpr size_t LIM = 160 * 1024 - 256;
  static constexpr int EC = lds(64) <= LIM ? 64 : lds(32) <= LIM ? 32 : 16;
  static constexpr int SUB = EC < 32 ? EC : 32;  // entries per dK / dV product
  // dS^T tile [BLK][DSS] (keys as rows): with rows EC + 16 elements apart, the eight rows that half a
  // wave's transposing reads touch fall in disjoint bank windows (as for the K/V tiles)
  static constexpr int DSS = EC + 16;
  static constexpr size_t DS_BYTES = (size_t)BLK * DSS * sizeof(T);
  static constexpr int per_cu(size_t b) { return (int)((size_t)160 * 1024 / b); }
  static constexpr bool DS_LDS =
      TL::bf && D <= 64 && lds(EC) + DS_BYTES <= LIM && per_cu(lds(EC) + DS_BYTES) >= per_cu(lds(EC));
  static constexpr size_t LDS = lds(EC) + (DS_LDS ? DS_BYTES : 0);
};

// The entries flow through a three-stage pipeline, one chunk of EC per stage and iteration:
//   A  resolve: entry -> token (local) or pair id (remote: the entry's slot of the block's pair list),
//      in registers of threads tid < EC;
//   B  gather: the chunk's query and output-gradient rows, normaliser and row dot, in registers;
//   C  products on the rows staged in LDS.
// While chunk k is in C, chunk k+1's reads (B) and chunk k+2's pair lookups (A) are in flight.
// bf16 with D <= 64 and 64-key blocks: held to three waves per SIMD (no spills at that budget), so
// that three work-groups per CU hide each other's read latency.
constexpr int kv_min_waves(int bytes, int D, int BLK) { return bytes == 2 && D <= 64 && BLK == 64 ? 3 : 1; }

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(kv_min_waves((int)sizeof(T), D, BLK)))) void k_bwd_kv(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, const T* __restrict__ dO,
                                                    const float* __restrict__ lse, const float* __restrict__ Dv,
                                                    const int32_t* __restrict__ poff,
                                                    const int32_t* __restrict__ ioff,
                                                    const int32_t* __restrict__ items, T* __restrict__ dq_part,
                                                    T* __restrict__ dK, T* __restrict__ dV, Shape s) {
  using C = KvCfg<T, D, BLK>;
  using TL = Tile<T, D, BLK>;
  constexpr int EC = C::EC, SUB = C::SUB, NTHR = C::NTHR, NW = C::NW;
  static_assert(!TL::bf || SUB == 32, "bf16 products take the entries 32 at a time");
  static_assert(EC <= NTHR, "one resolving thread per entry of a chunk");
  constexpr int NCH = D / TL::VEC;                      // 16-byte pieces per row
  constexpr int RPT = (EC * NCH + NTHR - 1) / NTHR;     // pieces per thread per chunk and array
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vs = Ks + TL::K_ELEMS;
  T* Qs = Vs + TL::V_ELEMS;              // [EC][KST] the chunk's query rows
  T* dOs = Qs + EC * TL::KST;            // [EC][KST] the chunk's output-gradient rows
  T* dsT = dOs + EC * TL::KST;           // [BLK][DSS] dS^T of the chunk, keys as rows (DS_LDS)
  int* mtok = (int*)(dsT + (C::DS_LDS ? BLK * C::DSS : 0));  // [2][EC] token of each entry (-1: none), by chunk parity
  int* mpair = mtok + 2 * EC;              // [2][EC] pair id t R + r (-1: local entry)
  float* mlse = (float*)(mpair + 2 * EC);  // [2][EC] log2 normaliser of the token
  float* mdd = mlse + 2 * EC;              // [2][EC] D = dO . O of the token
  // block-major order: early blocks, which later tokens select most, start first
  const int bhn = s.B * s.H;
  const int i = blockIdx.x / bhn, bh = blockIdx.x % bhn;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s4 = lane >> 4, r16 = lane & 15;
  const size_t rowbase = (size_t)bh * s.S;
  const int nl = (min(i + s.L, s.nb) - i) * BLK;
  int npair = 0, it0 = 0;  // this block's list: npair pairs in the work items from it0 on, in order
  if (s.R > 0 && i < s.ne) {
    const int32_t* po = poff + (size_t)bh * (s.ne + 1) + i;
    npair = po[1] - po[0];
    it0 = ioff[(size_t)bh * (s.ne + 1) + i];
  }
  const int32_t* recs = items + item_record(s, bh, it0);
  {
    KVRegs<T, D, BLK, NTHR> kv;
    kv.load(K + (rowbase + (size_t)i * BLK) * D, V + (rowbase + (size_t)i * BLK) * D, tid);
    kv.store(Ks, Vs, tid);
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
  {
    const int nloc = nl;
    const int ntot = nloc + npair;
    const int nch = (ntot + EC - 1) / EC;
    // ---- pipeline registers
    int aT = -1, aP = -1;  // stage A of thread tid < EC: local token, or pair id (aT = -2)
    u32x4 qr[RPT], gr[RPT];
    float bl = 0.f, bd = 0.f;
    auto stage_a = [&](int k) __attribute__((always_inline)) {
      aT = -1;
      aP = -1;
      const int e = k * EC + tid;
      if (tid < EC && e < ntot) {
        if (e < nloc) {
          aT = i * BLK + e;
        } else {
          const int er = e - nloc;
          aP = recs[(size_t)(er / kItemPairs) * kItemInts + kItemHead + er % kItemPairs];
          if ((unsigned)aP >= (unsigned)(s.S * s.R)) aP = -1;  // only ids of this (b,h) are ever gathered
          aT = aP < 0 ? -1 : -2;
        }
      }
    };
    auto commit_a = [&](int slot) __attribute__((always_inline)) {
      if (tid < EC) {
        mtok[slot * EC + tid] = aT == -2 ? aP / s.R : aT;
        mpair[slot * EC + tid] = aP;
      }
    };
    auto stage_b = [&](int slot) __attribute__((always_inline)) {
      const int* tk = mtok + slot * EC;
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        const int x = u * NTHR + tid;
        if ((EC * NCH) % NTHR == 0 || x < EC * NCH) {
          const int t = tk[x / NCH];
          const size_t g = (rowbase + (t >= 0 ? t : 0)) * D + (x % NCH) * TL::VEC;
          const u32x4 z = {0u, 0u, 0u, 0u};
          qr[u] = t >= 0 ? *(const u32x4*)(Q + g) : z;
          gr[u] = t >= 0 ? *(const u32x4*)(dO + g) : z;
        }
      }
      if (tid < EC) {
        const int t = tk[tid];
        bl = t >= 0 ? lse[rowbase + (t >= 0 ? t : 0)] : 0.f;
        bd = t >= 0 ? Dv[rowbase + (t >= 0 ? t : 0)] : 0.f;
      }
    };
    auto commit_b = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        const int x = u * NTHR + tid;
        if ((EC * NCH) % NTHR == 0 || x < EC * NCH) {
          const int row = x / NCH, ch = x % NCH;
          *(u32x4*)(Qs + row * TL::KST + ch * TL::VEC) = qr[u];
          *(u32x4*)(dOs + row * TL::KST + ch * TL::VEC) = gr[u];
        }
      }
      if (tid < EC) {
        mlse[slot * EC + tid] = bl;
        mdd[slot * EC + tid] = bd;
      }
    };
    if (nch > 0) {
      stage_a(0);
      commit_a(0);
      __syncthreads();
      stage_b(0);
      if (nch > 1) stage_a(1);
    }
    for (int k = 0; k < nch; ++k) {
      const int cur = k & 1, nxt = cur ^ 1;
      commit_b(cur);
      if (k + 1 < nch) commit_a(nxt);
      __syncthreads();
      if (k + 1 < nch) stage_b(nxt);
      if (k + 2 < nch) stage_a(k + 2);
      const int* tk = mtok + cur * EC;
      const int* pk = mpair + cur * EC;
      const float* lk = mlse + cur * EC;
      const float* dk_ = mdd + cur * EC;
      // ---- dV, dK of this wave's keys, entries as rows: lane (key r16) holds entries 16rt + 4s4 + k.
      // Only entries below BLK (the tokens of query block i) can precede a key of block i; every later
      // entry is a later token, and an unused entry (token -1) has zero query and gradient rows and a
      // zero normaliser and row dot, so whatever weight it gets it adds exactly zero.  The causal test
      // is therefore made only in chunks that hold entries below BLK.  In a chunk with remote entries
      // (DS_LDS) each lane also leaves its key's four dS values of each row tile in dsT, in bf16 as
      // the dK product takes them.
      const bool has_remote = npair > 0 && (k + 1) * EC > nloc;
      auto products = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int h = 0; h < EC / SUB; ++h) {
          const T* qh = Qs + h * SUB * TL::KST;
          const T* gh = dOs + h * SUB * TL::KST;
          f32x4 p[SUB / 16], ds[SUB / 16];
#pragma unroll
          for (int rt = 0; rt < SUB / 16; ++rt) {
            const f32x4 sc = score_tile<T, D, SUB>(kf, qh, rt, lane);
            const f32x4 dp = score_tile<T, D, SUB>(vf, gh, rt, lane);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const int e = h * SUB + 16 * rt + 4 * s4 + kk;
              const float ex = fast_exp2(fmaf(sc[kk], c, -lk[e]));
              const float pv = !MASKED || tk[e] >= key_tok ? ex : 0.f;
              p[rt][kk] = pv;
              ds[rt][kk] = pv * (dp[kk] - dk_[e]);
            }
            if constexpr (C::DS_LDS) {
              if (has_remote) {
                const bf16x4 w = {(bf16)ds[rt][0], (bf16)ds[rt][1], (bf16)ds[rt][2], (bf16)ds[rt][3]};
                *(bf16x4*)(dsT + (16 * wave + r16) * C::DSS + h * SUB + 16 * rt + 4 * s4) = w;
              }
            }
          }
          pv_block<T, D, SUB>(dv, p, gh, lane);
          pv_block<T, D, SUB>(dk, ds, qh, lane);
        }
      };
      if (k * EC < BLK)
        products(std::true_type{});
      else
        products(std::false_type{});
      // ---- the remote entries' dQ shares (scale dS K over block i): lane (entry 16g + r16) takes dS of
      // keys 16n + 4s4 + k, read back from dsT or recomputed with the keys as rows
      auto store_share = [&](int pid, const auto& dst) __attribute__((always_inline)) {
        f32x4 dq[TL::ND];
#pragma unroll
        for (int dt = 0; dt < TL::ND; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (C::DS_LDS)
          pv_block_bf16<D, BLK>(dq, dst, Ks, lane);
        else
          pv_block<T, D, BLK>(dq, dst, Ks, lane);
        if (pid >= 0) {
          const size_t pr = rowbase * s.R + pid;  // the pair (token, slot)
#pragma unroll
          for (int dt = 0; dt < TL::ND; ++dt) store4<T>(dq_part + pr * D + 16 * dt + 4 * s4, dq[dt], s.scale);
        }
      };
      if constexpr (C::DS_LDS) {
        if (has_remote) {
          __syncthreads();  // every wave's dS columns are in dsT
          for (int g = wave; g < EC / 16; g += NW) {
            const int el = 16 * g + r16;
            const int pid = pk[el];
            if (__builtin_amdgcn_readfirstlane(__ballot(pid >= 0) != 0ull ? 1 : 0) == 0) continue;  // all local
            bf16x4 dst[TL::NT];  // dS^T[16n + 4s4 + k][el], column el of four rows per transposing read
#pragma unroll
            for (int n = 0; n < TL::NT; ++n) dst[n] = tr_col4(dsT + (16 * n + 4 * s4) * C::DSS + 16 * g, C::DSS, r16);
            store_share(pid, dst);
          }
        }
      } else {
        for (int g = wave; g < EC / 16; g += NW) {
          const int el = 16 * g + r16;
          const int pid = pk[el];
          if (__builtin_amdgcn_readfirstlane(__ballot(pid >= 0) != 0ull ? 1 : 0) == 0) continue;  // all local
          QFrag<T, D> qf, gf;
          load_q<T, D>(qf, Qs + el * TL::KST, lane);
          load_q<T, D>(gf, dOs + el * TL::KST, lane);
          const float le = lk[el], de = dk_[el];
          f32x4 dst[TL::NT];  // dS^T[16n + 4s4 + k][el]
#pragma unroll
          for (int n = 0; n < TL::NT; ++n) {
            const f32x4 sc = score_tile<T, D, BLK>(qf, Ks, n, lane);
            const f32x4 dp = score_tile<T, D, BLK>(gf, Vs, n, lane);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dst[n][kk] = fast_exp2(fmaf(sc[kk], c, -le)) * (dp[kk] - de);
          }
          store_share(pid, dst);
        }
      }
      __syncthreads();  // chunk k's rows and metadata are overwritten next
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

// One work-group per query block, one wave per 16 of its tokens: dQ over the L local blocks
// (recomputing P and dS; the next block's K / V read is in flight while the current one is used; only
// the diagonal block needs the causal test), scaled, plus the remote blocks' shares in slot order.  The
// first RS = min(R, 1) shares are requested at entry with the query and gradient rows (their addresses
// do not depend on the selection; an unused one is ignored); a second would not fit four waves per SIMD
// without spilling, and measured no faster.
constexpr int q_min_waves(int bytes, int D) { return bytes == 2 && D <= 64 ? 4 : 1; }

template <typename T, int D, int BLK, int RS>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(q_min_waves((int)sizeof(T), D)))) void k_bwd_q(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, const T* __restrict__ dO,
                                                   const float* __restrict__ lse, const float* __restrict__ Dv,
                                                   const int32_t* __restrict__ sel, const T* __restrict__ dq_part,
                                                   T* __restrict__ dQ, Shape s) {
  using TL = Tile<T, D, BLK>;
  constexpr int NTHR = BLK * 4;
  extern __shared__ __align__(16) char lds_raw[];
  T* Ks = (T*)lds_raw;
  T* Vs = Ks + TL::K_ELEMS;
  int j, bh;
  query_block_of(s, blockIdx.x, gridDim.x, &bh, &j);  // query blocks of one head in order per XCD
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave * 16 + (lane & 15);
  const int t = j * BLK + qi;
  const int c4 = 4 * (lane >> 4);
  const size_t rowbase = (size_t)bh * s.S;
  const int j0 = max(0, j - s.L + 1);
  KVRegs<T, D, BLK, NTHR> kv;
  kv.load(K + (rowbase + (size_t)j0 * BLK) * D, V + (rowbase + (size_t)j0 * BLK) * D, tid);
  QFrag<T, D> qf, gf;
  load_q<T, D>(qf, Q + (rowbase + t) * D, lane);
  load_q<T, D>(gf, dO + (rowbase + t) * D, lane);
  const float lt = lse[rowbase + t], dt_ = Dv[rowbase + t];
  const int32_t* row = sel + (rowbase + t) * s.R;
  constexpr int RA = RS > 0 ? RS : 1;
  int sr[RA];
  Raw4<T> praw[RA][TL::ND];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const size_t pr = (rowbase + t) * s.R + r;
    sr[r] = row[r];
#pragma unroll
    for (int dt = 0; dt < TL::ND; ++dt) praw[r][dt] = *(const Raw4<T>*)(dq_part + pr * D + 16 * dt + c4);
  }
  const float c = s.scale * kLog2e;
  f32x4 dq[TL::ND];
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto block_step = [&](auto diag_tag, int jj) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    if (jj != j0) __syncthreads();  // the previous block is no longer read
    kv.store(Ks, Vs, tid);
    __syncthreads();
    if (jj < j) {
      const size_t nx = (rowbase + (size_t)(jj + 1) * BLK) * D;
      kv.load(K + nx, V + nx, tid);
    }
    f32x4 ds[TL::NT];
#pragma unroll
    for (int n = 0; n < TL::NT; ++n) {
      const f32x4 sc = score_tile<T, D, BLK>(qf, Ks, n, lane);
      const f32x4 dp = score_tile<T, D, BLK>(gf, Vs, n, lane);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float ex = fast_exp2(fmaf(sc[k], c, -lt));
        const float pv = !DIAG || 16 * n + c4 + k <= qi ? ex : 0.f;
        ds[n][k] = pv * (dp[k] - dt_);
      }
    }
    pv_block<T, D, BLK>(dq, ds, Ks, lane);
  };
  if (s.L == 2 && j >= 1) {
    block_step(std::false_type{}, j - 1);
    block_step(std::true_type{}, j);
  } else {
    for (int jj = j0; jj < j; ++jj) block_step(std::false_type{}, jj);
    block_step(std::true_type{}, j);
  }
  // the remote shares in slot order (entries used by the forward: 0 <= sel <= j - L, first of a repeat)
#pragma unroll
  for (int dt = 0; dt < TL::ND; ++dt) dq[dt] *= s.scale;
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    bool ok = sr[r] >= 0 && sr[r] <= j - s.L;
#pragma unroll
    for (int p = 0; p < r; ++p) ok = ok && sr[p] != sr[r];
    if (ok)
#pragma unroll
      for (int dt = 0; dt < TL::ND; ++dt) dq[dt] += unpack4<T>(praw[r][dt]);
  }
  for (int r = RS; r < s.R; ++r) {
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

template <typename T, int D, int BLK, int RS>
hipError_t launch_bwd_q(const Shape& s, const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                        const int32_t* sel, void* dq, const Buffers& b, long long nwg, hipStream_t st) {
  const size_t ql = Tile<T, D, BLK>::LDS_BYTES;
  hipError_t e;
  if (ql > 65536 && (e = hipFuncSetAttribute((const void*)k_bwd_q<T, D, BLK, RS>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ql)) != hipSuccess)
    return e;
  hipLaunchKernelGGL((k_bwd_q<T, D, BLK, RS>), dim3((unsigned)nwg), dim3(BLK * 4), ql, st, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)d_o, lse, b.dvec, sel, (const T*)b.part_o, (T*)dq, s);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t bwd_impl(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel, const void* o,
                    const float* lse, const void* d_o, void* dq, void* dk, void* dv, const Buffers& b, hipStream_t st,
                    hipEvent_t* ev) {
  const long long n = (long long)s.B * s.H * s.S;
  constexpr int LPT = D * (int)sizeof(T) / 16;
  const long long blocks = (n * LPT + 255) / 256;
  hipError_t e;
  if ((e = mark_event(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_dot<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, (const T*)o, (const T*)d_o,
                     b.dvec, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr size_t kl = KvCfg<T, D, BLK>::LDS;
  if (kl > 65536 && (e = hipFuncSetAttribute((const void*)k_bwd_kv<T, D, BLK>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kl)) != hipSuccess)
    return e;
  if ((e = mark_event(ev, 1, st)) != hipSuccess) return e;
  const unsigned nwg = (unsigned)((long long)s.nb * s.B * s.H);
  hipLaunchKernelGGL((k_bwd_kv<T, D, BLK>), dim3(nwg), dim3(BLK * 4), kl, st, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)d_o, lse, b.dvec, b.poff, b.ioff, b.items, (T*)b.part_o,
                     (T*)dk, (T*)dv, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark_event(ev, 2, st)) != hipSuccess) return e;
  return s.R >= 1 ? launch_bwd_q<T, D, BLK, 1>(s, q, k, v, d_o, lse, sel, dq, b, nwg, st)
                    : launch_bwd_q<T, D, BLK, 0>(s, q, k, v, d_o, lse, sel, dq, b, nwg, st);
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

hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v, const int32_t* sel,
                                  const void* out, const float* lse, const void* d_out, void* dq, void* dk, void* dv,
                                  const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  if (s.dtype == MDR_BF16) return bwd_d<bf16>(s, q, k, v, sel, out, lse, d_out, dq, dk, dv, b, st, ev);
  return bwd_d<float>(s, q, k, v, sel, out, lse, d_out, dq, dk, dv, b, st, ev);
}

}  // namespace mdr
