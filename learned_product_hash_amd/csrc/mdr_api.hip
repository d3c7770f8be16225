// C ABI of the routed-attention library: host-side validation, workspace planning and the
// launch sequences.  No entry point allocates memory or keeps state between calls.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "mdr_internal.h"

using namespace mdr;

namespace {

mdr_status shape_from_config(const mdr_config* cfg, bool mixer, Shape* out) {
  if (!cfg) return MDR_ERR_INVALID_ARG;
  const mdr_config& c = *cfg;
  if (c.batch < 1 || c.seq < 1 || c.heads < 1 || c.head_dim < 1 || c.block < 1 || c.subspaces < 1 ||
      c.codes < 1 || c.capacity < 1 || c.probes < 1 || c.max_cand < 0 || c.remote < 0 || c.local < 1)
    return MDR_ERR_INVALID_ARG;
  if (c.seq % c.block != 0) return MDR_ERR_INVALID_ARG;
  if (c.dtype != MDR_F32 && c.dtype != MDR_BF16) return MDR_ERR_INVALID_ARG;
  if (c.overflow_policy != MDR_OVERFLOW_DROP && c.overflow_policy != MDR_OVERFLOW_REDIRECT) return MDR_ERR_INVALID_ARG;
  if (!(c.softmax_scale >= 0.f) || isinf(c.softmax_scale)) return MDR_ERR_INVALID_ARG;
  if (mixer && (c.width < 1 || !(c.rope_base > 0.f) || isinf(c.rope_base))) return MDR_ERR_INVALID_ARG;
  if (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128) return MDR_ERR_UNSUPPORTED;
  if (c.block != 32 && c.block != 64 && c.block != 128) return MDR_ERR_UNSUPPORTED;
  if (c.subspaces > kMaxSubspaces || c.subspaces * c.codes > kMaxCodesTotal) return MDR_ERR_UNSUPPORTED;
  long long A = 1;
  for (int g = 0; g < c.subspaces; ++g) {
    A *= c.codes;
    if (A > kMaxAddresses) return MDR_ERR_UNSUPPORTED;
  }
  if (c.probes > A) return MDR_ERR_INVALID_ARG;
  if (c.probes > kMaxProbes || c.remote > kMaxRemote) return MDR_ERR_UNSUPPORTED;
  const int nb = c.seq / c.block;
  if (nb > kMaxBlocks) return MDR_ERR_UNSUPPORTED;
  if ((long long)c.batch * c.heads > 65535) return MDR_ERR_UNSUPPORTED;
  if (mixer && (long long)c.heads * c.head_dim > (1LL << 30)) return MDR_ERR_UNSUPPORTED;
  Shape s;
  memset(&s, 0, sizeof(s));
  s.B = c.batch;
  s.H = c.heads;
  s.S = c.seq;
  s.D = c.head_dim;
  s.W = c.width;
  s.blk = c.block;
  s.nb = nb;
  s.G = c.subspaces;
  s.C = c.codes;
  s.A = (int)A;
  s.cap = c.capacity;
  s.P = c.probes;
  // at most probes * capacity candidates can exist, so a larger cut changes nothing
  const long long pc = (long long)c.probes * c.capacity;
  long long M = c.max_cand > 0 && c.max_cand < pc ? (long long)c.max_cand : pc;
  s.M = (int)(M > (1LL << 20) ? (1LL << 20) : M);
  s.R = c.remote;
  s.L = c.local;
  s.dtype = c.dtype;
  s.scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / sqrtf((float)c.head_dim);
  s.rope_base = c.rope_base;
  s.policy = c.overflow_policy;
  const long long ne = nb > c.local ? nb - c.local : 0;
  s.ne = (int)ne;
  // pair binning: at most kMaxBinRanges token ranges per (b,h), each a whole number of 256-token probe
  // work-groups; remote work items of kItemPairs pairs, at most one partial item per block
  const long long tb = ((c.seq + kMaxBinRanges - 1) / kMaxBinRanges + 255) / 256 * 256;
  s.tbin = (int)tb;
  s.ng = (int)((c.seq + tb - 1) / tb);
  const long long pairs = (long long)c.seq * c.remote;
  const long long items = ne + (pairs + kItemPairs - 1) / kItemPairs;
  if (pairs >= (1LL << 31) || items * c.batch * c.heads >= (1LL << 31)) return MDR_ERR_UNSUPPORTED;
  s.max_items = (int)items;
  s.pin = (c.batch * c.heads) % kXcds == 0;
  s.csr_lds = ((long long)s.A + 1 + ne) * 4 <= 16384;
  s.fixed_probe = probe_fixed_shape(s);
  if (probe_lds_bytes(s) > 160 * 1024) return MDR_ERR_UNSUPPORTED;
  if (s.R > 0 && ne > 0 && (remote_lds_bytes(s) > 160 * 1024 || pair_scatter_lds_bytes(s) > 160 * 1024))
    return MDR_ERR_UNSUPPORTED;
  if (s.policy == MDR_OVERFLOW_REDIRECT && ((long long)s.A + 2 * ne) * 4 > 160 * 1024) return MDR_ERR_UNSUPPORTED;
  *out = s;
  return MDR_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions; with base == nullptr only the size is computed.  parts (optional) receives the
// bytes of each group of regions.
// Requested size of each region (for the index self-check).
struct Region {
  const char* p;
  size_t bytes;
};
constexpr int kMaxRegions = 64;

size_t layout(const Shape& s, char* base, Buffers* b, mdr_workspace_parts* parts = nullptr, Region* regs = nullptr,
              int* nregs = nullptr) {
  const size_t BH = (size_t)s.B * s.H, e = s.dtype == MDR_BF16 ? 2 : 4;
  size_t off = 0;
  mdr_workspace_parts pt;
  memset(&pt, 0, sizeof(pt));
  size_t* group = &pt.summaries;
  int nr = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    const size_t n = align_up(bytes ? bytes : 4);
    if (regs && nr < kMaxRegions) regs[nr++] = Region{p, bytes};
    off += n;
    *group += n;
    return p;
  };
  Buffers t;
  group = &pt.summaries;
  t.ksum = (float*)take(BH * s.nb * s.D * 4);
  t.addr = (int32_t*)take(BH * s.nb * 4);
  group = &pt.posting_lists;
  t.off = (int32_t*)take(BH * (s.A + 1) * 4);
  t.idx = (int32_t*)take(BH * s.nb * 4);
  t.overflow = (int32_t*)take(BH * 4);
  group = &pt.selection;
  t.sel = (int32_t*)take(BH * s.S * s.R * 4);
  t.ncand = (int32_t*)take(BH * s.S * 4);
  group = &pt.pair_lists;
  t.phist = (int32_t*)take(BH * s.ng * s.ne * 4);
  t.poff = (int32_t*)take(BH * (s.ne + 1) * 4);
  t.ioff = (int32_t*)take(BH * (s.ne + 1) * 4);
  t.items = (int32_t*)take(BH * (size_t)s.max_items * kItemInts * 4);
  group = &pt.partials;
  t.part_o = take(BH * s.S * s.R * s.D * e);
  t.part_lse = (float*)take(BH * s.S * s.R * 4);
  group = &pt.backward;
  t.dvec = (float*)take(BH * s.S * 4);
  if (s.policy == MDR_OVERFLOW_REDIRECT) {
    group = &pt.summaries;
    t.alt = (int32_t*)take(BH * s.nb * 4);
    group = &pt.posting_lists;
    t.roff = (int32_t*)take(BH * (s.A + 1) * 4);
    t.ridx = (int32_t*)take(BH * s.nb * 4);
    t.rtime = (int32_t*)take(BH * s.nb * 4);
  } else {
    t.alt = t.roff = t.ridx = t.rtime = nullptr;
  }
  t.ndrop = nullptr;
  t.amargin = nullptr;
  t.probes = nullptr;
  t.sel_score = t.pmargin = t.smargin = nullptr;
  if (s.W > 0) {
    group = &pt.mixer;
    const size_t qkv = BH * s.S * s.D * e;
    t.mq = take(qkv);
    t.mk = take(qkv);
    t.mv = take(qkv);
    t.mo = take(qkv);
    t.mwt = take(4 * (size_t)s.W * s.H * s.D * e);
  } else {
    t.mq = t.mk = t.mv = t.mo = t.mwt = nullptr;
  }
  t.lse = nullptr;
  if (b) *b = t;
  pt.total = off;
  if (parts) *parts = pt;
  if (nregs) *nregs = nr;
  return off;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

mdr_status hip_status(hipError_t e) { return e == hipSuccess ? MDR_OK : MDR_ERR_HIP; }

#define MDR_TRY(call)                          \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return MDR_ERR_HIP;  \
  } while (0)

mdr_status check_workspace(const Shape& s, void* ws, size_t ws_bytes, Buffers* b) {
  const size_t need = layout(s, nullptr, nullptr);
  if (!ws || ((uintptr_t)ws & 255) != 0) return MDR_ERR_INVALID_ARG;
  if (ws_bytes < need) return MDR_ERR_WORKSPACE;
  layout(s, (char*)ws, b);
  return MDR_OK;
}

// Decode: the core config plus the per-token limits of the decode kernel.
mdr_status decode_shape(const mdr_config* cfg, Shape* out) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if ((long long)(s.R + s.L) * s.blk > kDecMaxKeys || s.M > kDecMaxCand) return MDR_ERR_UNSUPPORTED;
  if (s.policy != MDR_OVERFLOW_DROP) return MDR_ERR_UNSUPPORTED;
  *out = s;
  return MDR_OK;
}

// Blocks a token at position pos may see remotely: i <= pos / block - L.
int decode_eligible(const Shape& s, int pos) {
  const int e = pos / s.blk - s.L + 1;
  return e > 0 ? e : 0;
}

size_t decode_layout(const Shape& s, char* base, DecState* d) {
  const size_t BH = (size_t)s.B * s.H;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes ? bytes : 4);
    return p;
  };
  DecState t;
  t.ring = (int32_t*)take(BH * s.A * (s.cap + 1) * 4);
  t.overflow = (int32_t*)take(BH * 4);
  t.summarized = (int32_t*)take(BH * 4);
  t.filed = (int32_t*)take(BH * 4);
  t.addr = (int32_t*)take(BH * s.nb * 4);
  t.ksum = (float*)take(BH * s.nb * s.D * 4);
  if (d) *d = t;
  return off;
}

mdr_status check_decode_state(const Shape& s, void* state, size_t bytes, DecState* d) {
  if (!state || ((uintptr_t)state & 255) != 0) return MDR_ERR_INVALID_ARG;
  if (bytes < decode_layout(s, nullptr, nullptr)) return MDR_ERR_WORKSPACE;
  decode_layout(s, (char*)state, d);
  return MDR_OK;
}

void apply_routing(const mdr_routing* r, Buffers* b) {
  if (!r) return;
  if (r->ksum) b->ksum = r->ksum;
  if (r->addr) b->addr = r->addr;
  if (r->post_off) b->off = r->post_off;
  if (r->post_idx) b->idx = r->post_idx;
  if (r->overflow) b->overflow = r->overflow;
  if (r->sel) b->sel = r->sel;
  if (r->n_cand) b->ncand = r->n_cand;
  b->ndrop = r->n_drop;
  b->amargin = r->addr_margin;
  b->probes = r->probes;
  b->sel_score = r->sel_score;
  b->pmargin = r->probe_margin;
  b->smargin = r->sel_margin;
  if (b->alt) {  // redirect policy
    if (r->alt) b->alt = r->alt;
    if (r->redir_off) b->roff = r->redir_off;
    if (r->redir_idx) b->ridx = r->redir_idx;
    if (r->redir_time) b->rtime = r->redir_time;
  }
}

bool routing_aligned(const mdr_routing* r) {
  return !r || aligned16(r->ksum);
}

// The stages of the core on post-RoPE q, k, v already in device memory.
// ev (optional, MDR_CORE_KERNELS + 1 entries): recorded before each kernel and after the last.
// have_address: the summaries, addresses (and alternates) and cleared pair counts are already in
// the buffers (the mixer's fused projection wrote them).
mdr_status run_core(const Shape& s, const void* q, const void* k, const void* v, const float* cb, const float* bias,
                    const int32_t* force, void* out, const Buffers& b, hipStream_t st, hipEvent_t* ev = nullptr,
                    bool have_address = false) {
  const bool binned = pairs_binned(s);  // else the remote kernel scans the selection itself
  MDR_TRY(mark_event(ev, 0, st));
  const bool redirect = s.policy == MDR_OVERFLOW_REDIRECT;
  if (!have_address)
    MDR_TRY(launch_address(s, k, cb, bias, b.ksum, b.addr, binned ? b.phist : nullptr, st, 0, -1,
                           redirect ? b.alt : nullptr, b.amargin));
  MDR_TRY(mark_event(ev, 1, st));
  // the posting lists are built inside the probe kernel where a specialised probe exists (the post
  // interval of a profiled call is then empty); the redirect lists need the whole CSR first
  const bool fused = probe_fuses_post(s) && !redirect;
  if (!fused) MDR_TRY(launch_post(s, b.addr, b.off, b.idx, b.overflow, st));
  if (redirect) MDR_TRY(launch_post_redirect(s, b.addr, b.alt, b.off, b.idx, b.roff, b.ridx, b.rtime, b.overflow, st));
  MDR_TRY(mark_event(ev, 2, st));
  const FusedPost fp{b.addr, b.off, b.idx, b.overflow};
  const ProbeExtra ex{redirect ? b.roff : nullptr, b.ridx, b.rtime, b.ndrop, b.probes, b.sel_score, b.pmargin,
                      b.smargin};
  MDR_TRY(launch_probe_rerank(s, q, cb, bias, b.ksum, b.off, b.idx, force, b.sel, b.ncand,
                              binned ? b.phist : nullptr, st, fused ? &fp : nullptr, ex));
  MDR_TRY(mark_event(ev, 3, st));
  if (binned) MDR_TRY(launch_pair_scatter(s, b.sel, b.phist, b.poff, b.ioff, b.items, st, false));
  MDR_TRY(launch_attend(s, q, k, v, b.sel, out, b, st, ev ? ev + 4 : nullptr));
  MDR_TRY(mark_event(ev, MDR_CORE_KERNELS, st));
  return MDR_OK;
}

}  // namespace

extern "C" {

int mdr_abi_version(void) { return MDR_ABI_VERSION; }

const char* mdr_status_string(int status) {
  switch (status) {
    case MDR_OK: return "MDR_OK";
    case MDR_ERR_INVALID_ARG: return "MDR_ERR_INVALID_ARG";
    case MDR_ERR_UNSUPPORTED: return "MDR_ERR_UNSUPPORTED";
    case MDR_ERR_WORKSPACE: return "MDR_ERR_WORKSPACE";
    case MDR_ERR_HIP: return "MDR_ERR_HIP";
    default: return "MDR_UNKNOWN_STATUS";
  }
}

mdr_status mdr_check_config(const mdr_config* cfg) {
  Shape s;
  return shape_from_config(cfg, cfg && cfg->width > 0, &s);
}

mdr_status mdr_workspace_size(const mdr_config* cfg, size_t* bytes) {
  if (!bytes) return MDR_ERR_INVALID_ARG;
  Shape s;
  const mdr_status st = shape_from_config(cfg, cfg && cfg->width > 0, &s);
  if (st != MDR_OK) return st;
  *bytes = layout(s, nullptr, nullptr);
  return MDR_OK;
}

mdr_status mdr_workspace_breakdown(const mdr_config* cfg, mdr_workspace_parts* parts) {
  if (!parts) return MDR_ERR_INVALID_ARG;
  Shape s;
  const mdr_status st = shape_from_config(cfg, cfg && cfg->width > 0, &s);
  if (st != MDR_OK) return st;
  layout(s, nullptr, nullptr, parts);
  return MDR_OK;
}

mdr_status mdr_routed_attention(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                const float* codebook, const float* code_bias, const int32_t* force, void* out,
                                const mdr_routing* routing, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if (!q || !k || !v || !codebook || !out) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(codebook) ||
      !routing_aligned(routing))
    return MDR_ERR_INVALID_ARG;
  Buffers b;
  st = check_workspace(s, workspace, workspace_bytes, &b);
  if (st != MDR_OK) return st;
  apply_routing(routing, &b);
  return run_core(s, q, k, v, codebook, code_bias, force, out, b, (hipStream_t)stream);
}

}  // extern "C"

// ---- the entry point that allocates nothing: its workspace is a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes `scratch` itself (on the host that name is
// only a stand-in, not a device address): each device's copy is looked up once with
// hipGetSymbolAddress, with that device current, and that address is used from then on.
namespace mdr {
constexpr size_t kNoAllocScratchBytes = (size_t)MDR_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
}  // namespace mdr

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's copy of the scratch array (looked up on the first call on the device).
mdr_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MDR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MDR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MDR_OK;
}

}  // namespace

extern "C" {

mdr_status mdr_routed_attention_noalloc(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                        const float* codebook, const float* code_bias, const int32_t* force,
                                        void* out, const mdr_routing* routing, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if (!q || !k || !v || !codebook || !out) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(codebook) ||
      !routing_aligned(routing))
    return MDR_ERR_INVALID_ARG;
  if (layout(s, nullptr, nullptr) > kNoAllocScratchBytes) return MDR_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MDR_OK) return st;
  Buffers b;
  st = check_workspace(s, ws, kNoAllocScratchBytes, &b);
  if (st != MDR_OK) return st;
  apply_routing(routing, &b);
  return run_core(s, q, k, v, codebook, code_bias, force, out, b, (hipStream_t)stream);
}

mdr_status mdr_routed_attention_profiled(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                         const float* codebook, const float* code_bias, const int32_t* force,
                                         void* out, const mdr_routing* routing, void* workspace,
                                         size_t workspace_bytes, void* const* events, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if (!q || !k || !v || !codebook || !out || !events) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(codebook) ||
      !routing_aligned(routing))
    return MDR_ERR_INVALID_ARG;
  Buffers b;
  st = check_workspace(s, workspace, workspace_bytes, &b);
  if (st != MDR_OK) return st;
  apply_routing(routing, &b);
  return run_core(s, q, k, v, codebook, code_bias, force, out, b, (hipStream_t)stream, (hipEvent_t*)events);
}

mdr_status mdr_mixer_forward(const mdr_config* cfg, const void* x, const void* wq, const void* wk, const void* wv,
                             const void* wo, const float* codebook, const float* code_bias, void* delta,
                             const mdr_routing* routing, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, true, &s);
  if (st != MDR_OK) return st;
  if (!x || !wq || !wk || !wv || !wo || !codebook || !delta) return MDR_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) || !aligned16(wo) || !aligned16(delta) ||
      !aligned16(codebook) || !routing_aligned(routing))
    return MDR_ERR_INVALID_ARG;
  Buffers b;
  st = check_workspace(s, workspace, workspace_bytes, &b);
  if (st != MDR_OK) return st;
  apply_routing(routing, &b);
  hipStream_t hs = (hipStream_t)stream;
  const bool fused = qkv_fuses_address(s);
  // the fused projection reads Wq, Wk, Wv transposed, the tiled output projection Wo
  const int tfirst = fused ? 0 : 3, tlast = project_out_tiled(s) ? 4 : 3;
  MDR_TRY(launch_transpose_weights(s, wq, wk, wv, wo, b.mwt, tfirst, tlast - tfirst, hs));
  if (fused) {
    MDR_TRY(launch_qkv_fused(s, x, b.mq, b.mk, b.mv, codebook, code_bias, b.ksum, b.addr,
                             s.policy == MDR_OVERFLOW_REDIRECT ? b.alt : nullptr, pairs_binned(s) ? b.phist : nullptr,
                             b.mwt, hs, b.amargin));
  } else {
    MDR_TRY(launch_project_heads(s, x, wq, b.mq, true, hs));
    MDR_TRY(launch_project_heads(s, x, wk, b.mk, true, hs));
    MDR_TRY(launch_project_heads(s, x, wv, b.mv, false, hs));
  }
  st = run_core(s, b.mq, b.mk, b.mv, codebook, code_bias, nullptr, b.mo, b, hs, nullptr, fused);
  if (st != MDR_OK) return st;
  MDR_TRY(launch_project_out(s, b.mo, wo, delta, b.mwt, hs));
  return MDR_OK;
}

mdr_status mdr_stage_address(const mdr_config* cfg, const void* k, const float* codebook, const float* code_bias,
                             float* ksum, int32_t* addr, int32_t* alt, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  if (!k || !codebook || !ksum || !addr) return MDR_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(ksum)) return MDR_ERR_INVALID_ARG;
  return hip_status(launch_address(s, k, codebook, code_bias, ksum, addr, nullptr, (hipStream_t)stream, 0, -1, alt));
}

mdr_status mdr_stage_post(const mdr_config* cfg, const int32_t* addr, const int32_t* alt, int32_t* post_off,
                          int32_t* post_idx, int32_t* redir_off, int32_t* redir_idx, int32_t* redir_time,
                          int32_t* overflow, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  if (!addr || !post_off || !post_idx || !overflow) return MDR_ERR_INVALID_ARG;
  const bool redirect = s.policy == MDR_OVERFLOW_REDIRECT;
  if (redirect && (!alt || !redir_off || !redir_idx || !redir_time)) return MDR_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  MDR_TRY(launch_post(s, addr, post_off, post_idx, overflow, hs));
  if (redirect)
    MDR_TRY(launch_post_redirect(s, addr, alt, post_off, post_idx, redir_off, redir_idx, redir_time, overflow, hs));
  return MDR_OK;
}

mdr_status mdr_stage_probe_rerank(const mdr_config* cfg, const void* q, const float* codebook,
                                  const float* code_bias, const float* ksum, const int32_t* post_off,
                                  const int32_t* post_idx, const int32_t* redir_off, const int32_t* redir_idx,
                                  const int32_t* redir_time, const int32_t* force, int32_t* sel, int32_t* n_cand,
                                  int32_t* n_drop, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  if (!q || !codebook || !ksum || !post_off || !post_idx || (!sel && s.R > 0)) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(ksum)) return MDR_ERR_INVALID_ARG;
  const bool redirect = s.policy == MDR_OVERFLOW_REDIRECT;
  if (redirect && (!redir_off || !redir_idx || !redir_time)) return MDR_ERR_INVALID_ARG;
  const ProbeExtra ex{redirect ? redir_off : nullptr, redir_idx, redir_time, n_drop};
  return hip_status(launch_probe_rerank(s, q, codebook, code_bias, ksum, post_off, post_idx, force, sel, n_cand,
                                        nullptr, (hipStream_t)stream, nullptr, ex));
}

mdr_status mdr_stage_attend_lse(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if (!q || !k || !v || !out || (!sel && s.R > 0)) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MDR_ERR_INVALID_ARG;
  Buffers b;
  st = check_workspace(s, workspace, workspace_bytes, &b);
  if (st != MDR_OK) return st;
  b.lse = lse;
  hipStream_t hs = (hipStream_t)stream;
  if (pairs_binned(s)) {
    MDR_TRY(launch_pair_count(s, sel, b.phist, hs));
    MDR_TRY(launch_pair_scatter(s, sel, b.phist, b.poff, b.ioff, b.items, hs, false));
  }
  MDR_TRY(launch_attend(s, q, k, v, sel, out, b, hs));
  return MDR_OK;
}

mdr_status mdr_stage_attend(const mdr_config* cfg, const void* q, const void* k, const void* v, const int32_t* sel,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return mdr_stage_attend_lse(cfg, q, k, v, sel, out, nullptr, workspace, workspace_bytes, stream);
}

static mdr_status backward_core(const mdr_config* cfg, const void* q, const void* k, const void* v, const int32_t* sel,
                                const void* out, const float* lse, const void* d_out, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, hipEvent_t* ev, void* stream) {
  Shape s;
  mdr_status st = shape_from_config(cfg, false, &s);
  if (st != MDR_OK) return st;
  s.W = 0;
  if (!q || !k || !v || !out || !lse || !d_out || !dq || !dk || !dv || (!sel && s.R > 0)) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(d_out) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return MDR_ERR_INVALID_ARG;
  Buffers b;
  st = check_workspace(s, workspace, workspace_bytes, &b);
  if (st != MDR_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  MDR_TRY(mark_event(ev, 0, hs));
  if (s.R > 0 && s.ne > 0) {
    MDR_TRY(launch_pair_count(s, sel, b.phist, hs));
    MDR_TRY(launch_pair_scatter(s, sel, b.phist, b.poff, b.ioff, b.items, hs, true));
  }
  MDR_TRY(launch_attend_backward(s, q, k, v, sel, out, lse, d_out, dq, dk, dv, b, hs, ev ? ev + 1 : nullptr));
  MDR_TRY(mark_event(ev, MDR_BACKWARD_KERNELS, hs));
  return MDR_OK;
}

mdr_status mdr_stage_attend_backward(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                     const int32_t* sel, const void* out, const float* lse, const void* d_out,
                                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return backward_core(cfg, q, k, v, sel, out, lse, d_out, dq, dk, dv, workspace, workspace_bytes, nullptr, stream);
}

mdr_status mdr_stage_attend_backward_profiled(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                              const int32_t* sel, const void* out, const float* lse,
                                              const void* d_out, void* dq, void* dk, void* dv, void* workspace,
                                              size_t workspace_bytes, void* const* events, void* stream) {
  if (!events) return MDR_ERR_INVALID_ARG;
  return backward_core(cfg, q, k, v, sel, out, lse, d_out, dq, dk, dv, workspace, workspace_bytes,
                       (hipEvent_t*)events, stream);
}

// ---- host self-check of the kernels' index arithmetic

namespace {

struct Checker {
  char* msg;
  size_t len;
  bool ok = true;
  void fail(const char* what, long long a, long long b) {
    if (ok && msg && len) snprintf(msg, len, "%s: %lld outside [0, %lld)", what, a, b);
    ok = false;
  }
  // index idx (in elements of esize bytes) must address inside the region of `bytes` bytes
  void in(const char* what, long long idx, long long n) {
    if (idx < 0 || idx >= n) fail(what, idx, n);
  }
};

size_t region_bytes(const Region* regs, int nr, const void* p) {
  for (int r = 0; r < nr; ++r)
    if (regs[r].p == p) return regs[r].bytes;
  return 0;
}

}  // namespace

mdr_status mdr_selfcheck_indices(const mdr_config* cfg, char* msg, size_t msg_len) {
  Shape s;
  mdr_status st = shape_from_config(cfg, cfg && cfg->width > 0, &s);
  if (st != MDR_OK) return st;
  if (msg && msg_len) msg[0] = 0;
  Region regs[kMaxRegions];
  int nr = 0;
  Buffers b;
  char* const base = (char*)((uintptr_t)1 << 40);  // never dereferenced: only offsets are compared
  const size_t total = layout(s, base, &b, nullptr, regs, &nr);
  Checker ck{msg, msg_len};
  const long long BH = (long long)s.B * s.H;
  const long long rows = BH * s.S;  // rows of Q, K, V, O
  // workspace regions: 256-byte aligned, in order, inside the workspace
  for (int r = 0; r < nr; ++r) {
    const long long o = (long long)(regs[r].p - base);
    if (o % 256) ck.fail("region alignment", o % 256, 1);
    ck.in("region end", o + (long long)regs[r].bytes - 1, (long long)total);
    if (r + 1 < nr && o + (long long)regs[r].bytes > (long long)(regs[r + 1].p - base))
      ck.fail("region overlap", o + (long long)regs[r].bytes, (long long)(regs[r + 1].p - base));
  }
  const bool remote = s.R > 0 && s.ne > 0;
  if (remote) {
    const long long n_items = (long long)(region_bytes(regs, nr, b.items) / 4);
    const long long n_phist = (long long)(region_bytes(regs, nr, b.phist) / 4);
    const long long n_plse = (long long)(region_bytes(regs, nr, b.part_lse) / 4);
    const long long n_po = (long long)(region_bytes(regs, nr, b.part_o) / (s.dtype == MDR_BF16 ? 2 : 4));
    const long long n_poff = (long long)(region_bytes(regs, nr, b.poff) / 4);
    // remote kernel: every work-group id maps to one (b,h, item) or to none; every item is covered once
    const long long grid = remote_grid(s);
    char* seen = (char*)calloc((size_t)(BH * s.max_items), 1);
    if (!seen) return MDR_ERR_UNSUPPORTED;
    for (long long id = 0; id < grid && ck.ok; ++id) {
      int bh, k;
      remote_work_of(s, id, &bh, &k);
      if (bh >= BH) continue;
      ck.in("remote item", k, s.max_items);
      ck.in("remote (b,h)", bh, BH);
      if (!ck.ok) break;
      if (seen[(size_t)bh * s.max_items + k]++) ck.fail("remote item mapped twice", k, s.max_items);
      ck.in("item record", (long long)(item_record(s, bh, k) + kItemInts - 1), n_items);
      // any block the item may name, any pair id it may hold
      ck.in("remote K/V row", (long long)(block_row(s, bh, s.ne - 1) + s.blk - 1), rows);
      ck.in("partial normaliser", (long long)partial_index(s, bh, s.S * s.R - 1), n_plse);
      ck.in("partial row", (long long)(partial_index(s, bh, s.S * s.R - 1) * s.D + s.D - 1), n_po);
    }
    for (long long x = 0; x < BH * s.max_items && ck.ok; ++x)
      if (!seen[x]) ck.fail("remote item never run", x, BH * s.max_items);
    free(seen);
    // pair counts: probe (every 64-token group: 256-, 128- or 64-token work-groups), count and scatter work-groups
    for (int bh = 0; bh < BH && ck.ok; ++bh) {
      for (int t0 = 0; t0 < s.S; t0 += 64) ck.in("pair counts row", (long long)(pair_counts_row(s, bh, t0) + s.ne - 1), n_phist);
      for (int g = 0; g < s.ng; ++g) {
        ck.in("scatter range", (long long)g * s.tbin, s.S);
        ck.in("scatter counts row", (long long)(pair_counts_row(s, bh, g * s.tbin) + s.ne - 1), n_phist);
      }
      ck.in("block offsets", (long long)bh * (s.ne + 1) + s.ne, n_poff);
    }
    // item slots under extreme count distributions of one (b,h): every pair in one block, one pair per
    // block with the rest in the last, and an even spread
    const long long pairs = (long long)s.S * s.R;
    for (int dist = 0; dist < 3 && ck.ok; ++dist) {
      long long istart = 0;
      for (int i = 0; i < s.ne && ck.ok; ++i) {
        long long cnt = dist == 0 ? (i == s.ne - 1 ? pairs : 0)
                        : dist == 1 ? (i == s.ne - 1 ? pairs - (s.ne - 1) : 1)
                                    : pairs / s.ne + (i < pairs % s.ne ? 1 : 0);
        if (cnt < 0) cnt = 0;
        const long long ni = (cnt + kItemPairs - 1) / kItemPairs;
        if (ni > 0) {
          ck.in("work items of a block", istart + ni - 1, s.max_items);
          ck.in("item pair slot", (long long)item_pair_slot(s, (int)BH - 1, (int)istart, (int)cnt - 1), n_items);
        }
        istart += ni;
      }
    }
  }
  // the scanning remote kernel (short sequences): a bijection onto (b,h, eligible block i); the
  // selection rows it reads (tokens (i + L) blk .. S - 1) and the pair ids it can form stay inside
  if (remote && remote_scans(s)) {
    const int n = (int)(BH * s.ne);
    char* seen = (char*)calloc((size_t)n, 1);
    if (!seen) return MDR_ERR_UNSUPPORTED;
    const long long n_plse = (long long)(region_bytes(regs, nr, b.part_lse) / 4);
    for (int id = 0; id < n && ck.ok; ++id) {
      int bh, i;
      remote_block_of(s, id, n, &bh, &i);
      ck.in("scanned block", (long long)bh * s.ne + i, n);
      if (!ck.ok) break;
      if (seen[(size_t)bh * s.ne + i]++) ck.fail("scanned block mapped twice", i, s.ne);
      ck.in("scan length", (long long)(s.S - (i + s.L) * s.blk), kScanMaxTokens + 1);
      ck.in("scanned K/V row", (long long)(block_row(s, bh, i) + s.blk - 1), rows);
      ck.in("scanned selection entry", ((long long)bh * s.S + s.S - 1) * s.R + s.R - 1, rows * s.R);
      ck.in("scanned partial", (long long)partial_index(s, bh, s.S * s.R - 1), n_plse);
    }
    free(seen);
  }
  // query-block kernels (local attention, backward dQ): a bijection onto (b,h, j), windows inside
  {
    const int n = (int)(BH * s.nb);
    char* seen = (char*)calloc((size_t)n, 1);
    if (!seen) return MDR_ERR_UNSUPPORTED;
    for (int id = 0; id < n && ck.ok; ++id) {
      int bh, j;
      query_block_of(s, id, n, &bh, &j);
      ck.in("query block", (long long)bh * s.nb + j, n);
      if (!ck.ok) break;
      if (seen[(size_t)bh * s.nb + j]++) ck.fail("query block mapped twice", j, s.nb);
      const int j0 = j - s.L + 1 > 0 ? j - s.L + 1 : 0;
      ck.in("local window first row", (long long)block_row(s, bh, j0), rows);
      ck.in("local window last row", (long long)(block_row(s, bh, j) + s.blk - 1), rows);
    }
    free(seen);
  }
  return ck.ok ? MDR_OK : MDR_ERR_INVALID_ARG;
}

// ---- streaming decode

size_t mdr_decode_state_size(const mdr_config* cfg) {
  Shape s;
  if (decode_shape(cfg, &s) != MDR_OK) return 0;
  return decode_layout(s, nullptr, nullptr);
}

mdr_status mdr_decode_state_view(const mdr_config* cfg, void* state, mdr_decode_view* view) {
  Shape s;
  mdr_status st = decode_shape(cfg, &s);
  if (st != MDR_OK) return st;
  if (!state || !view || ((uintptr_t)state & 255) != 0) return MDR_ERR_INVALID_ARG;
  DecState d;
  decode_layout(s, (char*)state, &d);
  view->ring = d.ring;
  view->overflow = d.overflow;
  view->summarized = d.summarized;
  view->filed = d.filed;
  view->addr = d.addr;
  view->ksum = d.ksum;
  return MDR_OK;
}

mdr_status mdr_decode_prime(const mdr_config* cfg, const void* k_cache, const float* codebook,
                            const float* code_bias, int32_t n_tokens, void* state, size_t state_bytes, void* stream) {
  Shape s;
  mdr_status st = decode_shape(cfg, &s);
  if (st != MDR_OK) return st;
  if (!k_cache || !codebook || !aligned16(k_cache) || !aligned16(codebook)) return MDR_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens >= s.S) return MDR_ERR_INVALID_ARG;
  DecState d;
  st = check_decode_state(s, state, state_bytes, &d);
  if (st != MDR_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const long long BH = (long long)s.B * s.H;
  const int complete = n_tokens / s.blk;
  const int target = decode_eligible(s, n_tokens);
  MDR_TRY(launch_ring_reset(d.ring, BH * s.A, s.cap, hs));
  MDR_TRY(launch_fill(d.overflow, BH, 0, hs));
  MDR_TRY(launch_fill(d.filed, BH, 0, hs));
  MDR_TRY(launch_fill(d.summarized, BH, complete, hs));
  if (complete > 0) MDR_TRY(launch_address(s, k_cache, codebook, code_bias, d.ksum, d.addr, nullptr, hs, 0, complete));
  MDR_TRY(launch_decode_file(s, k_cache, codebook, code_bias, d, target, hs));
  return MDR_OK;
}

mdr_status mdr_decode_step(const mdr_config* cfg, const void* q_new, const void* k_cache, const void* v_cache,
                           const float* codebook, const float* code_bias, const int32_t* force, int32_t pos,
                           int32_t n_new, void* out, int32_t* sel, void* state, size_t state_bytes, void* stream) {
  Shape s;
  mdr_status st = decode_shape(cfg, &s);
  if (st != MDR_OK) return st;
  if (!q_new || !k_cache || !v_cache || !codebook || !out) return MDR_ERR_INVALID_ARG;
  if (!aligned16(q_new) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(codebook))
    return MDR_ERR_INVALID_ARG;
  if (pos < 0 || n_new < 1 || (long long)pos + n_new > s.S) return MDR_ERR_INVALID_ARG;
  if (pos / s.blk != (pos + n_new - 1) / s.blk) return MDR_ERR_INVALID_ARG;  // one query block per call
  if (n_new > 65535) return MDR_ERR_UNSUPPORTED;
  DecState d;
  st = check_decode_state(s, state, state_bytes, &d);
  if (st != MDR_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  // steps continue where the previous call ended, so a block can become eligible only when pos opens
  // a new query block; the filing kernel (which files [filed, eligible) itself) runs only then
  if (pos == 0 || decode_eligible(s, pos) != decode_eligible(s, pos - 1))
    MDR_TRY(launch_decode_file(s, k_cache, codebook, code_bias, d, decode_eligible(s, pos), hs));
  MDR_TRY(launch_decode_attend(s, q_new, k_cache, v_cache, codebook, code_bias, d, force, pos, n_new, out, sel, hs));
  return MDR_OK;
}

}  // extern "C"
