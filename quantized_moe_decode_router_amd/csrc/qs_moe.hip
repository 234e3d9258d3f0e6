// qs_moe.hip -- the C ABI declared in include/qs_moe.h.
//
// Ownership: the handle owns one device allocation per layer (router, bias,
// repacked routed matrices, shared expert) and one scratch allocation sized
// for max_tokens at create time, so decode neither allocates nor
// synchronises.  Upload stages raw blocks through a device buffer the
// handle keeps until destroy and re-lays them out with a repack kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "qs_moe.h"
#include "qs_kernels.h"
#include "qs_layout.h"
#include "qs_persist.h"
#include "qs_big.h"

using namespace qs;

namespace {

struct LayerDev {
  uint8_t* base = nullptr;   // single allocation
  float* router = nullptr;
  float* bias = nullptr;
  uint8_t* gate = nullptr;
  uint8_t* up = nullptr;
  uint8_t* down = nullptr;
  bool q4k = false;          // routed experts in the Q4_K-style format (a tail layer)
  uint8_t* sg = nullptr;     // shared expert rows (srow_bytes each)
  uint8_t* su = nullptr;
  uint8_t* sd = nullptr;
  bool uploaded = false;
  // a paged layer: its routed experts as records [gate | up | down] in
  // pinned host memory, E * rec_bytes, and the address the GPU reads them at
  uint8_t* host = nullptr;
  uint64_t host_dev = 0;
  size_t rec_bytes = 0;
};

// One decode call over paged layers whose ids have not been applied to the
// expert cache yet: its ids travel to pinned host memory behind the call.
struct PendingCall {
  hipEvent_t ev = nullptr;
  int32_t* ids = nullptr;    // pinned [nL][T][k] of the call's paged layers
  int layer0 = 0, nL = 0, T = 0;
};

struct Scratch {
  uint8_t* base = nullptr;
  size_t bytes = 0;
  double* logits;
  int32_t* ids;
  float* wts;
  int32_t* cnt;
  int32_t* off;
  int32_t* pairs;
  int32_t* n_active;
  int32_t* active;
  int32_t* tok_order;
  uint32_t* xh;
  uint32_t* xl;
  float* xs;
  int32_t* xa;
  uint32_t* ah;
  uint32_t* al;
  float* as;
  int32_t* aa;
  float* ash;
  float* xbuf[2];
  double* rinv;
  uint64_t* ll_lg;   // small-batch persistent flow: flagged logits, SwiGLU outputs, residual stream
  uint64_t* ll_a;
  uint64_t* llx[2];
  uint64_t* ll_dot;  // steering partials [T][kMaxGrid]
  size_t ll_bytes;   // bytes of the flagged buffers (contiguous, zeroed at create)
  float* mb;     // steering: MoE outputs before the projection [T][H] (= sb: the
                 // batched kernel's steered combine reads each sb entry once,
                 // in the thread that then writes mb there; the small-batch
                 // kernel does not use sb)
  float* part;   // steering: per-workgroup partial dot products [T][kMaxGrid]
  float* af;     // batched persistent flow: SwiGLU outputs of MFMA buckets [P][F]
  float* ob;     // routed down outputs by bucket position [P][H]
  float* sb;     // shared-expert down outputs [T][H]
};

// What one decode launch needs besides the weights: the scratch carve, the
// synchronisation words and the two flag counters that keep stale flagged
// words and barrier arrivals from matching later calls.
struct CallState {
  Scratch* s;
  uint32_t* sync;
  uint32_t* epoch;      // barriers completed on `sync`
  uint32_t* ll_epoch;   // flags used by the small-batch kernel so far
  void* zero_base;      // what to clear when the flags wrap (every flagged word
  size_t zero_bytes;    // any call on this state may have written)
};

}  // namespace

struct qs_moe {
  qs_moe_config cfg;
  int device = 0;
  size_t gu_stride = 0;      // bytes per repacked gate/up expert matrix
  size_t dn_stride = 0;      // bytes per repacked down expert matrix
  size_t gu_stride4 = 0;     // the same for the Q4_K-style tail layers
  size_t dn_stride4 = 0;
  size_t layer_bytes = 0;
  std::vector<LayerDev> layers;
  Scratch s;
  uint32_t* cbtab = nullptr; // device codebook quad tables
  uint8_t* staging = nullptr;
  size_t staging_bytes = 0;
  uint64_t total_bytes = 0;
  // persistent kernel
  LayerPtrs* d_layers = nullptr;  // device table of every layer's pointers
  uint32_t* sync = nullptr;       // barrier words
  uint32_t epoch = 0;             // barriers completed on `sync`
  int grid = 0;                   // workgroups of the batched kernel (one per CU)
  int grid_small = 0;             // workgroups of the small-batch kernel: at most
                                  // H / kDownRows, so every workgroup owns a down tile
  int wait_limit = 0;             // polls of a bounded wait before it gives up (0 = default)
  uint32_t* host_err = nullptr;   // pinned host word the error flag is read into
  size_t lds_limit = 0;           // LDS bytes per workgroup available on the device
  bool persist_small_ok = false; // T <= kSmallT instantiation usable
  bool persist_big_ok = false;   // batched instantiation usable
  bool steer_small_ok = false;   // the instantiations with the steered combine usable
  bool steer_big_ok = false;
  bool q4k_ok = false;           // the batched Q4_K-style instantiation (tail layers) usable
  bool q4k_steer_ok = false;
  bool q4k_small_ok[2] = {false, false};   // the small-batch Q4_K-style instantiations, [steer]
  bool q4k_fixed_ok = false;                // and their fixed-shape ones
  int mfma_min = 1;               // bucket size from which the MFMA path runs
  bool mfma_explicit = false;     // the config set mfma_min_tokens
  bool fixed_ok = false;          // the fixed-shape small-batch kernels are usable
  bool big_fixed_ok = false;      // the fixed-shape batched kernel is usable
  bool fixed_steer_ok = false;    // the same with the steered combine
  bool big_fixed_steer_ok = false;
  bool pg_small_ok[2] = {false, false};   // the instantiations for paged layers, [steer]
  bool pg_big_ok[2] = {false, false};
  bool pg_q4k_ok[2] = {false, false};
  bool pg_fixed_ok = false;       // the fixed-shape instantiations for paged layers
  bool pg_big_fixed_ok = false;
  uint32_t ll_epoch = 0;          // flags used by the small-batch kernel so far
  float* steer_dirs = nullptr;    // steering directions, device fp32 [n_layers][H] (null: none set)
  float steer_scale = 0.f;
  // ---- expert paging (layers [resident_layers, n_layers) are paged)
  int n_paged = 0;
  size_t slot_bytes = 0;          // one cache slot: the largest paged record
  uint8_t* slots = nullptr;       // HBM [cache_slots][slot_bytes]
  uint64_t* d_emap = nullptr;     // device [n_paged][E]: the address each expert is read at
  uint8_t* pstage = nullptr;      // HBM: one paged layer's records, re-laid before the copy to host
  int32_t* ids_buf = nullptr;     // device [n_layers][max_tokens][k]: ids of a call whose caller passes none
  std::vector<uint64_t> emap;     // host mirror of d_emap
  std::vector<int32_t> slot_of;   // [n_paged * E] slot holding the expert, or -1
  std::vector<int32_t> owner;     // [cache_slots] key (paged layer * E + expert) or -1
  std::vector<int32_t> lru_prev, lru_next;   // the occupied slots, least recent first
  int lru_head = -1, lru_tail = -1;
  std::set<int32_t> free_slots;
  std::vector<int32_t> copy_key;  // [cache_slots] key to copy into the slot at the next flush, or -1
  std::vector<int32_t> copy_list; // the slots whose copy_key is set
  std::vector<int32_t> dirty;     // keys whose map entry changed since the last flush
  std::vector<uint8_t> seen;      // [E] marks of one layer's uses
  uint64_t c_hits = 0, c_misses = 0, c_admits = 0, c_evicts = 0, c_preloaded = 0;
  uint64_t host_bytes = 0;
  std::vector<PendingCall> ring;  // pending calls, oldest at ring_head
  int ring_head = 0, ring_count = 0;
  int32_t* ring_ids = nullptr;    // pinned, the ring's id buffers
};

namespace {

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (dev >= 0 && dev != prev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

#define QS_HIP(call)                                                      \
  do {                                                                    \
    hipError_t err_ = (call);                                             \
    if (err_ != hipSuccess) {                                             \
      fprintf(stderr, "qs_moe: %s failed: %s\n", #call, hipGetErrorString(err_)); \
      return QS_E_HIP;                                                    \
    }                                                                     \
  } while (0)

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "qs_moe: %s failed: %s\n", what, hipGetErrorString(e));
  return false;
}

size_t gate_up_block_bytes(const qs_moe_config& c) {
  return c.gate_up_format == QS_FMT_CB2 ? kCB2Bytes : kQ2KBytes;
}

int validate_config(const qs_moe_config* c) {
  if (!c) return QS_E_INVAL;
  if (c->abi_version != QS_MOE_ABI_VERSION) return QS_E_INVAL;
  if (c->hidden < 256 || c->hidden > 16384 || c->hidden % 256) return QS_E_INVAL;
  if (c->expert_ffn < 256 || c->expert_ffn > 16384 || c->expert_ffn % 256) return QS_E_INVAL;
  if (c->n_experts < 1 || c->n_experts > 1024) return QS_E_INVAL;
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return QS_E_INVAL;
  if (c->shared_ffn < 0 || c->shared_ffn > 16384 || c->shared_ffn % 64) return QS_E_INVAL;
  if (c->gate_up_format != QS_FMT_CB2 && c->gate_up_format != QS_FMT_Q2K) return QS_E_INVAL;
  if (c->down_format != QS_FMT_CB2 && c->down_format != QS_FMT_Q2K) return QS_E_INVAL;
  if (c->n_layers < 1 || c->n_layers > 4096) return QS_E_INVAL;
  if (c->max_tokens < 1 || c->max_tokens > kMaxTokens) return QS_E_INVAL;
  if ((long)c->max_tokens * c->top_k > kMaxPairs) return QS_E_INVAL;
  if (c->mfma_min_tokens < 0) return QS_E_INVAL;
  if (c->device < -1) return QS_E_INVAL;
  if (c->shared_format != QS_FMT_BF16 && c->shared_format != QS_FMT_Q8) return QS_E_INVAL;
  if (c->tail_layers < 0 || c->tail_layers > c->n_layers) return QS_E_INVAL;
  if (c->expert_paging != 0 && c->expert_paging != 1) return QS_E_INVAL;
  if (!c->expert_paging && (c->resident_layers || c->cache_slots)) return QS_E_INVAL;
  if (c->resident_layers < 0 || c->resident_layers > c->n_layers) return QS_E_INVAL;
  if (c->cache_slots < 0 || (long)c->cache_slots > (long)(c->n_layers - c->resident_layers) * c->n_experts)
    return QS_E_INVAL;
  if (c->down_format != QS_FMT_Q2K) return QS_E_UNSUPPORTED;
  return QS_OK;
}

// Signed int8 quads of the codebook with the sign nibbles applied.
void build_cb_tables(const int8_t* cb, std::vector<uint32_t>& tab) {
  tab.assign(kCbTabWords, 0);
  for (int idx = 0; idx < 256; ++idx)
    for (int s = 0; s < 16; ++s) {
      uint32_t lo = 0, hi = 0;
      for (int b = 0; b < 4; ++b) {
        const int vlo = ((s >> b) & 1) ? -cb[idx * 8 + b] : cb[idx * 8 + b];
        const int vhi = ((s >> b) & 1) ? -cb[idx * 8 + 4 + b] : cb[idx * 8 + 4 + b];
        lo |= (uint32_t)(uint8_t)(int8_t)vlo << (8 * b);
        hi |= (uint32_t)(uint8_t)(int8_t)vhi << (8 * b);
      }
      tab[idx * 16 + s] = lo;
      tab[4096 + s * 256 + idx] = hi;
    }
}

template <typename T>
T* carve(uint8_t*& p, size_t count) {
  T* r = (T*)p;
  p += align_up(count * sizeof(T), 256);
  return r;
}

// Words of the small-batch kernel's flagged buffers (batches of up to kSmallT).
struct LLWords {
  size_t lg, a, x, dot;
};
LLWords ll_words(const qs_moe_config& c) {
  const size_t T = std::min(c.max_tokens, kSmallT), P = T * c.top_k, F = c.expert_ffn;
  return LLWords{T * c.n_experts * 2, 2 * P * (F / 4) + 2 * P * (F / 16) + T * (size_t)c.shared_ffn,
                 T * (size_t)c.hidden, T * (size_t)kMaxGrid};
}

size_t scratch_bytes(const qs_moe_config& c) {
  const size_t T = c.max_tokens, E = c.n_experts, k = c.top_k, H = c.hidden, F = c.expert_ffn;
  const size_t P = T * k;
  size_t b = 0;
  auto add = [&](size_t n) { b += align_up(n, 256); };
  const LLWords lw = ll_words(c);
  add(lw.lg * 8); add(lw.a * 8); add(lw.x * 8); add(lw.x * 8); add(lw.dot * 8);
  add(T * E * 8);                 // logits
  add(P * 4); add(P * 4);         // ids, wts
  add(E * 4); add((E + 1) * 4);   // cnt, off
  add(P * 4); add(4); add(E * 4); add(P * 4);  // pairs, n_active, active, tok_order
  add(T * H); add(T * H);         // xh, xl (H/4 dwords)
  add(T * (H / 16) * 4); add(T * (H / 16) * 4);
  add(P * F); add(P * F);         // ah, al
  add(P * (F / 16) * 4); add(P * (F / 16) * 4);
  add(T * (size_t)(c.shared_ffn ? c.shared_ffn : 1) * 4);
  add(T * H * 4); add(T * H * 4); // residual ping-pong
  add(T * 8);                     // rinv
  add(P * F * 4);                 // af
  add(P * H * 4);                 // ob
  add(T * H * 4);                 // sb (and mb)
  add(T * (size_t)kMaxGrid * 4);  // part
  return b;
}

void carve_scratch(const qs_moe_config& c, Scratch& s) {
  const size_t T = c.max_tokens, E = c.n_experts, k = c.top_k, H = c.hidden, F = c.expert_ffn;
  const size_t P = T * k;
  uint8_t* p = s.base;
  const LLWords lw = ll_words(c);
  s.ll_lg = carve<uint64_t>(p, lw.lg);
  s.ll_a = carve<uint64_t>(p, lw.a);
  s.llx[0] = carve<uint64_t>(p, lw.x);
  s.llx[1] = carve<uint64_t>(p, lw.x);
  s.ll_dot = carve<uint64_t>(p, lw.dot);
  s.ll_bytes = (size_t)(p - s.base);
  s.logits = carve<double>(p, T * E);
  s.ids = carve<int32_t>(p, P);
  s.wts = carve<float>(p, P);
  s.cnt = carve<int32_t>(p, E);
  s.off = carve<int32_t>(p, E + 1);
  s.pairs = carve<int32_t>(p, P);
  s.n_active = carve<int32_t>(p, 1);
  s.active = carve<int32_t>(p, E);
  s.tok_order = carve<int32_t>(p, P);
  s.xh = carve<uint32_t>(p, T * H / 4);
  s.xl = carve<uint32_t>(p, T * H / 4);
  s.xs = carve<float>(p, T * H / 16);
  s.xa = carve<int32_t>(p, T * H / 16);
  s.ah = carve<uint32_t>(p, P * F / 4);
  s.al = carve<uint32_t>(p, P * F / 4);
  s.as = carve<float>(p, P * F / 16);
  s.aa = carve<int32_t>(p, P * F / 16);
  s.ash = carve<float>(p, T * (size_t)(c.shared_ffn ? c.shared_ffn : 1));
  s.xbuf[0] = carve<float>(p, T * H);
  s.xbuf[1] = carve<float>(p, T * H);
  s.rinv = carve<double>(p, T);
  s.af = carve<float>(p, P * F);
  s.ob = carve<float>(p, P * H);
  s.sb = carve<float>(p, T * H);
  s.mb = s.sb;
  s.part = carve<float>(p, T * (size_t)kMaxGrid);
}

void free_all(qs_moe* h) {
  for (auto& L : h->layers) {
    if (L.base) (void)hipFree(L.base);
    if (L.host) (void)hipHostFree(L.host);
  }
  if (h->slots) (void)hipFree(h->slots);
  if (h->d_emap) (void)hipFree(h->d_emap);
  if (h->pstage) (void)hipFree(h->pstage);
  if (h->ids_buf) (void)hipFree(h->ids_buf);
  for (auto& pc : h->ring)
    if (pc.ev) (void)hipEventDestroy(pc.ev);
  if (h->ring_ids) (void)hipHostFree(h->ring_ids);
  if (h->s.base) (void)hipFree(h->s.base);
  if (h->steer_dirs) (void)hipFree(h->steer_dirs);
  if (h->cbtab) (void)hipFree(h->cbtab);
  if (h->staging) (void)hipFree(h->staging);
  if (h->d_layers) (void)hipFree(h->d_layers);
  if (h->sync) (void)hipFree(h->sync);
  if (h->host_err) (void)hipHostFree(h->host_err);
}

__global__ void k_sync_reset(uint32_t* s) {
  for (int i = threadIdx.x; i < kSyncWords; i += blockDim.x) s[i] = 0;
}

// Zero n 16-byte words (a kernel rather than hipMemsetAsync, so a caller may
// capture the decode call in a graph).
__global__ void k_zero16(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

void launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  if (n) hipLaunchKernelGGL(k_zero16, dim3(blocks), dim3(256), 0, st, (uint4*)p, n);
}

// ------------------------------------------------------ expert paging ---
// The expert cache's policy runs on the host: least-recently-used over all
// slots, a use per distinct (layer, expert) of a call's paged layers in
// (layer, token, rank) order.  The device sees only its result, the map of
// each paged expert to the address it is read at (a slot, or its host
// record).  A flush enqueues the admitted experts' copies (DMA engines) and
// then the changed map entries on the stream, ahead of the next decode
// launch; a launch never runs between the two.
constexpr int kRing = 8;          // decode calls whose ids may be in flight to the host
constexpr int kEmapBatch = 48;    // map entries per update launch (kernel arguments)

struct EmapUpd {
  int32_t n;
  int32_t idx[kEmapBatch];
  uint64_t val[kEmapBatch];
};

__global__ void k_emap_set(uint64_t* emap, EmapUpd u) {
  const int i = threadIdx.x;
  if (i < u.n) emap[u.idx[i]] = u.val[i];
}

uint64_t host_addr(const qs_moe* h, int key) {
  const int E = h->cfg.n_experts;
  const LayerDev& L = h->layers[h->cfg.resident_layers + key / E];
  return L.host_dev + (uint64_t)(key % E) * L.rec_bytes;
}

uint64_t slot_addr(const qs_moe* h, int v) { return (uint64_t)(uintptr_t)(h->slots + (size_t)v * h->slot_bytes); }

void lru_unlink(qs_moe* h, int v) {
  const int p = h->lru_prev[v], n = h->lru_next[v];
  (p >= 0 ? h->lru_next[p] : h->lru_head) = n;
  (n >= 0 ? h->lru_prev[n] : h->lru_tail) = p;
  h->lru_prev[v] = h->lru_next[v] = -1;
}

void lru_push_back(qs_moe* h, int v) {   // most recent end
  h->lru_prev[v] = h->lru_tail;
  h->lru_next[v] = -1;
  (h->lru_tail >= 0 ? h->lru_next[h->lru_tail] : h->lru_head) = v;
  h->lru_tail = v;
}

void lru_push_front(qs_moe* h, int v) {  // least recent end
  h->lru_next[v] = h->lru_head;
  h->lru_prev[v] = -1;
  (h->lru_head >= 0 ? h->lru_prev[h->lru_head] : h->lru_tail) = v;
  h->lru_head = v;
}

// Slot v now holds `key`; its bytes are copied at the next flush.
void slot_take(qs_moe* h, int v, int key) {
  h->owner[v] = key;
  h->slot_of[key] = v;
  if (h->copy_key[v] < 0) h->copy_list.push_back(v);
  h->copy_key[v] = key;
  h->dirty.push_back(key);
}

// One use of expert `key` by a decode call.
void cache_use(qs_moe* h, int key) {
  const int s = h->slot_of[key];
  if (s >= 0) {
    ++h->c_hits;
    lru_unlink(h, s);
    lru_push_back(h, s);
    return;
  }
  ++h->c_misses;
  int v;
  if (!h->free_slots.empty()) {
    v = *h->free_slots.begin();
    h->free_slots.erase(h->free_slots.begin());
  } else if (h->lru_head >= 0) {
    v = h->lru_head;
    lru_unlink(h, v);
    const int old = h->owner[v];
    h->slot_of[old] = -1;
    h->dirty.push_back(old);
    ++h->c_evicts;
  } else {
    return;   // no slots at all
  }
  slot_take(h, v, key);
  lru_push_back(h, v);
  ++h->c_admits;
}

// The uses of one completed call.
void cache_apply(qs_moe* h, const PendingCall& pc) {
  const qs_moe_config& c = h->cfg;
  const int E = c.n_experts, k = c.top_k, R = c.resident_layers;
  const int lp0 = std::max(pc.layer0, R);
  for (int l = lp0; l < pc.layer0 + pc.nL; ++l) {
    const int32_t* id = pc.ids + (size_t)(l - lp0) * pc.T * k;
    for (int i = 0; i < pc.T * k; ++i) {
      const int e = id[i];
      if (e < 0 || e >= E || h->seen[e]) continue;
      h->seen[e] = 1;
      cache_use(h, (l - R) * E + e);
    }
    for (int i = 0; i < pc.T * k; ++i)
      if (id[i] >= 0 && id[i] < E) h->seen[id[i]] = 0;
  }
}

// Enqueue the pending slot copies, then the changed map entries.
int cache_flush(qs_moe* h, hipStream_t st) {
  const int E = h->cfg.n_experts;
  for (const int v : h->copy_list) {
    const int key = h->copy_key[v];
    if (key < 0) continue;              // freed again before this flush
    h->copy_key[v] = -1;
    if (h->owner[v] != key) continue;   // replaced again before this flush
    const LayerDev& L = h->layers[h->cfg.resident_layers + key / E];
    QS_HIP(hipMemcpyAsync(h->slots + (size_t)v * h->slot_bytes, L.host + (size_t)(key % E) * L.rec_bytes,
                          L.rec_bytes, hipMemcpyHostToDevice, st));
  }
  h->copy_list.clear();
  std::sort(h->dirty.begin(), h->dirty.end());
  h->dirty.erase(std::unique(h->dirty.begin(), h->dirty.end()), h->dirty.end());
  for (size_t i0 = 0; i0 < h->dirty.size(); i0 += kEmapBatch) {
    EmapUpd u{};
    u.n = (int)std::min<size_t>(kEmapBatch, h->dirty.size() - i0);
    for (int j = 0; j < u.n; ++j) {
      const int key = h->dirty[i0 + j];
      const int v = h->slot_of[key];
      const uint64_t a = v >= 0 ? slot_addr(h, v) : host_addr(h, key);
      h->emap[key] = a;
      u.idx[j] = key;
      u.val[j] = a;
    }
    hipLaunchKernelGGL(k_emap_set, dim3(1), dim3(64), 0, st, h->d_emap, u);
    QS_HIP(hipGetLastError());
  }
  h->dirty.clear();
  return QS_OK;
}

// Apply the pending calls that have completed (all of them, waiting, with
// `wait`), then flush.
int cache_poll(qs_moe* h, hipStream_t st, bool wait) {
  while (h->ring_count > 0) {
    PendingCall& pc = h->ring[h->ring_head];
    if (wait) {
      QS_HIP(hipEventSynchronize(pc.ev));
    } else {
      const hipError_t q = hipEventQuery(pc.ev);
      if (q == hipErrorNotReady) {
        (void)hipGetLastError();
        break;
      }
      QS_HIP(q);
    }
    cache_apply(h, pc);
    h->ring_head = (h->ring_head + 1) % kRing;
    --h->ring_count;
  }
  return cache_flush(h, st);
}

// After a decode call over layers [layer0, layer0 + nL): its paged layers'
// ids (device [nL][T][k] at ids) go to host memory behind it.
int cache_record(qs_moe* h, const int32_t* ids, int layer0, int nL, int T, hipStream_t st) {
  const int k = h->cfg.top_k, lp0 = std::max(layer0, h->cfg.resident_layers);
  if (lp0 >= layer0 + nL) return QS_OK;
  if (h->ring_count == kRing) {   // the oldest pending call must be applied first
    PendingCall& old = h->ring[h->ring_head];
    QS_HIP(hipEventSynchronize(old.ev));
    cache_apply(h, old);
    h->ring_head = (h->ring_head + 1) % kRing;
    --h->ring_count;
  }
  PendingCall& pc = h->ring[(h->ring_head + h->ring_count) % kRing];
  const size_t n = (size_t)(layer0 + nL - lp0) * T * k;
  QS_HIP(hipMemcpyAsync(pc.ids, ids + (size_t)(lp0 - layer0) * T * k, n * 4, hipMemcpyDeviceToHost, st));
  QS_HIP(hipEventRecord(pc.ev, st));
  pc.layer0 = layer0;
  pc.nL = nL;
  pc.T = T;
  ++h->ring_count;
  return QS_OK;
}

// Paging state at create: every paged expert is read from host memory.
int setup_paging(qs_moe* h) {
  const qs_moe_config& c = h->cfg;
  const size_t E = c.n_experts, keys = (size_t)h->n_paged * E, S = c.cache_slots;
  if (S) {
    if (!hip_ok(hipMalloc(&h->slots, S * h->slot_bytes), "hipMalloc(cache slots)")) {
      h->slots = nullptr;
      return QS_E_NOMEM;
    }
    h->total_bytes += S * h->slot_bytes;
  }
  // (+16: the small-batch kernel copies a layer's map in 16-byte units)
  if (!hip_ok(hipMalloc(&h->d_emap, keys * 8 + 16), "hipMalloc(expert map)")) {
    h->d_emap = nullptr;
    return QS_E_NOMEM;
  }
  const size_t idsn = (size_t)c.n_layers * c.max_tokens * c.top_k;
  if (!hip_ok(hipMalloc(&h->ids_buf, idsn * 4), "hipMalloc(ids)")) {
    h->ids_buf = nullptr;
    return QS_E_NOMEM;
  }
  h->total_bytes += keys * 8 + idsn * 4;
  const size_t per = (size_t)h->n_paged * c.max_tokens * c.top_k;
  void* hp = nullptr;
  if (!hip_ok(hipHostMalloc(&hp, kRing * per * 4, hipHostMallocDefault), "hipHostMalloc(ids ring)"))
    return QS_E_NOMEM;
  h->ring_ids = (int32_t*)hp;
  h->ring.resize(kRing);
  for (int i = 0; i < kRing; ++i) {
    QS_HIP(hipEventCreateWithFlags(&h->ring[i].ev, hipEventDisableTiming));
    h->ring[i].ids = h->ring_ids + i * per;
  }
  h->emap.resize(keys);
  for (size_t key = 0; key < keys; ++key) h->emap[key] = host_addr(h, (int)key);
  QS_HIP(hipMemcpy(h->d_emap, h->emap.data(), keys * 8, hipMemcpyHostToDevice));
  h->slot_of.assign(keys, -1);
  h->owner.assign(S, -1);
  h->lru_prev.assign(S, -1);
  h->lru_next.assign(S, -1);
  h->copy_key.assign(S, -1);
  h->seen.assign(E, 0);
  for (size_t v = 0; v < S; ++v) h->free_slots.insert((int32_t)v);
  return QS_OK;
}

// A re-uploaded paged layer: its cached experts are dropped (their slots
// become free) and read from the new host records.
void cache_drop_layer(qs_moe* h, int pl) {
  const int E = h->cfg.n_experts;
  for (int e = 0; e < E; ++e) {
    const int key = pl * E + e, v = h->slot_of[key];
    if (v < 0) continue;
    lru_unlink(h, v);
    h->owner[v] = -1;
    h->copy_key[v] = -1;
    h->free_slots.insert(v);
    h->slot_of[key] = -1;
    h->dirty.push_back(key);
  }
}

// Shape of one persistent launch: LDS carve plus as much weight-staging
// buffer (up to kPfbMax) as the device's LDS leaves, the router unit, and
// whether the buffer holds one piece of every kind the kernel stages (the
// same sizes the kernel's staging plans use).
struct PersistShape {
  bool ok = false;
  uint32_t pfb = 0, pfa = 0;
  size_t lds = 0;
  int r_et = 1, r_tt = 1;
};

// fmt: the routed gate/up format of the launch's layers (QS_FMT_Q4K for
// the tail layers, whose down matrices are Q4_K-style too)
PersistShape big_shape(const qs_moe* h, int T, int fmt) {
  const qs_moe_config& c = h->cfg;
  PersistShape p;
  const bool cb2 = fmt == QS_FMT_CB2;
  const size_t base = big_layout(c.n_experts, T, T * c.top_k, cb2, 0).end;
  if (base >= h->lds_limit || h->grid < 8) return p;
  p.pfb = (uint32_t)std::min((size_t)kPfbMax, (h->lds_limit - base) & ~(size_t)15);
  p.lds = base + p.pfb;
  p.r_tt = T < 4 ? T : 4;
  while (p.r_et < 4 && (c.n_experts + p.r_et - 1) / p.r_et > h->grid) p.r_et *= 2;
  p.ok = big_plan(c.hidden, c.expert_ffn, c.shared_ffn, c.shared_format == QS_FMT_Q8, fmt,
                  fmt == QS_FMT_Q4K ? kFmtQ4K : kFmtQ2K, p.pfb, p.r_et * c.hidden * 4).ok;
  return p;
}

// (row, 64-weight chunk) units per thread in a 16-row gate/up tile of the
// small-batch kernel (the lane layout of gu_tile_load).
int gu_units(int H) {
  const int nch = H / kChunkW;
  int lpr = 64;
  while (nch % lpr) lpr >>= 1;
  const int slots = kPersistThreads / lpr;
  return (slots >= kGateTile ? 1 : kGateTile / slots) * (nch / lpr);
}

const void* persist_fixed_fn(const qs_moe* h, int T, bool steer = false, bool paged = false);

// paged: for the instantiations of paged layers, which have no fixed shape.
// fmt: the routed format of the launch's layers (-1: the 2-bit layers;
// QS_FMT_Q4K: the tail layers, gate/up and down both Q4_K-style)
PersistShape persist_shape(const qs_moe* h, int T, bool small, bool paged = false, int fmt = -1) {
  const qs_moe_config& c = h->cfg;
  const bool q4k = fmt == QS_FMT_Q4K;
  if (!small) return big_shape(h, T, q4k ? QS_FMT_Q4K : c.gate_up_format);
  PersistShape p;
  const bool cb2 = !q4k && c.gate_up_format == QS_FMT_CB2;
  const bool sq8 = c.shared_format == QS_FMT_Q8;
  // the shared expert through registers: the fixed-shape kernels above
  // hidden 2048 (sh_regs), the only small-batch kernels there
  const bool shregs = c.hidden > 2048 && !paged && !q4k;
  const size_t base = lds_layout(c.n_experts, T, T * c.top_k, c.hidden, c.expert_ffn, c.shared_ffn, sq8, cb2,
                                 small, 0, shregs, paged).end;
  if (base >= h->lds_limit || h->grid_small < 8) return p;
  p.pfb = (uint32_t)std::min((size_t)kPfbMax, (h->lds_limit - base) & ~(size_t)15);
  p.lds = base + p.pfb;
  p.r_tt = T < 4 ? T : 4;
  while (p.r_et < 4 && (c.n_experts + p.r_et - 1) / p.r_et > h->grid_small) p.r_et *= 2;
  const uint64_t H = c.hidden, F = c.expert_ffn, Fs = c.shared_ffn, nbh = H / 256, nb = F / 256;
  const uint64_t rb = (uint64_t)p.r_et * H * 4, item = big_item_b(c.hidden, sq8);
  const uint64_t tile = 2ull * 16 * nbh * (64 + (cb2 ? 4 : 16) + (cb2 ? 2 : 4));
  const uint64_t sd = big_sdrows_b(c.shared_ffn, sq8), pe = 8 * nb * blk_bytes(q4k ? kFmtQ4K : kFmtQ2K);
  auto a16 = [](uint64_t v) { return (v + 15) & ~15ull; };
  bool fits;
  if (small) {
    // region A: router rows + one shared item (phase R; no item when the
    // shared expert streams through registers); region B and the x limbs
    // after it: experts' down rows (D).  The shared down rows have their own
    // slot (none with registers).
    const uint64_t sitem = 4 * (uint64_t)srow_bytes(c.hidden, sq8);
    const uint64_t r_sh = a16(rb) + (Fs && !shregs ? sitem : 0);
    const uint64_t xl = 2 * a16((uint64_t)T * H) + 2 * a16((uint64_t)T * H / 4);
    const uint64_t A = a16(r_sh);
    p.pfa = (uint32_t)A;
    // the routed gate/up tiles stream through registers (at most kGuUnits
    // (row, chunk) units per thread and tile), not through the staging buffer
    // Hidden sizes above 2048 take the small-batch kernel only in a
    // fixed-shape instantiation: on the 4096-wide large-layer shape at T = 1
    // the generic one measured 83 us per layer against the batched kernel's
    // 73, the fixed one 57.
    fits = A <= p.pfb && (p.pfb - A) + xl >= pe && gu_units(c.hidden) <= kGuUnits &&
           (c.hidden <= 2048 || (!paged && !q4k && persist_fixed_fn(h, T) != nullptr));
    // with registers: a row's chunks per lane fit one register round
    if (shregs)
      fits = fits && (H / 4 + 511) / 512 <= (uint64_t)kShPairsLds && (Fs + 511) / 512 <= (uint64_t)kShDnRegs;
    (void)sd;
    // each flagged read is at most 32 words per thread
    const uint64_t P = (uint64_t)T * c.top_k;
    const uint64_t wa = 2 * P * (F / 4) + 2 * P * (F / 16) + (uint64_t)T * Fs;
    fits = fits && wa <= 32u * kPersistThreads && (uint64_t)T * H <= 32u * kPersistThreads &&
           2ull * T * c.n_experts <= 32u * kPersistThreads;
    // the gate/up items' cost split (gu_range) in 32-bit arithmetic: total
    // cost at most (F / 16) * 2 P
    fits = fits && 2ull * (h->grid_small + 1) * (F / kGateTile) * 2 * P < (1ull << 31);
  } else {
    fits = rb <= p.pfb && tile <= p.pfb && a16(sd) + pe <= p.pfb;
    // at least one shared item ahead of the routed tiles' slot
    if (Fs) fits = fits && item + tile <= p.pfb;
  }
  p.ok = fits;
  return p;
}

const void* persist_fn(bool cb2, bool small, bool steer = false) {
  if (steer) {
    if (cb2) return small ? (const void*)k_persist_small<2, true> : (const void*)k_persist_big<2, true>;
    return small ? (const void*)k_persist_small<1, true> : (const void*)k_persist_big<1, true>;
  }
  if (cb2) return small ? (const void*)k_persist_small<2, false> : (const void*)k_persist_big<2, false>;
  return small ? (const void*)k_persist_small<1, false> : (const void*)k_persist_big<1, false>;
}

// The instantiations for launches over paged layers (generic shapes only).
const void* persist_paged_fn(int fmt, bool small, bool steer) {
  if (fmt == kFmtQ4K)
    return steer ? (const void*)k_persist_big_paged<4, true> : (const void*)k_persist_big_paged<4, false>;
  if (fmt == kFmtCB2) {
    if (small) return steer ? (const void*)k_persist_small_paged<2, true> : (const void*)k_persist_small_paged<2, false>;
    return steer ? (const void*)k_persist_big_paged<2, true> : (const void*)k_persist_big_paged<2, false>;
  }
  if (small) return steer ? (const void*)k_persist_small_paged<1, true> : (const void*)k_persist_small_paged<1, false>;
  return steer ? (const void*)k_persist_big_paged<1, true> : (const void*)k_persist_big_paged<1, false>;
}

// Small-batch instantiations with the layer shape fixed at compile time:
// hidden 2048, 256 experts, top-8, expert width 512, shared width 512
// (bf16 or 8-bit) or 0, codebook gate/up, one workgroup per CU of a 256-CU
// device; with the steered combine (STEER) for the bf16 shared expert.
template <int FS, int SQ8, bool STEER = false, bool PG = false>
const void* fixed_a3b(int T) {
  switch (T) {
    case 1: return (const void*)k_persist_small_fixed<2, 2048, 256, 8, 512, FS, SQ8, 1, 256, STEER, PG>;
    case 2: return (const void*)k_persist_small_fixed<2, 2048, 256, 8, 512, FS, SQ8, 2, 256, STEER, PG>;
    case 3: return (const void*)k_persist_small_fixed<2, 2048, 256, 8, 512, FS, SQ8, 3, 256, STEER, PG>;
    case 4: return (const void*)k_persist_small_fixed<2, 2048, 256, 8, 512, FS, SQ8, 4, 256, STEER, PG>;
    default: return nullptr;
  }
}

// Batched instantiations with the layer shape fixed (the batch size stays a
// run-time value): the shapes above, and hidden 4096, 256 experts, top-6,
// expert and shared width 2048.
const void* persist_big_fixed_fn(const qs_moe* h, bool steer = false, bool paged = false) {
  const qs_moe_config& c = h->cfg;
  if (h->grid != 256 || c.gate_up_format != QS_FMT_CB2 || c.n_experts != 256) return nullptr;
  const bool sq8 = c.shared_format == QS_FMT_Q8;
  if (paged)   // paged layers: the A3B shape with the bf16 shared expert, unsteered
    return !steer && c.hidden == 2048 && c.top_k == 8 && c.expert_ffn == 512 && c.shared_ffn == 512 && !sq8
               ? (const void*)k_persist_big_fixed<2, 2048, 256, 8, 512, 512, 0, 256, false, true>
               : nullptr;
  if (steer) {
    if (c.hidden == 2048 && c.top_k == 8 && c.expert_ffn == 512 && c.shared_ffn == 512 && !sq8)
      return (const void*)k_persist_big_fixed<2, 2048, 256, 8, 512, 512, 0, 256, true>;
    return nullptr;
  }
  if (c.hidden == 2048 && c.top_k == 8 && c.expert_ffn == 512) {
    if (c.shared_ffn == 512 && sq8) return (const void*)k_persist_big_fixed<2, 2048, 256, 8, 512, 512, 1, 256>;
    if (c.shared_ffn == 512) return (const void*)k_persist_big_fixed<2, 2048, 256, 8, 512, 512, 0, 256>;
    if (c.shared_ffn == 0) return (const void*)k_persist_big_fixed<2, 2048, 256, 8, 512, 0, 0, 256>;
  }
  if (c.hidden == 4096 && c.top_k == 6 && c.expert_ffn == 2048 && c.shared_ffn == 2048 && !sq8)
    return (const void*)k_persist_big_fixed<2, 4096, 256, 6, 2048, 2048, 0, 256>;
  return nullptr;
}

// The fixed-shape kernel for a T-token call of this handle, or nullptr:
// the A3B shapes above at T = 1..4, and the large-layer shape (hidden 4096,
// 256 experts, top-6, expert and shared width 2048, bf16 shared expert) at
// T = 1.
const void* persist_fixed_fn(const qs_moe* h, int T, bool steer, bool paged) {
  const qs_moe_config& c = h->cfg;
  if (paged)   // paged layers: the A3B shape with the bf16 shared expert, unsteered
    return !steer && h->grid_small == 256 && c.gate_up_format == QS_FMT_CB2 && c.hidden == 2048 &&
                   c.n_experts == 256 && c.top_k == 8 && c.expert_ffn == 512 && c.shared_ffn == 512 &&
                   c.shared_format == QS_FMT_BF16
               ? fixed_a3b<512, 0, false, true>(T)
               : nullptr;
  if (!steer && T == 1 && h->grid_small == 256 && c.gate_up_format == QS_FMT_CB2 && c.hidden == 4096 &&
      c.n_experts == 256 && c.top_k == 6 && c.expert_ffn == 2048 && c.shared_ffn == 2048 &&
      c.shared_format == QS_FMT_BF16)
    return (const void*)k_persist_small_fixed<2, 4096, 256, 6, 2048, 2048, 0, 1, 256>;
  if (h->grid_small != 256 || c.gate_up_format != QS_FMT_CB2 || c.hidden != 2048 || c.n_experts != 256 ||
      c.top_k != 8 || c.expert_ffn != 512)
    return nullptr;
  if (steer) return c.shared_ffn == 512 && c.shared_format != QS_FMT_Q8 ? fixed_a3b<512, 0, true>(T) : nullptr;
  if (c.shared_ffn == 512 && c.shared_format == QS_FMT_Q8) return fixed_a3b<512, 1>(T);
  if (c.shared_ffn == 512) return fixed_a3b<512, 0>(T);
  if (c.shared_ffn == 0) return fixed_a3b<0, 0>(T);
  return nullptr;
}

// The fixed-shape small-batch instantiations of the Q4_K-style tail layers:
// the A3B shape with the bf16 shared expert, T = 1..4, unsteered.
const void* q4k_fixed_fn(const qs_moe* h, int T) {
  const qs_moe_config& c = h->cfg;
  if (h->grid_small != 256 || c.hidden != 2048 || c.n_experts != 256 || c.top_k != 8 || c.expert_ffn != 512 ||
      c.shared_ffn != 512 || c.shared_format != QS_FMT_BF16)
    return nullptr;
  switch (T) {
    case 1: return (const void*)k_persist_small_fixed<kFmtQ4K, 2048, 256, 8, 512, 512, 0, 1, 256>;
    case 2: return (const void*)k_persist_small_fixed<kFmtQ4K, 2048, 256, 8, 512, 512, 0, 2, 256>;
    case 3: return (const void*)k_persist_small_fixed<kFmtQ4K, 2048, 256, 8, 512, 512, 0, 3, 256>;
    case 4: return (const void*)k_persist_small_fixed<kFmtQ4K, 2048, 256, 8, 512, 512, 0, 4, 256>;
    default: return nullptr;
  }
}

// The batched instantiation of the Q4_K-style tail layers (GEMV items only).
const void* persist_q4k_fn(bool steer) {
  return steer ? (const void*)k_persist_big<kFmtQ4K, true> : (const void*)k_persist_big<kFmtQ4K, false>;
}

// Every workgroup must be resident at once for the grid barrier (a
// cooperative launch also enforces this).
bool fn_resident(const void* fn, size_t lds) {
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kPersistThreads, lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return occ >= 1;
}

bool persist_resident(const qs_moe* h, bool small, size_t lds, bool steer = false) {
  const void* fn = persist_fn(h->cfg.gate_up_format == QS_FMT_CB2, small, steer);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kPersistThreads, lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return occ >= 1;
}

// Set up the persistent kernels: layer table, barrier words, grid size and
// the residency check of each instantiation at its largest launch.
int setup_persistent(qs_moe* h) {
  const qs_moe_config& c = h->cfg;
  std::vector<LayerPtrs> tab(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerDev& L = h->layers[l];
    const int pl = l - c.resident_layers;   // paged layers read their experts through the map
    const uint64_t* em = L.host ? h->d_emap + (size_t)pl * c.n_experts : nullptr;
    tab[l] = LayerPtrs{L.router, L.bias, L.gate, L.up, L.down, L.sg, L.su, L.sd, em};
  }
  if (!hip_ok(hipMalloc(&h->d_layers, tab.size() * sizeof(LayerPtrs)), "hipMalloc(layers)")) {
    h->d_layers = nullptr;
    return QS_E_NOMEM;
  }
  if (!hip_ok(hipMemcpy(h->d_layers, tab.data(), tab.size() * sizeof(LayerPtrs), hipMemcpyHostToDevice),
              "hipMemcpy(layers)"))
    return QS_E_HIP;
  if (!hip_ok(hipMalloc(&h->sync, kSyncWords * 4), "hipMalloc(sync)")) {
    h->sync = nullptr;
    return QS_E_NOMEM;
  }
  if (!hip_ok(hipMemset(h->sync, 0, kSyncWords * 4), "hipMemset(sync)")) return QS_E_HIP;
  h->total_bytes += tab.size() * sizeof(LayerPtrs) + kSyncWords * 4;
  hipDeviceProp_t prop;
  if (!hip_ok(hipGetDeviceProperties(&prop, h->device), "hipGetDeviceProperties")) return QS_E_HIP;
  int coop = 0;
  (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h->device);
  h->grid = std::min(prop.multiProcessorCount & ~7, kMaxGrid);
  // The small-batch kernel exchanges data through flagged words that are
  // reused from layer to layer.  A workgroup rewrites layer l's words only
  // after it has seen layer l+1's input complete, which every workgroup
  // produces only after reading layer l's words -- provided every workgroup
  // owns a down tile (kDownRows output rows).  Hence at most H / kDownRows
  // workgroups.
  h->grid_small = std::min(h->grid, (c.hidden / kDownRows) & ~7);
  // dynamic LDS available to a workgroup: the device's LDS minus the largest
  // static LDS of the persistent instantiations (the block-wide vote of the
  // barrier keeps a few bytes there)
  size_t static_lds = 0;
  for (int cb = 0; cb < 2; ++cb)
    for (int sm = 0; sm < 2; ++sm)
      for (int st = 0; st < 2; ++st) {
        hipFuncAttributes fa;
        if (hipFuncGetAttributes(&fa, persist_fn(cb != 0, sm != 0, st != 0)) != hipSuccess) {
          (void)hipGetLastError();
          return QS_OK;
        }
        static_lds = std::max(static_lds, (size_t)fa.sharedSizeBytes);
      }
  for (int st = 0; st < 2; ++st) {
    const void* fns[] = {persist_q4k_fn(st != 0), persist_paged_fn(kFmtQ4K, false, st != 0),
                         st ? (const void*)k_persist_small<kFmtQ4K, true> : (const void*)k_persist_small<kFmtQ4K, false>,
                         persist_paged_fn(kFmtCB2, true, st != 0), persist_paged_fn(kFmtCB2, false, st != 0),
                         persist_paged_fn(kFmtQ2K, true, st != 0), persist_paged_fn(kFmtQ2K, false, st != 0)};
    for (const void* fn : fns) {
      hipFuncAttributes fa;
      if (hipFuncGetAttributes(&fa, fn) != hipSuccess) {
        (void)hipGetLastError();
        return QS_OK;
      }
      static_lds = std::max(static_lds, (size_t)fa.sharedSizeBytes);
    }
  }
  const size_t dev_lds = prop.maxSharedMemoryPerMultiProcessor;
  h->lds_limit = dev_lds > static_lds ? (dev_lds - static_lds) & ~(size_t)255 : 0;
  if (!coop || h->grid < 8) return QS_OK;
  // the largest LDS of each instantiation: the carve grows with T
  size_t lds_small = 0, lds_big = 0;
  for (int T = 1; T <= c.max_tokens; ++T) {
    if (T <= kSmallT) {
      const PersistShape p = persist_shape(h, T, true);
      if (p.ok) lds_small = std::max(lds_small, p.lds);
    }
    const PersistShape p = persist_shape(h, T, false);     // also the fallback of small batches
    if (p.ok) lds_big = std::max(lds_big, p.lds);
  }
  h->persist_small_ok = lds_small && persist_resident(h, true, lds_small);
  h->persist_big_ok = lds_big && persist_resident(h, false, lds_big);
  size_t lds4 = 0, lds_pg = 0;
  if (c.tail_layers > 0) {   // the Q4_K-style tail layers: the batched kernel at every T
    bool all = true;
    for (int T = 1; T <= c.max_tokens; ++T) {
      const PersistShape p = big_shape(h, T, QS_FMT_Q4K);
      all = all && p.ok;
      if (p.ok) lds4 = std::max(lds4, p.lds);
    }
    if (!all) lds4 = 0;
    h->q4k_ok = lds4 && fn_resident(persist_q4k_fn(false), lds4);
    h->q4k_steer_ok = h->q4k_ok && fn_resident(persist_q4k_fn(true), lds4);
    size_t lds4s = 0;   // the small-batch kernel for the tail layers' small batches
    for (int T = 1; T <= std::min(c.max_tokens, kSmallT); ++T) {
      const PersistShape p = persist_shape(h, T, true, false, QS_FMT_Q4K);
      if (p.ok) lds4s = std::max(lds4s, p.lds);
    }
    for (int st = 0; st < 2; ++st)
      h->q4k_small_ok[st] = lds4s && h->grid_small >= 8 &&
                            fn_resident(st ? (const void*)k_persist_small<kFmtQ4K, true>
                                           : (const void*)k_persist_small<kFmtQ4K, false>, lds4s);
    h->q4k_fixed_ok = h->q4k_small_ok[0];
    for (int T = 1; T <= kSmallT && h->q4k_fixed_ok; ++T) {
      const void* fn = q4k_fixed_fn(h, T);
      h->q4k_fixed_ok = fn && fn_resident(fn, lds4s);
    }
  }
  if (h->n_paged) {
    const int gf = c.gate_up_format == QS_FMT_CB2 ? kFmtCB2 : kFmtQ2K;
    // (the paged small-batch carve also holds the layer's expert map)
    for (int T = 1; T <= std::min(c.max_tokens, kSmallT); ++T) {
      const PersistShape p = persist_shape(h, T, true, true);
      if (p.ok) lds_pg = std::max(lds_pg, p.lds);
    }
    for (int st = 0; st < 2; ++st) {
      h->pg_small_ok[st] = lds_pg && fn_resident(persist_paged_fn(gf, true, st != 0), lds_pg);
      h->pg_big_ok[st] = lds_big && fn_resident(persist_paged_fn(gf, false, st != 0), lds_big);
      h->pg_q4k_ok[st] = lds4 && fn_resident(persist_paged_fn(kFmtQ4K, false, st != 0), lds4);
    }
  }
  h->steer_small_ok = h->persist_small_ok && persist_resident(h, true, lds_small, true);
  h->steer_big_ok = h->persist_big_ok && persist_resident(h, false, lds_big, true);
  // fixed-shape instantiations: the same LDS limits, checked one by one
  auto resident = [](const void* fn, size_t lds) {
    int occ = 0;
    const bool ok = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kPersistThreads, lds) == hipSuccess &&
                    occ >= 1;
    (void)hipGetLastError();
    return ok;
  };
  if (h->persist_big_ok) {
    const void* fn = persist_big_fixed_fn(h);
    h->big_fixed_ok = fn && resident(fn, lds_big);
    const void* fs = persist_big_fixed_fn(h, true);
    h->big_fixed_steer_ok = fs && resident(fs, lds_big);
  }
  if (h->n_paged) {
    const void* fb = persist_big_fixed_fn(h, false, true);
    h->pg_big_fixed_ok = h->pg_big_ok[0] && fb && resident(fb, lds_big);
    h->pg_fixed_ok = h->pg_small_ok[0];
    for (int T = 1; T <= kSmallT && h->pg_fixed_ok; ++T) {
      const void* fn = persist_fixed_fn(h, T, false, true);
      h->pg_fixed_ok = fn && resident(fn, lds_pg);
    }
  }
  h->fixed_ok = h->persist_small_ok;
  h->fixed_steer_ok = h->persist_small_ok;
  for (int T = 1; T <= kSmallT; ++T) {
    const void* fn = persist_fixed_fn(h, T);
    if (fn && h->fixed_ok) h->fixed_ok = resident(fn, lds_small);
    const void* fs = persist_fixed_fn(h, T, true);
    if (fs && h->fixed_steer_ok) h->fixed_steer_ok = resident(fs, lds_small);
  }
  return QS_OK;
}

// The kernel a T-token call runs: small batches take the small-batch
// instantiation when its working set fits and (with an explicit threshold)
// no bucket can reach the MFMA size, otherwise the batched one.  False when
// neither fits.
bool choose_kernel(const qs_moe* h, int T, bool& small, PersistShape& p, bool paged = false) {
  small = T <= kSmallT && (!h->mfma_explicit || T < h->mfma_min) &&
          (paged ? h->pg_small_ok[0] : h->persist_small_ok);
  if (small) {
    p = persist_shape(h, T, true, paged);
    small = p.ok;
  }
  if (!small) {
    if (!(paged ? h->pg_big_ok[0] : h->persist_big_ok)) return false;
    p = persist_shape(h, T, false);
    if (!p.ok) return false;
  }
  return true;
}

// Layers [layer0, layer0 + nL), all of one routed format, as one cooperative
// launch.  q4k: the Q4_K-style tail layers (batched kernel, GEMV items).
int launch_segment(qs_moe* h, const CallState& cs, int layer0, int nL, const float* x, float* y, int T,
                   bool residual, bool prenorm, bool steer, int32_t* ids_out, float* w_out, hipStream_t st,
                   bool q4k, bool exclusive) {
  const qs_moe_config& c = h->cfg;
  const bool cb2 = !q4k && c.gate_up_format == QS_FMT_CB2;
  // a launch over any paged layer takes the instantiations that read the map
  const bool paged = h->n_paged && layer0 + nL > c.resident_layers;
  bool small = false;
  PersistShape p;
  if (q4k) {
    // small batches of resident tail layers: the small-batch kernel when it fits
    small = !paged && T <= kSmallT && (!h->mfma_explicit || T < h->mfma_min) && h->q4k_small_ok[steer];
    if (small) {
      p = persist_shape(h, T, true, false, QS_FMT_Q4K);
      small = p.ok;
    }
    if (!small) {
      if (!(paged ? h->pg_q4k_ok[steer] : steer ? h->q4k_steer_ok : h->q4k_ok)) return QS_E_UNSUPPORTED;
      p = big_shape(h, T, QS_FMT_Q4K);
      if (!p.ok) return QS_E_UNSUPPORTED;
    }
  } else {
    if (!choose_kernel(h, T, small, p, paged)) return QS_E_UNSUPPORTED;   // (create checked every T)
    if (steer && !(paged ? (small ? h->pg_small_ok[1] : h->pg_big_ok[1])
                         : (small ? h->steer_small_ok : h->steer_big_ok)))
      return QS_E_UNSUPPORTED;
  }
  // the batched kernel's grid barriers: five per layer (six with steering)
  // but none after the last
  const uint32_t barriers = small ? 0u : (steer ? 6u : 5u) * nL - 1u;
  if (small && *cs.ll_epoch > 0xF0000000u - 3u * (uint32_t)nL) {
    // flags are about to wrap: clear the flagged buffers and start again
    launch_zero(cs.zero_base, cs.zero_bytes, st);
    *cs.ll_epoch = 0;
  }
  if (*cs.epoch + barriers > (1u << 26)) {
    hipLaunchKernelGGL(k_sync_reset, dim3(1), dim3(256), 0, st, cs.sync);
    *cs.epoch = 0;
  }
  const Scratch& s = *cs.s;
  PersistArgs a{};
  a.layers = h->d_layers + layer0;
  a.G = small ? h->grid_small : h->grid;
  a.spin_ll = h->wait_limit ? h->wait_limit : kLLSpinMax;
  a.spin_bar = h->wait_limit ? h->wait_limit : kSpinMax;
  a.n_layers = nL;
  a.T = T; a.H = c.hidden; a.E = c.n_experts; a.k = c.top_k; a.F = c.expert_ffn; a.Fs = c.shared_ffn;
  a.gq2k = !q4k && c.gate_up_format == QS_FMT_Q2K;
  a.gfmt = q4k ? kFmtQ4K : c.gate_up_format;
  a.dfmt = q4k ? kFmtQ4K : kFmtQ2K;
  a.sq8 = c.shared_format == QS_FMT_Q8;
  a.prenorm = prenorm;
  a.residual = residual;
  a.r_tt = p.r_tt;
  a.r_et = p.r_et;
  a.pfb = p.pfb;
  a.pfa = p.pfa;
  a.gu_stride = q4k ? h->gu_stride4 : h->gu_stride;
  a.dn_stride = q4k ? h->dn_stride4 : h->dn_stride;
  a.cbtab = h->cbtab;
  a.x_in = x; a.y_out = y; a.ids_out = ids_out; a.w_out = w_out;
  a.logits = s.logits; a.rinv = s.rinv; a.ids = s.ids; a.wts = s.wts;
  a.xh = s.xh; a.xl = s.xl; a.xs = s.xs; a.xa = s.xa;
  a.ah = s.ah; a.al = s.al; a.as = s.as; a.aa = s.aa; a.ash = s.ash;
  a.xbuf0 = s.xbuf[0]; a.xbuf1 = s.xbuf[1];
  // default threshold: one-token buckets of a one-token batch stay on the
  // GEMV items (measured faster there: Flash stack T = 1, 1680 vs 1274 tok/s)
  a.mfma_min = !h->mfma_explicit && T == 1 ? 2 : h->mfma_min;
  if (q4k) a.mfma_min = 1 << 30;   // GEMV items only (batched kernel)
  a.ll_lg = s.ll_lg; a.ll_a = s.ll_a; a.llx0 = s.llx[0]; a.llx1 = s.llx[1];
  a.ll_epoch = *cs.ll_epoch;
  a.af = s.af; a.ob = s.ob; a.sb = s.sb;
  a.ll_dot = s.ll_dot; a.mb = s.mb; a.part = s.part;
  a.sscale = h->steer_scale;
  a.sdir = steer ? h->steer_dirs + (size_t)layer0 * c.hidden : nullptr;
  a.sync = cs.sync;
  a.epoch0 = *cs.epoch;
  void* args[] = {&a};
  // the fixed-shape kernel needs the router unit it assumes (one expert per
  // workgroup, all tokens at once)
  const void* fn = nullptr;
  if (paged) {
    if (!q4k && !steer && small && h->pg_fixed_ok && p.r_et == 1 && p.r_tt == T)
      fn = persist_fixed_fn(h, T, false, true);
    if (!q4k && !steer && !small && h->pg_big_fixed_ok && p.r_et == 1) fn = persist_big_fixed_fn(h, false, true);
    if (!fn) fn = persist_paged_fn(q4k ? kFmtQ4K : cb2 ? kFmtCB2 : kFmtQ2K, small, steer);
  } else if (q4k) {
    if (small && !steer && h->q4k_fixed_ok && p.r_et == 1 && p.r_tt == T) fn = q4k_fixed_fn(h, T);
    if (!fn)
      fn = small ? (steer ? (const void*)k_persist_small<kFmtQ4K, true> : (const void*)k_persist_small<kFmtQ4K, false>)
                 : persist_q4k_fn(steer);
  } else {
    if (small && (steer ? h->fixed_steer_ok : h->fixed_ok) && p.r_et == 1 && p.r_tt == T)
      fn = persist_fixed_fn(h, T, steer);
    if (!small && (steer ? h->big_fixed_steer_ok : h->big_fixed_ok) && p.r_et == 1)
      fn = persist_big_fixed_fn(h, steer);
    if (!fn) fn = persist_fn(cb2, small, steer);
  }
  // (every workgroup must be resident at once: a cooperative launch
  // guarantees it; an exclusive caller guarantees that nothing else holds
  // the compute units, and the create-time occupancy check that one
  // workgroup fits each of the grid's CUs)
  hipError_t e = exclusive ? hipLaunchKernel(fn, dim3(a.G), dim3(kPersistThreads), args, (size_t)p.lds, st)
                           : hipLaunchCooperativeKernel(fn, dim3(a.G), dim3(kPersistThreads), args,
                                                        (unsigned)p.lds, st);
  if (e != hipSuccess) {
    fprintf(stderr, "qs_moe: persistent launch failed: %s\n", hipGetErrorString(e));
    return QS_E_HIP;
  }
  *cs.epoch += barriers;
  if (small) *cs.ll_epoch += 3u * (uint32_t)nL;
  return QS_OK;
}

// The whole decode call: one launch per run of layers of one routed format
// (the 2-bit layers, then the Q4_K-style tail layers), chained through y.
int launch_persistent(qs_moe* h, const CallState& cs, int layer0, int nL, const float* x, float* y, int T,
                      bool residual, bool prenorm, bool steer, int32_t* ids_out, float* w_out, hipStream_t st,
                      bool exclusive) {
  const qs_moe_config& c = h->cfg;
  const int split = c.n_layers - c.tail_layers;   // the first tail layer
  if (layer0 + nL <= split || layer0 >= split)
    return launch_segment(h, cs, layer0, nL, x, y, T, residual, prenorm, steer, ids_out, w_out, st,
                          layer0 >= split, exclusive);
  // (several layers: the residual chain, so the second run continues in y)
  const int n1 = split - layer0;
  int rc = launch_segment(h, cs, layer0, n1, x, y, T, residual, prenorm, steer, ids_out, w_out, st, false,
                          exclusive);
  if (rc) return rc;
  const size_t skip = (size_t)n1 * T * c.top_k;
  return launch_segment(h, cs, split, nL - n1, y, y, T, residual, prenorm, steer, ids_out ? ids_out + skip : nullptr,
                        w_out ? w_out + skip : nullptr, st, true, exclusive);
}

int check_layer_range(const qs_moe* h, int layer0, int n) {
  if (layer0 < 0 || n < 1 || layer0 + n > h->cfg.n_layers) return QS_E_INVAL;
  for (int l = layer0; l < layer0 + n; ++l)
    if (!h->layers[l].uploaded) return QS_E_STATE;
  return QS_OK;
}

// Router, top-k and grouping of one layer.
int launch_route(qs_moe* h, const LayerDev& L, const float* x, int T, bool prenorm,
                 int32_t* ids_out, float* w_out, hipStream_t st) {
  const qs_moe_config& c = h->cfg;
  const int E = c.n_experts, k = c.top_k, H = c.hidden;
  Scratch& s = h->s;
  hipLaunchKernelGGL(k_router, dim3((E + 3) / 4), dim3(256), 0, st, L.router, L.bias, x, T, H, E,
                     (int)prenorm, s.logits, s.rinv);
  hipLaunchKernelGGL(k_topk, dim3(T), dim3(64), 0, st, (const double*)s.logits, E, k, s.ids, s.wts,
                     ids_out, w_out);
  GroupOut g{s.cnt, s.off, s.pairs, s.n_active, s.active, s.tok_order};
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, st, (const int32_t*)s.ids, T, k, E, g);
  return hipGetLastError() == hipSuccess ? QS_OK : QS_E_HIP;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Host-side argument checks of a decode call (nothing is enqueued on error).
int check_decode_args(const qs_moe* h, int layer0, int n_layers, const float* x, const float* y,
                      int n_tokens, uint32_t flags) {
  if (!h || !x || !y) return QS_E_INVAL;
  const qs_moe_config& c = h->cfg;
  if (flags & ~(QS_DECODE_RESIDUAL | QS_DECODE_RMSNORM | QS_DECODE_STEER | QS_DECODE_EXCLUSIVE)) return QS_E_INVAL;
  if (n_tokens < 1 || n_tokens > c.max_tokens) return QS_E_INVAL;
  if (((uintptr_t)x | (uintptr_t)y) & 15) return QS_E_INVAL;
  const bool residual = flags & QS_DECODE_RESIDUAL;
  if (!residual && n_layers != 1) return QS_E_INVAL;
  const size_t act_bytes = (size_t)n_tokens * c.hidden * sizeof(float);
  if (!residual && ranges_overlap(x, act_bytes, y, act_bytes)) return QS_E_INVAL;
  if (residual && x != y && ranges_overlap(x, act_bytes, y, act_bytes)) return QS_E_INVAL;
  const int rc = check_layer_range(h, layer0, n_layers);
  if (rc) return rc;
  if ((flags & QS_DECODE_STEER) && !h->steer_dirs) return QS_E_STATE;   // no qs_moe_set_steering
  return QS_OK;
}

// ---------------------------------------------- static decode scratch ---
// qs_moe_decode_static keeps every per-call buffer (sync words, flagged
// words, logits, activation limbs, partial outputs) in one file-scope device
// array instead of the handle's allocation.  Each device the library runs
// on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in: its device address, per device, comes from
// hipGetSymbolAddress once (at the first qs_moe_create on that device) and
// only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = size_t(12) << 20;
constexpr size_t kStaticSyncBytes = 4096;       // the sync words, then the carve
constexpr int kMaxDevices = 64;

struct StaticDev {
  uint8_t* base = nullptr;   // device address of `scratch` on this device
  uint32_t epoch = 0;        // barriers completed on its sync words
  uint32_t ll_epoch = 0;     // flags used on its flagged words
};
StaticDev g_static[kMaxDevices];
std::mutex g_static_mu;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// With `dev` current: look up this device's copy of the array and zero it
// (sync words, and flagged words that must never match a later flag).
int static_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return QS_OK;   // the static variant then refuses
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDev& sd = g_static[dev];
  if (sd.base) return QS_OK;
  void* ptr = nullptr;
  if (!hip_ok(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return QS_E_HIP;
  launch_zero(ptr, kStaticScratchBytes, nullptr);
  if (!hip_ok(hipGetLastError(), "zero static scratch") || !hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize"))
    return QS_E_HIP;
  sd.base = (uint8_t*)ptr;
  return QS_OK;
}

}  // namespace

extern "C" {

QS_API const char* qs_moe_status_string(int status) {
  switch (status) {
    case QS_OK: return "ok";
    case QS_E_INVAL: return "invalid argument";
    case QS_E_NOMEM: return "out of memory";
    case QS_E_HIP: return "HIP runtime error";
    case QS_E_STATE: return "layer not uploaded";
    case QS_E_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

QS_API int qs_moe_create(const qs_moe_config* cfg, const int8_t* codebook, qs_moe** out) {
  if (!out) return QS_E_INVAL;
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  const bool need_cb = cfg->gate_up_format == QS_FMT_CB2 || cfg->down_format == QS_FMT_CB2;
  if (need_cb && !codebook) return QS_E_INVAL;

  qs_moe* h = new (std::nothrow) qs_moe();
  if (!h) return QS_E_NOMEM;
  h->cfg = *cfg;
  // default: the small-batch kernel (GEMV only) up to kSmallT tokens, the
  // matrix cores for every bucket of a larger batch in the batched kernel
  // (measured: T = 16 +39 %, T = 32 +32 % over a threshold of 16)
  h->mfma_explicit = cfg->mfma_min_tokens != 0;
  h->mfma_min = cfg->mfma_min_tokens ? cfg->mfma_min_tokens : 1;
  DeviceGuard dg(cfg->device);
  if (!dg.ok) {
    fprintf(stderr, "qs_moe: hipSetDevice(%d) failed\n", cfg->device);
    delete h;
    return QS_E_HIP;
  }
  if (!hip_ok(hipGetDevice(&h->device), "hipGetDevice")) {
    delete h;
    return QS_E_HIP;
  }
  const qs_moe_config& c = h->cfg;
  const size_t E = c.n_experts, H = c.hidden, F = c.expert_ffn, Fs = c.shared_ffn;
  const size_t gu_blk = F * (H / kBlockW), dn_blk = H * (F / kBlockW);
  h->gu_stride = align_up(gu_blk * gate_up_block_bytes(c), 256);
  h->dn_stride = align_up(dn_blk * kQ2KBytes, 256);
  h->gu_stride4 = align_up(gu_blk * blk_bytes(kFmtQ4K), 256);
  h->dn_stride4 = align_up(dn_blk * blk_bytes(kFmtQ4K), 256);
  const bool sq8 = c.shared_format == QS_FMT_Q8;
  const size_t sgu = Fs * (size_t)srow_bytes((int)H, sq8), sdn = H * (size_t)srow_bytes((int)Fs, sq8);
  h->layers.resize(c.n_layers);
  rc = QS_OK;
  h->n_paged = c.expert_paging ? c.n_layers - c.resident_layers : 0;
  for (int l = 0; l < c.n_layers && rc == QS_OK; ++l) {
    LayerDev& L = h->layers[l];
    L.q4k = l >= c.n_layers - c.tail_layers;
    const size_t gs = L.q4k ? h->gu_stride4 : h->gu_stride, ds = L.q4k ? h->dn_stride4 : h->dn_stride;
    const bool paged = h->n_paged && l >= c.resident_layers;
    size_t lb = align_up(E * H * 4, 256) + align_up(E * 4, 256) + (paged ? 0 : 2 * E * gs + E * ds);
    if (Fs) lb += 2 * align_up(sgu, 256) + align_up(sdn, 256);
    if (!hip_ok(hipMalloc(&L.base, lb), "hipMalloc(layer)")) {
      L.base = nullptr;
      rc = QS_E_NOMEM;
      break;
    }
    uint8_t* p = L.base;
    L.router = carve<float>(p, E * H);
    L.bias = carve<float>(p, E);
    if (paged) {   // the routed experts: one record per expert in pinned host memory
      L.rec_bytes = 2 * gs + ds;
      void* hp = nullptr;
      if (!hip_ok(hipHostMalloc(&hp, E * L.rec_bytes, hipHostMallocDefault), "hipHostMalloc(experts)")) {
        rc = QS_E_NOMEM;
        break;
      }
      L.host = (uint8_t*)hp;
      void* dp = nullptr;
      if (!hip_ok(hipHostGetDevicePointer(&dp, hp, 0), "hipHostGetDevicePointer")) {
        rc = QS_E_HIP;
        break;
      }
      L.host_dev = (uint64_t)(uintptr_t)dp;
      h->host_bytes += E * L.rec_bytes;
      h->slot_bytes = std::max(h->slot_bytes, L.rec_bytes);
    } else {
      L.gate = p; p += E * gs;
      L.up = p; p += E * gs;
      L.down = p; p += E * ds;
    }
    if (Fs) {
      L.sg = carve<uint8_t>(p, sgu);
      L.su = carve<uint8_t>(p, sgu);
      L.sd = carve<uint8_t>(p, sdn);
    }
    h->total_bytes += lb;
    h->layer_bytes = std::max(h->layer_bytes, lb);
  }
  if (rc == QS_OK) {
    h->s.bytes = scratch_bytes(c);
    if (!hip_ok(hipMalloc(&h->s.base, h->s.bytes), "hipMalloc(scratch)")) {
      h->s.base = nullptr;
      rc = QS_E_NOMEM;
    } else {
      carve_scratch(c, h->s);
      h->total_bytes += h->s.bytes;
      if (!hip_ok(hipMemset(h->s.base, 0, h->s.ll_bytes), "hipMemset(flags)")) rc = QS_E_HIP;
    }
  }
  if (rc == QS_OK) {
    std::vector<uint32_t> tab;
    std::vector<int8_t> ones(256 * 8, 1);
    build_cb_tables(codebook ? codebook : ones.data(), tab);
    if (!hip_ok(hipMalloc(&h->cbtab, tab.size() * 4), "hipMalloc(codebook)")) {
      h->cbtab = nullptr;
      rc = QS_E_NOMEM;
    } else if (!hip_ok(hipMemcpy(h->cbtab, tab.data(), tab.size() * 4, hipMemcpyHostToDevice),
                       "hipMemcpy(codebook)")) {
      rc = QS_E_HIP;
    } else {
      h->total_bytes += tab.size() * 4;
    }
  }
  if (rc == QS_OK && h->n_paged) rc = setup_paging(h);
  if (rc == QS_OK) rc = setup_persistent(h);
  if (rc == QS_OK) rc = static_setup(h->device);
  if (rc == QS_OK) {
    if (!hip_ok(hipHostMalloc((void**)&h->host_err, 256, hipHostMallocDefault), "hipHostMalloc(status)")) {
      h->host_err = nullptr;
      rc = QS_E_NOMEM;
    }
  }
  if (rc == QS_OK) {
    // every batch size up to max_tokens must have a persistent kernel that
    // fits the device (there is no other decode path), for the 2-bit layers
    // and for the Q4_K-style tail layers
    // (with paging, layers [resident_layers, n_layers) run the paged
    // instantiations, and a call that reaches them runs them throughout)
    const int split = c.n_layers - c.tail_layers, R = h->n_paged ? c.resident_layers : c.n_layers;
    const bool res2 = split > 0 && (R > 0 || !h->n_paged), pg2 = h->n_paged && R < split;
    for (int T = 1; T <= c.max_tokens && rc == QS_OK; ++T) {
      bool small = false;
      PersistShape p;
      if ((res2 && !choose_kernel(h, T, small, p)) || (pg2 && !choose_kernel(h, T, small, p, true))) {
        fprintf(stderr, "qs_moe: no persistent decode kernel fits a %d-token call of this shape\n", T);
        rc = QS_E_UNSUPPORTED;
      }
    }
    if (rc == QS_OK && c.tail_layers > 0 && (!h->q4k_ok || (h->n_paged && !h->pg_q4k_ok[0]))) {
      fprintf(stderr, "qs_moe: the batched decode kernel of the Q4_K-style layers does not fit this shape\n");
      rc = QS_E_UNSUPPORTED;
    }
  }
  if (rc != QS_OK) {
    free_all(h);
    delete h;
    return rc;
  }
  *out = h;
  return QS_OK;
}

QS_API int qs_moe_upload(qs_moe* h, int layer, const qs_moe_layer_weights* w, void* hip_stream) {
  if (!h || !w) return QS_E_INVAL;
  const qs_moe_config& c = h->cfg;
  if (layer < 0 || layer >= c.n_layers) return QS_E_INVAL;
  if (!w->router || !w->gate || !w->up || !w->down) return QS_E_INVAL;
  if (c.shared_ffn && (!w->shared_gate || !w->shared_up || !w->shared_down)) return QS_E_INVAL;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  const size_t E = c.n_experts, H = c.hidden, F = c.expert_ffn, Fs = c.shared_ffn;
  LayerDev& L = h->layers[layer];
  L.uploaded = false;
  QS_HIP(hipMemcpyAsync(L.router, w->router, E * H * 4, hipMemcpyDefault, st));
  if (w->router_bias)
    QS_HIP(hipMemcpyAsync(L.bias, w->router_bias, E * 4, hipMemcpyDefault, st));
  else
    QS_HIP(hipMemsetAsync(L.bias, 0, E * 4, st));
  const bool sq8 = c.shared_format == QS_FMT_Q8;
  if (Fs && !sq8) {   // bf16 rows are already the kernels' layout
    QS_HIP(hipMemcpyAsync(L.sg, w->shared_gate, Fs * H * 2, hipMemcpyDefault, st));
    QS_HIP(hipMemcpyAsync(L.su, w->shared_up, Fs * H * 2, hipMemcpyDefault, st));
    QS_HIP(hipMemcpyAsync(L.sd, w->shared_down, Fs * H * 2, hipMemcpyDefault, st));
  }
  const size_t gu_blk = F * (H / kBlockW), dn_blk = H * (F / kBlockW);
  const bool q4 = L.q4k;   // a tail layer: every routed matrix in the Q4_K-style format
  const size_t gbb = q4 ? (size_t)kQ4KBytes : gate_up_block_bytes(c);
  const size_t dbb = q4 ? (size_t)kQ4KBytes : (size_t)kQ2KBytes;
  const size_t q8_raw = Fs * (H / kQ8W) * (size_t)kQ8Bytes;   // one shared matrix in 8-bit blocks
  const size_t need = std::max({E * gu_blk * gbb, E * dn_blk * dbb, sq8 ? q8_raw : (size_t)0});
  if (h->staging_bytes < need) {
    if (h->staging) QS_HIP(hipFree(h->staging));
    h->staging = nullptr;
    h->staging_bytes = 0;
    if (hipMalloc(&h->staging, need) != hipSuccess) {
      h->staging = nullptr;
      return QS_E_NOMEM;
    }
    h->staging_bytes = need;
  }
  struct Job { const void* src; uint8_t* dst; size_t nblk; size_t stride; int fmt; };
  const int gfmt = q4 ? kFmtQ4K : c.gate_up_format, dfmt = q4 ? kFmtQ4K : kFmtQ2K;
  const size_t gst = q4 ? h->gu_stride4 : h->gu_stride, dst_ = q4 ? h->dn_stride4 : h->dn_stride;
  const bool paged = L.host != nullptr;
  if (paged && !h->pstage) {   // a paged layer's records are re-laid in HBM, then copied to host
    if (hipMalloc(&h->pstage, E * h->slot_bytes) != hipSuccess) {
      h->pstage = nullptr;
      return QS_E_NOMEM;
    }
  }
  // a paged layer: expert e's record [gate | up | down] at e * rec_bytes
  const size_t rs = L.rec_bytes;
  const Job jobs[3] = {
      {w->gate, paged ? h->pstage : L.gate, gu_blk, paged ? rs : gst, gfmt},
      {w->up, paged ? h->pstage + gst : L.up, gu_blk, paged ? rs : gst, gfmt},
      {w->down, paged ? h->pstage + 2 * gst : L.down, dn_blk, paged ? rs : dst_, dfmt},
  };
  for (const Job& j : jobs) {
    const size_t raw = j.fmt == kFmtCB2 ? kCB2Bytes : j.fmt == kFmtQ4K ? kQ4KBytes : kQ2KBytes;
    QS_HIP(hipMemcpyAsync(h->staging, j.src, E * j.nblk * raw, hipMemcpyDefault, st));
    const size_t total = E * j.nblk;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (j.fmt == kFmtCB2)
      hipLaunchKernelGGL(k_repack_cb2, grid, dim3(256), 0, st, (const uint8_t*)h->staging, j.dst,
                         j.nblk, j.stride, E);
    else if (j.fmt == kFmtQ4K)
      hipLaunchKernelGGL(k_repack_q4k, grid, dim3(256), 0, st, (const uint8_t*)h->staging, j.dst,
                         j.nblk, j.stride, E);
    else
      hipLaunchKernelGGL(k_repack_q2k, grid, dim3(256), 0, st, (const uint8_t*)h->staging, j.dst,
                         j.nblk, j.stride, E);
    QS_HIP(hipGetLastError());
  }
  if (Fs && sq8) {    // 8-bit blocks -> padded rows [codes | scales]
    struct SJob { const void* src; uint8_t* dst; size_t rows; int K; };
    const SJob sj[3] = {{w->shared_gate, L.sg, Fs, (int)H}, {w->shared_up, L.su, Fs, (int)H},
                        {w->shared_down, L.sd, H, (int)Fs}};
    for (const SJob& j : sj) {
      QS_HIP(hipMemcpyAsync(h->staging, j.src, q8_raw, hipMemcpyDefault, st));
      const size_t total = j.rows * (size_t)(j.K / kQ8W);
      hipLaunchKernelGGL(k_repack_q8, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                         (const uint8_t*)h->staging, j.dst, j.rows, j.K, srow_bytes(j.K, true));
      QS_HIP(hipGetLastError());
    }
  }
  if (paged) {
    QS_HIP(hipMemcpyAsync(L.host, h->pstage, E * rs, hipMemcpyDeviceToHost, st));
    cache_drop_layer(h, layer - c.resident_layers);
    const int rc = cache_flush(h, st);
    if (rc) return rc;
  }
  QS_HIP(hipStreamSynchronize(st));
  L.uploaded = true;
  return QS_OK;
}

QS_API int qs_moe_decode(qs_moe* h, int layer0, int n_layers, const float* x, float* y, int n_tokens,
                  uint32_t flags, int32_t* ids_out, float* w_out, void* hip_stream) {
  int rc = check_decode_args(h, layer0, n_layers, x, y, n_tokens, flags);
  if (rc) return rc;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  const CallState cs{&h->s, h->sync, &h->epoch, &h->ll_epoch, h->s.base, h->s.ll_bytes};
  hipStream_t st = (hipStream_t)hip_stream;
  const bool paged = h->n_paged && layer0 + n_layers > h->cfg.resident_layers;
  if (paged) {   // admissions of earlier calls that have completed
    rc = cache_poll(h, st, false);
    if (rc) return rc;
  }
  int32_t* ids = paged && !ids_out ? h->ids_buf : ids_out;
  rc = launch_persistent(h, cs, layer0, n_layers, x, y, n_tokens, (flags & QS_DECODE_RESIDUAL) != 0,
                         (flags & QS_DECODE_RMSNORM) != 0, (flags & QS_DECODE_STEER) != 0, ids, w_out, st,
                         (flags & QS_DECODE_EXCLUSIVE) != 0);
  if (rc || !paged) return rc;
  return cache_record(h, ids, layer0, n_layers, n_tokens, st);
}

QS_API int qs_moe_decode_static(qs_moe* h, int layer0, int n_layers, const float* x, float* y,
                                int n_tokens, uint32_t flags, int32_t* ids_out, float* w_out,
                                void* hip_stream) {
  int rc = check_decode_args(h, layer0, n_layers, x, y, n_tokens, flags);
  if (rc) return rc;
  if (h->device < 0 || h->device >= kMaxDevices) return QS_E_UNSUPPORTED;
  // this call's scratch, carved for exactly n_tokens tokens
  qs_moe_config cc = h->cfg;
  cc.max_tokens = n_tokens;
  const size_t need = kStaticSyncBytes + scratch_bytes(cc);
  if (need > kStaticScratchBytes) {
    fprintf(stderr, "qs_moe: qs_moe_decode_static needs %zu bytes of scratch for %d tokens of this shape; "
            "its static scratch holds %zu\n", need, n_tokens, kStaticScratchBytes);
    return QS_E_UNSUPPORTED;
  }
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDev& sd = g_static[h->device];
  if (!sd.base) return QS_E_STATE;            // set up by qs_moe_create on this device
  Scratch s;
  s.base = sd.base + kStaticSyncBytes;
  s.bytes = scratch_bytes(cc);
  carve_scratch(cc, s);
  const CallState cs{&s, (uint32_t*)sd.base, &sd.epoch, &sd.ll_epoch, s.base,
                     kStaticScratchBytes - kStaticSyncBytes};
  return launch_persistent(h, cs, layer0, n_layers, x, y, n_tokens, (flags & QS_DECODE_RESIDUAL) != 0,
                           (flags & QS_DECODE_RMSNORM) != 0, (flags & QS_DECODE_STEER) != 0, ids_out, w_out,
                           (hipStream_t)hip_stream, (flags & QS_DECODE_EXCLUSIVE) != 0);
}

QS_API int qs_moe_sync_status(qs_moe* h, void* hip_stream) {
  if (!h) return QS_E_INVAL;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  // the handle's error flag and that of the device's static scratch (the
  // calls of qs_moe_decode_static)
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDev* sd = h->device >= 0 && h->device < kMaxDevices && g_static[h->device].base ? &g_static[h->device]
                                                                                        : nullptr;
  h->host_err[0] = h->host_err[1] = 0;
  QS_HIP(hipMemcpyAsync(h->host_err, h->sync + kSyncError, 4, hipMemcpyDeviceToHost, st));
  if (sd) QS_HIP(hipMemcpyAsync(h->host_err + 1, (uint32_t*)sd->base + kSyncError, 4, hipMemcpyDeviceToHost, st));
  QS_HIP(hipStreamSynchronize(st));
  if (h->host_err[0] == 0 && h->host_err[1] == 0) return QS_OK;
  // A wait gave up: the barrier counters may be out of step with the epoch.
  // Clear every sync word (the error flag included) with a kernel, so the
  // next call starts from a consistent state.  The flagged buffers need no
  // reset: the flags of later calls are larger than any written so far.
  if (h->host_err[0]) {
    hipLaunchKernelGGL(k_sync_reset, dim3(1), dim3(256), 0, st, h->sync);
    h->epoch = 0;
  }
  if (h->host_err[1]) {
    hipLaunchKernelGGL(k_sync_reset, dim3(1), dim3(256), 0, st, (uint32_t*)sd->base);
    sd->epoch = 0;
  }
  QS_HIP(hipGetLastError());
  QS_HIP(hipStreamSynchronize(st));
  fprintf(stderr, "qs_moe: a decode call gave up a bounded wait; its outputs are undefined\n");
  return QS_E_HIP;
}

QS_API int qs_moe_set_steering(qs_moe* h, const float* dirs, float scale, void* hip_stream) {
  if (!h || !std::isfinite(scale)) return QS_E_INVAL;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  const qs_moe_config& c = h->cfg;
  const size_t bytes = (size_t)c.n_layers * c.hidden * sizeof(float);
  if (!dirs) {
    if (h->steer_dirs) {
      QS_HIP(hipDeviceSynchronize());   // no decode call still reads them
      QS_HIP(hipFree(h->steer_dirs));
      h->total_bytes -= bytes;
    }
    h->steer_dirs = nullptr;
    h->steer_scale = 0.f;
    return QS_OK;
  }
  if (!h->steer_dirs) {
    if (hipMalloc(&h->steer_dirs, bytes) != hipSuccess) {
      h->steer_dirs = nullptr;
      return QS_E_NOMEM;
    }
    h->total_bytes += bytes;
  }
  QS_HIP(hipMemcpyAsync(h->steer_dirs, dirs, bytes, hipMemcpyDefault, st));
  QS_HIP(hipStreamSynchronize(st));
  h->steer_scale = scale;
  return QS_OK;
}

QS_API int qs_moe_set_wait_limit(qs_moe* h, int32_t polls) {
  if (!h || polls < 0) return QS_E_INVAL;
  h->wait_limit = polls;
  return QS_OK;
}

QS_API int qs_moe_route(qs_moe* h, int layer, const float* x, int n_tokens, uint32_t flags,
                        double* logits_out, int32_t* ids_out, float* w_out, int32_t* group_out,
                        void* hip_stream) {
  if (!h || !x) return QS_E_INVAL;
  const qs_moe_config& c = h->cfg;
  if (flags & ~QS_DECODE_RMSNORM) return QS_E_INVAL;
  if (n_tokens < 1 || n_tokens > c.max_tokens) return QS_E_INVAL;
  if ((uintptr_t)x & 15) return QS_E_INVAL;
  int rc = check_layer_range(h, layer, 1);
  if (rc) return rc;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  rc = launch_route(h, h->layers[layer], x, n_tokens, (flags & QS_DECODE_RMSNORM) != 0, ids_out,
                    w_out, st);
  if (rc) return rc;
  const size_t E = c.n_experts, P = (size_t)n_tokens * c.top_k;
  Scratch& s = h->s;
  if (logits_out)
    QS_HIP(hipMemcpyAsync(logits_out, s.logits, n_tokens * E * 8, hipMemcpyDeviceToDevice, st));
  if (group_out) {
    QS_HIP(hipMemcpyAsync(group_out, s.cnt, E * 4, hipMemcpyDeviceToDevice, st));
    QS_HIP(hipMemcpyAsync(group_out + E, s.off, (E + 1) * 4, hipMemcpyDeviceToDevice, st));
    QS_HIP(hipMemcpyAsync(group_out + 2 * E + 1, s.pairs, P * 4, hipMemcpyDeviceToDevice, st));
    QS_HIP(hipMemcpyAsync(group_out + 2 * E + 1 + P, s.n_active, 4, hipMemcpyDeviceToDevice, st));
    QS_HIP(hipMemcpyAsync(group_out + 2 * E + 2 + P, s.active, E * 4, hipMemcpyDeviceToDevice, st));
  }
  return QS_OK;
}

QS_API int qs_moe_dequant(qs_moe* h, int layer, int expert, int which, float* out, void* hip_stream) {
  if (!h || !out) return QS_E_INVAL;
  const qs_moe_config& c = h->cfg;
  if (which < 0 || which > 5) return QS_E_INVAL;
  if (which < 3 && (expert < 0 || expert >= c.n_experts)) return QS_E_INVAL;
  if (which >= 3 && c.shared_ffn == 0) return QS_E_INVAL;
  int rc = check_layer_range(h, layer, 1);
  if (rc) return rc;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  const LayerDev& L = h->layers[layer];
  const size_t H = c.hidden, F = c.expert_ffn;
  if (which >= 3) {
    const bool sq8 = c.shared_format == QS_FMT_Q8;
    const uint8_t* mat = which == 3 ? L.sg : which == 4 ? L.su : L.sd;
    const size_t rows = which == 5 ? H : (size_t)c.shared_ffn;
    const int K = which == 5 ? c.shared_ffn : c.hidden;
    const size_t total = rows * (size_t)K;
    hipLaunchKernelGGL(k_dequant_shared, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, mat, rows, K,
                       sq8 ? 1 : 0, srow_bytes(K, sq8), out);
    QS_HIP(hipGetLastError());
    return QS_OK;
  }
  const uint8_t* mat;
  size_t nblk;
  int fmt;
  const size_t gs = L.q4k ? h->gu_stride4 : h->gu_stride;
  if (L.host) {   // a paged layer: the expert's host record, read over PCIe
    mat = (const uint8_t*)(uintptr_t)(L.host_dev + (uint64_t)expert * L.rec_bytes) + (size_t)which * gs;
  } else {
    mat = which == 0 ? L.gate + (size_t)expert * gs
                     : which == 1 ? L.up + (size_t)expert * gs
                                  : L.down + (size_t)expert * (L.q4k ? h->dn_stride4 : h->dn_stride);
  }
  if (which < 2) {
    nblk = F * (H / kBlockW);
    fmt = L.q4k ? kFmtQ4K : c.gate_up_format;
  } else {
    nblk = H * (F / kBlockW);
    fmt = L.q4k ? kFmtQ4K : kFmtQ2K;
  }
  const dim3 grid((unsigned)((nblk + 255) / 256));
  if (fmt == kFmtCB2)
    hipLaunchKernelGGL(k_dequant_cb2, grid, dim3(256), 0, st, mat, (const uint32_t*)h->cbtab, nblk, out);
  else if (fmt == kFmtQ4K)
    hipLaunchKernelGGL(k_dequant_q4k, grid, dim3(256), 0, st, mat, nblk, out);
  else
    hipLaunchKernelGGL(k_dequant_q2k, grid, dim3(256), 0, st, mat, nblk, out);
  QS_HIP(hipGetLastError());
  return QS_OK;
}

QS_API int qs_moe_cache_sync(qs_moe* h, void* hip_stream) {
  if (!h) return QS_E_INVAL;
  if (!h->n_paged) return QS_E_STATE;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  hipStream_t st = (hipStream_t)hip_stream;
  QS_HIP(hipStreamSynchronize(st));
  const int rc = cache_poll(h, st, true);
  if (rc) return rc;
  QS_HIP(hipStreamSynchronize(st));
  return QS_OK;
}

QS_API int qs_moe_cache_preload(qs_moe* h, const int32_t* keys, int n, void* hip_stream) {
  if (!h || n < 0 || (n && !keys)) return QS_E_INVAL;
  if (!h->n_paged) return QS_E_STATE;
  const qs_moe_config& c = h->cfg;
  for (int i = 0; i < n; ++i)
    if (keys[2 * i] < c.resident_layers || keys[2 * i] >= c.n_layers || keys[2 * i + 1] < 0 ||
        keys[2 * i + 1] >= c.n_experts)
      return QS_E_INVAL;
  int rc = qs_moe_cache_sync(h, hip_stream);
  if (rc) return rc;
  DeviceGuard dg(h->device);
  if (!dg.ok) return QS_E_HIP;
  // hottest first into the free slots; each later (colder) one goes to the
  // least-recent end, so the coldest preloaded expert is evicted first
  for (int i = 0; i < n && !h->free_slots.empty(); ++i) {
    const int key = (keys[2 * i] - c.resident_layers) * c.n_experts + keys[2 * i + 1];
    if (h->slot_of[key] >= 0) continue;
    const int v = *h->free_slots.begin();
    h->free_slots.erase(h->free_slots.begin());
    slot_take(h, v, key);
    lru_push_front(h, v);
    ++h->c_preloaded;
  }
  hipStream_t st = (hipStream_t)hip_stream;
  rc = cache_flush(h, st);
  if (rc) return rc;
  QS_HIP(hipStreamSynchronize(st));
  return QS_OK;
}

QS_API int qs_moe_cache_stats(qs_moe* h, uint64_t* out) {
  if (!h || !out) return QS_E_INVAL;
  if (!h->n_paged) return QS_E_STATE;
  const uint64_t S = (uint64_t)h->cfg.cache_slots;
  const uint64_t v[8] = {h->c_hits, h->c_misses, h->c_admits, h->c_evicts, h->c_preloaded,
                         S - (uint64_t)h->free_slots.size(), S, h->host_bytes};
  memcpy(out, v, sizeof(v));
  return QS_OK;
}

QS_API int qs_moe_cache_slots(qs_moe* h, int32_t* out) {
  if (!h || !out) return QS_E_INVAL;
  if (!h->n_paged) return QS_E_STATE;
  const int E = h->cfg.n_experts;
  for (int v = 0; v < h->cfg.cache_slots; ++v) {
    const int key = h->owner[v];
    out[2 * v] = key < 0 ? -1 : h->cfg.resident_layers + key / E;
    out[2 * v + 1] = key < 0 ? -1 : key % E;
  }
  return QS_OK;
}

QS_API int qs_moe_memory_bytes(const qs_moe* h, uint64_t* bytes) {
  if (!h || !bytes) return QS_E_INVAL;
  *bytes = h->total_bytes;
  return QS_OK;
}

QS_API int qs_moe_destroy(qs_moe* h) {
  if (!h) return QS_OK;
  int rc = QS_OK;
  {
    DeviceGuard dg(h->device);
    if (hipDeviceSynchronize() != hipSuccess) rc = QS_E_HIP;
    free_all(h);
  }
  delete h;
  return rc;
}

#ifdef QS_STAMPS
// Profiling builds only: copy the phase stamps to host memory.
QS_API int qs_debug_read_stamps(void* host_dst, size_t bytes) {
  if (bytes > sizeof(g_qs_stamps)) bytes = sizeof(g_qs_stamps);
  return hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_qs_stamps), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess
             ? QS_OK
             : QS_E_HIP;
}
#endif

}  // extern "C"
