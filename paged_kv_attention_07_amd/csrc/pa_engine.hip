// Multi-step driver: scheduler + kernels in one native call per step (the
// sequence and its sources are documented in include/pa_engine.h).  Host
// code only; every kernel is launched through the library's own C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "pa.h"
#include "pa_engine.h"
#include "pa_sched.h"

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ArenaLayout {
  // int32 offsets of [qsl S+1 | num_computed S | seq_lens S | copies 2S | table S x W]
  int32_t S, W, qsl, nc, sl, cp, bt;
  size_t size;  // int32 elements
  ArenaLayout(int32_t seqs, int32_t width)
      : S(seqs), W(width), qsl(0), nc(seqs + 1), sl(2 * seqs + 1), cp(3 * seqs + 1),
        bt(5 * seqs + 1), size((size_t)bt + (size_t)seqs * width) {}
  size_t used(int32_t num_seqs) const { return (size_t)bt + (size_t)num_seqs * W; }
};

struct DeviceLayout {
  size_t arena, slots, workspace, total;
};

bool config_ok(const pa_sched_config* c, const pa_engine_geometry* g) {
  return c && g && c->block_size == 16 && c->num_blocks > 0 && c->max_num_seqs > 0 &&
         c->max_num_batched_tokens > 0 && c->max_model_len > 0 && g->num_kv_heads > 0 &&
         g->num_q_heads > 0 && g->scale > 0.f;
}

DeviceLayout device_layout(const pa_sched_config* c, const pa_engine_geometry* g,
                           const ArenaLayout& a) {
  DeviceLayout d;
  d.arena = 0;
  d.slots = align256(a.size * sizeof(int32_t));
  d.workspace = d.slots + align256((size_t)c->max_num_batched_tokens * sizeof(int64_t));
  const size_t ws = pa_attention_workspace_size(
      c->max_num_seqs, c->max_num_batched_tokens, g->num_q_heads, g->num_kv_heads, g->head_dim,
      c->max_model_len, c->max_num_batched_tokens, g->num_splits);
  d.total = ws ? d.workspace + ws : 0;
  return d;
}

int32_t table_width(const pa_sched_config* c) { return (c->max_model_len + 15) / 16; }

}  // namespace

struct pa_engine {
  pa_sched_config cfg;
  pa_engine_geometry geo;
  pa_sched* sched = nullptr;
  ArenaLayout layout;
  DeviceLayout dlay;
  uint8_t* kv = nullptr;
  uint8_t* scratch = nullptr;
  size_t ws_bytes = 0;
  int32_t* host[2] = {nullptr, nullptr};     // page-locked arenas
  int64_t* ids[2] = {nullptr, nullptr};
  int64_t* pre[2] = {nullptr, nullptr};
  int32_t* toks[2] = {nullptr, nullptr};
  hipEvent_t copied[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int next = 0;
  explicit pa_engine(const pa_sched_config& c) : layout(c.max_num_seqs, table_width(&c)) {}
};

extern "C" {

size_t pa_engine_device_bytes(const pa_sched_config* config, const pa_engine_geometry* geometry) {
  if (!config_ok(config, geometry)) return 0;
  const ArenaLayout a(config->max_num_seqs, table_width(config));
  return device_layout(config, geometry, a).total;
}

void pa_engine_destroy(pa_engine* e) {
  if (!e) return;
  for (int i = 0; i < 2; ++i) {
    if (e->copied[i]) {
      (void)hipEventSynchronize(e->copied[i]);
      (void)hipEventDestroy(e->copied[i]);
    }
    if (e->host[i]) (void)hipHostFree(e->host[i]);
    delete[] e->ids[i];
    delete[] e->pre[i];
    delete[] e->toks[i];
  }
  pa_sched_destroy(e->sched);
  delete e;
}

int pa_engine_create(const pa_sched_config* config, const pa_engine_geometry* geometry,
                     void* kv_cache, void* device_scratch, size_t device_scratch_bytes,
                     pa_engine** out) {
  if (!out || !kv_cache || !device_scratch || !config_ok(config, geometry))
    return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(device_scratch) & 255u) != 0) return PA_ERR_INVALID_ARG;
  const size_t need = pa_engine_device_bytes(config, geometry);
  if (need == 0) return PA_ERR_UNSUPPORTED;
  if (device_scratch_bytes < need) return PA_ERR_WORKSPACE;
  pa_engine* e = new pa_engine(*config);
  e->cfg = *config;
  e->geo = *geometry;
  e->kv = static_cast<uint8_t*>(kv_cache);
  e->scratch = static_cast<uint8_t*>(device_scratch);
  e->dlay = device_layout(config, geometry, e->layout);
  e->ws_bytes = need - e->dlay.workspace;
  int st = pa_sched_create(config, &e->sched);
  if (st != PA_OK) {
    pa_engine_destroy(e);
    return st;
  }
  for (int i = 0; i < 2; ++i) {
    if (hipHostMalloc(reinterpret_cast<void**>(&e->host[i]), e->layout.size * sizeof(int32_t),
                      hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&e->copied[i], hipEventDisableTiming) != hipSuccess) {
      pa_engine_destroy(e);
      return PA_ERR_HIP;
    }
    e->ids[i] = new int64_t[config->max_num_seqs];
    e->pre[i] = new int64_t[config->max_num_seqs];
    e->toks[i] = new int32_t[config->max_num_batched_tokens];
  }
  *out = e;
  return PA_OK;
}

pa_sched* pa_engine_scheduler(pa_engine* e) { return e ? e->sched : nullptr; }

int pa_engine_step(pa_engine* e, const void* q, const void* k, const void* v, void* out,
                   void* stream, pa_sched_step* step) {
  if (!e || !q || !k || !v || !out || !step) return PA_ERR_INVALID_ARG;
  const int b = e->next;
  // the arena set is rewritten only after its previous copy has completed
  if (e->pending[b]) {
    if (hipEventSynchronize(e->copied[b]) != hipSuccess) return PA_ERR_HIP;
    e->pending[b] = false;
  }
  const ArenaLayout& L = e->layout;
  int32_t* h = e->host[b];
  pa_sched_step s;
  memset(&s, 0, sizeof(s));
  s.request_ids = e->ids[b];
  s.query_start_loc = h + L.qsl;
  s.num_computed = h + L.nc;
  s.seq_lens = h + L.sl;
  s.block_table = h + L.bt;
  s.token_ids = e->toks[b];
  s.copy_pairs = h + L.cp;
  s.preempted_ids = e->pre[b];
  s.block_table_stride = L.W;
  int st = pa_sched_schedule(e->sched, &s);
  if (st != PA_OK) return st;
  *step = s;
  e->next = b ^ 1;
  if (s.num_seqs == 0) return PA_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* d = reinterpret_cast<int32_t*>(e->scratch + e->dlay.arena);
  if (hipMemcpyAsync(d, h, L.used(s.num_seqs) * sizeof(int32_t), hipMemcpyHostToDevice, hs) !=
          hipSuccess ||
      hipEventRecord(e->copied[b], hs) != hipSuccess)
    return PA_ERR_HIP;
  e->pending[b] = true;

  const pa_engine_geometry& g = e->geo;
  const int32_t B = e->cfg.block_size;
  const int64_t nb = e->cfg.num_blocks;
  if (s.num_copies > 0) {
    st = pa_copy_blocks(e->kv, d + L.cp, s.num_copies, nb, B, g.num_kv_heads, g.head_dim,
                        g.dtype, stream);
    if (st != PA_OK) return st;
  }
  // slots, K/V store and attention in one launch (+ the split merge)
  int64_t* slots = reinterpret_cast<int64_t*>(e->scratch + e->dlay.slots);
  return pa_cache_and_attend_mixed(out, q, k, v, e->kv, nb, B, g.num_kv_heads, g.head_dim,
                                   g.dtype, d + L.bt, L.W, d + L.sl, d + L.qsl, d + L.nc, slots,
                                   s.num_seqs, s.num_tokens, s.max_query_len, s.max_seq_len,
                                   g.num_q_heads, g.scale, e->scratch + e->dlay.workspace,
                                   e->ws_bytes, g.num_splits, stream);
}

int pa_engine_update(pa_engine* e, const int32_t* sampled, int32_t num_seqs,
                     int64_t* finished_ids, int32_t* num_finished) {
  if (!e) return PA_ERR_INVALID_ARG;
  return pa_sched_update(e->sched, sampled, num_seqs, finished_ids, num_finished);
}

}  // extern "C"
