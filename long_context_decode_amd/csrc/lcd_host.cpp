// Host side of the C ABI declared in include/lcd.h: validation, memory layout,
// per-layer token bookkeeping and kernel launches.  Every check runs before any
// HIP call, so the validation paths work (and are tested) on machines without a
// GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "lcd.h"
#include "lcd_internal.h"

namespace {

thread_local std::string g_err;

lcd_status fail(lcd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lcd_status ok() {
  g_err.clear();
  return LCD_OK;
}

lcd_status hip_fail(hipError_t e, const char* what) {
  return fail(LCD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

// Checked product of non-negative factors; false on overflow.
bool mul_ok(uint64_t* acc, uint64_t f) { return !__builtin_mul_overflow(*acc, f, acc); }

constexpr int64_t kMaxSlots = int64_t(1) << 24;

struct Layout {
  int C = 0, esize = 0, G = 0;
  uint64_t layer_bytes = 0;  // one of K or V of one layer
  uint64_t kv_bytes = 0;
  uint64_t aux_bytes = 0, off_cos = 0, off_sin = 0, off_pos = 0, off_score = 0, off_victim = 0, off_arrive = 0;
  uint64_t off_open = 0;
  uint64_t ws_bytes = 0, ws_off_ml = 0, ws_off_logits = 0;
  int max_splits = 0, chunk_cap = 0;
  // mixed retrieval / streaming heads (DUO): streaming capacity, per-layer retrieval
  // head count, byte offset of each layer's K block and size of its K (= V) block,
  // and the per-layer head map (>= 0 retrieval index, < 0: -1 - streaming index)
  int C2 = 0;
  std::vector<int> duo_hret;
  std::vector<uint64_t> duo_off, duo_bytes;
  std::vector<int16_t> duo_map;
};

lcd_status check_config(const lcd_cache_config* c, Layout* L) {
  if (!c) return fail(LCD_EINVAL, "config is NULL");
  if (c->batch < 1 || c->n_layers < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(LCD_ESHAPE, "batch, n_layers, n_q_heads and n_kv_heads must be >= 1");
  // bounds that keep every row-head count, grid size and index product of the launch
  // planning inside 32-bit integers
  if ((int64_t)c->batch * c->n_q_heads > (int64_t(1) << 24) || c->n_layers > 65536)
    return fail(LCD_ESHAPE, "need batch * n_q_heads <= 2^24 and n_layers <= 65536");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(LCD_ESHAPE, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(LCD_ESHAPE, "head_dim %d not in {64, 128, 256}", c->head_dim);
  if (c->dtype != LCD_F32 && c->dtype != LCD_BF16) return fail(LCD_EINVAL, "unknown dtype %d", c->dtype);
  if (!lcd::decode_supported(c->dtype, c->head_dim, G))
    return fail(LCD_EUNSUPPORTED, "query heads per KV head %d not in {1, 2, 4, 6, 8}", G);
  int64_t C = 0;
  switch (c->policy) {
    case LCD_SINK_RING:
      if (c->n_sink < 0 || c->window < 1) return fail(LCD_ESHAPE, "need n_sink >= 0 and window >= 1");
      C = (int64_t)c->n_sink + c->window;
      break;
    case LCD_APPEND:
    case LCD_H2O:
      if (c->capacity < 1) return fail(LCD_ESHAPE, "capacity must be >= 1");
      C = c->capacity;
      if (c->policy == LCD_H2O && (c->n_recent < 1 || c->n_recent > c->capacity))
        return fail(LCD_ESHAPE, "H2O needs 1 <= n_recent <= capacity");
      if (c->policy == LCD_H2O && c->block_size > 1) {
        if (c->block_size != 16 && c->block_size != 32) return fail(LCD_ESHAPE, "H2O block_size must be 0, 1, 16 or 32");
        if (c->capacity % c->block_size) return fail(LCD_ESHAPE, "capacity must be a multiple of block_size");
        if (c->n_recent > c->capacity - c->block_size)
          return fail(LCD_ESHAPE, "block-level H2O needs n_recent <= capacity - block_size");
      } else if (c->policy == LCD_H2O && c->block_size < 0) {
        return fail(LCD_ESHAPE, "block_size must be >= 0");
      }
      break;
    case LCD_DUO:
      if (c->capacity < 1) return fail(LCD_ESHAPE, "capacity must be >= 1");
      if (c->n_sink < 0 || c->window < 1) return fail(LCD_ESHAPE, "need n_sink >= 0 and window >= 1");
      if (!c->retrieval) return fail(LCD_EINVAL, "DUO needs the retrieval head map");
      if (c->n_kv_heads > lcd::kMaxDuoHeads)
        return fail(LCD_EUNSUPPORTED, "DUO supports up to %d KV heads per layer", lcd::kMaxDuoHeads);
      for (int64_t i = 0; i < (int64_t)c->n_layers * c->n_kv_heads; ++i)
        if (c->retrieval[i] != 0 && c->retrieval[i] != 1) return fail(LCD_EINVAL, "retrieval flags must be 0 or 1");
      C = c->capacity;
      if ((int64_t)c->n_sink + c->window > kMaxSlots) return fail(LCD_ESHAPE, "n_sink + window exceeds the slot limit");
      break;
    default:
      return fail(LCD_EINVAL, "unknown policy %d", c->policy);
  }
  if (C > kMaxSlots) return fail(LCD_ESHAPE, "capacity %lld exceeds %lld slots", (long long)C, (long long)kMaxSlots);
  if (c->rope != 0 && c->rope != 1) return fail(LCD_EINVAL, "rope must be 0 or 1");
  if (c->rope == 1 && c->policy != LCD_SINK_RING)
    return fail(LCD_EUNSUPPORTED, "rotation at in-cache positions is defined for the sink + window cache only");
  const bool duo = c->policy == LCD_DUO;
  if (c->rope == 1 && !(std::isfinite(c->rope_base) && c->rope_base > 1.0))
    return fail(LCD_EINVAL, "rope_base must be finite and > 1");
  if (c->rope == 1 && std::max<int64_t>(C, 65) * c->head_dim >= (int64_t(1) << 31))
    return fail(LCD_ESHAPE, "a rotated cache needs (n_sink + window) * head_dim < 2^31 (position table below 4 GiB)");
  if (!(std::isfinite(c->scale) && c->scale >= 0.0)) return fail(LCD_EINVAL, "scale must be finite and >= 0");

  L->C = (int)C;
  L->esize = c->dtype == LCD_F32 ? 4 : 2;
  L->G = G;
  uint64_t lb = (uint64_t)c->batch;
  if (!mul_ok(&lb, c->n_kv_heads) || !mul_ok(&lb, (uint64_t)C) || !mul_ok(&lb, c->head_dim) ||
      !mul_ok(&lb, L->esize))
    return fail(LCD_ESIZE, "cache size overflows 64 bits");
  uint64_t kv = lb;
  if (!mul_ok(&kv, 2) || !mul_ok(&kv, c->n_layers)) return fail(LCD_ESIZE, "cache size overflows 64 bits");
  L->layer_bytes = lb;
  L->kv_bytes = kv;
  if (duo) {
    // per layer: K = [B][R_l][C][D] then [B][T_l][S + W][D]; V the same; layers in order
    L->C2 = c->n_sink + c->window;
    L->duo_hret.assign(c->n_layers, 0);
    L->duo_off.assign(c->n_layers, 0);
    L->duo_bytes.assign(c->n_layers, 0);
    L->duo_map.assign((size_t)c->n_layers * c->n_kv_heads, 0);
    const uint64_t row = (uint64_t)c->head_dim * L->esize;
    uint64_t off = 0;
    for (int l = 0; l < c->n_layers; ++l) {
      int r = 0, t = 0;
      for (int g = 0; g < c->n_kv_heads; ++g) {
        const bool ret = c->retrieval[(size_t)l * c->n_kv_heads + g] != 0;
        L->duo_map[(size_t)l * c->n_kv_heads + g] = (int16_t)(ret ? r++ : -1 - t++);
      }
      L->duo_hret[l] = r;
      // the slot counts fit 2^24 and heads 128, so (r*C + t*C2) < 2^32; times B*row below
      uint64_t blk = (uint64_t)r * C + (uint64_t)t * L->C2;
      if (!mul_ok(&blk, c->batch) || !mul_ok(&blk, row)) return fail(LCD_ESIZE, "cache size overflows 64 bits");
      L->duo_off[l] = off;
      L->duo_bytes[l] = blk;
      if (__builtin_add_overflow(off, 2 * blk, &off)) return fail(LCD_ESIZE, "cache size overflows 64 bits");
    }
    L->kv_bytes = off;
  }

  // arrival counters of the split merge: one per (layer, batch row, KV head)
  uint64_t aux = align256((uint64_t)c->n_layers * c->batch * c->n_kv_heads * sizeof(int32_t));
  L->off_arrive = 0;
  if (c->rope == 1) {
    // rows 0 .. max(C, 65) - 1: the decode kernel also reads the row of its per-lane
    // step (at most 64 positions) for angle additions
    const uint64_t tab = (uint64_t)std::max<int64_t>(C, 65) * (c->head_dim / 2) * sizeof(float);
    L->off_cos = aux;
    aux = align256(aux + tab);
    L->off_sin = aux;
    aux = align256(aux + tab);
  }
  if (c->policy == LCD_H2O) {
    const uint64_t per = (uint64_t)c->n_layers * c->batch * c->n_kv_heads * C;
    L->off_pos = aux;
    aux = align256(aux + per * sizeof(int32_t));
    L->off_score = aux;
    aux = align256(aux + per * sizeof(float));
    L->off_victim = aux;
    aux = align256(aux + (uint64_t)c->n_layers * c->batch * c->n_kv_heads * sizeof(int32_t));
    L->off_open = aux;  // block-level: the block receiving new tokens
    aux = align256(aux + (uint64_t)c->n_layers * c->batch * c->n_kv_heads * sizeof(int32_t));
  }
  L->aux_bytes = aux;

  L->chunk_cap = lcd::decode_chunk_cap(G);
  {
    // Bound on the split count of any plan with n <= C: plan_splits never exceeds
    // max(ceil(n / chunk_cap), 4 * target / bg) splits nor ceil(n / 64), all
    // non-decreasing in n.  Mixed heads plan over C or S + W with bg >= batch.
    const int64_t Cp = duo ? std::max<int64_t>(C, L->C2) : C;
    const int64_t bg = duo ? (int64_t)c->batch : (int64_t)c->batch * c->n_kv_heads;
    const int64_t by_min = (Cp + 63) / 64;
    const int64_t s_cap = (Cp + L->chunk_cap - 1) / L->chunk_cap;
    L->max_splits = (int)std::min<int64_t>(by_min, std::max<int64_t>(s_cap, 4 * (int64_t)lcd::kResidentWorkgroups / bg));
  }
  const int smax = L->max_splits;

  const uint64_t bhq = (uint64_t)c->batch * c->n_q_heads;
  uint64_t ws = align256((uint64_t)smax * bhq * c->head_dim * sizeof(float));
  L->ws_off_ml = ws;
  ws = align256(ws + (uint64_t)smax * bhq * 2 * sizeof(float));
  L->ws_off_logits = ws;
  if (c->policy == LCD_H2O) ws = align256(ws + bhq * (uint64_t)C * sizeof(float));
  L->ws_bytes = ws;
  return LCD_OK;
}

// Split plan for n attended slots of bg (row, KV head) pairs.  Cost model: workgroups
// run in rounds of kResidentWorkgroups, each as long as its chunk, so a plan costs
// rounds * chunk.  Candidates are the most splits that fit r rounds, r = 1..4, raised to
// the fewest the chunk cap allows and capped at ceil(n / 64); the cheapest wins, ties
// going to fewer splits.
void plan_splits(const Layout& L, int n, int bg, int* n_splits, int* chunk) {
  const int64_t target = lcd::kResidentWorkgroups;
  const int64_t by_min = (n + 63) / 64;
  const int64_t s_cap = (n + L.chunk_cap - 1) / L.chunk_cap;
  int64_t best_ch = 0, best_cost = -1;
  for (int64_t r = 1; r <= 4; ++r) {
    const int64_t sp = std::min<int64_t>(by_min, std::max<int64_t>(s_cap, r * target / bg));
    const int64_t c = ((n + sp - 1) / sp + 63) / 64 * 64;
    if (c > L.chunk_cap) continue;
    const int64_t wgs = (n + c - 1) / c * (int64_t)bg;
    const int64_t cost = (wgs + target - 1) / target * c;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && c > best_ch)) {
      best_cost = cost;
      best_ch = c;
    }
  }
  *chunk = (int)best_ch;
  *n_splits = (n + *chunk - 1) / *chunk;
}

}  // namespace

struct lcd_cache {
  lcd_cache_config cfg;
  Layout L;
  char* kv = nullptr;
  char* aux = nullptr;
  std::vector<int64_t> tokens;  // tokens appended per layer
  std::vector<int64_t> filled;  // slots holding a token per layer
  float qscale = 0.f;

  char* k_layer(int l) const {
    return cfg.policy == LCD_DUO ? kv + L.duo_off[l] : kv + (uint64_t)l * 2 * L.layer_bytes;
  }
  char* v_layer(int l) const { return k_layer(l) + (cfg.policy == LCD_DUO ? L.duo_bytes[l] : L.layer_bytes); }
  // DUO: start of the streaming heads inside a layer's K (or V) block
  uint64_t duo_str_off(int l) const {
    return (uint64_t)cfg.batch * L.duo_hret[l] * L.C * cfg.head_dim * L.esize;
  }
  float* cos_t() const { return cfg.rope ? reinterpret_cast<float*>(aux + L.off_cos) : nullptr; }
  float* sin_t() const { return cfg.rope ? reinterpret_cast<float*>(aux + L.off_sin) : nullptr; }
  uint64_t per_layer_slots() const { return (uint64_t)cfg.batch * cfg.n_kv_heads * L.C; }
  int32_t* pos(int l) const {
    return cfg.policy == LCD_H2O ? reinterpret_cast<int32_t*>(aux + L.off_pos) + l * per_layer_slots() : nullptr;
  }
  float* score(int l) const {
    return cfg.policy == LCD_H2O ? reinterpret_cast<float*>(aux + L.off_score) + l * per_layer_slots() : nullptr;
  }
  int32_t* arrivals(int l) const {
    return reinterpret_cast<int32_t*>(aux + L.off_arrive) + (uint64_t)l * cfg.batch * cfg.n_kv_heads;
  }
  int32_t* victim(int l) const {
    return cfg.policy == LCD_H2O
               ? reinterpret_cast<int32_t*>(aux + L.off_victim) + (uint64_t)l * cfg.batch * cfg.n_kv_heads
               : nullptr;
  }
  int32_t* open_block(int l) const {
    return cfg.policy == LCD_H2O
               ? reinterpret_cast<int32_t*>(aux + L.off_open) + (uint64_t)l * cfg.batch * cfg.n_kv_heads
               : nullptr;
  }
  // H2O eviction granule (1 = token) and, per layer, slots used in the open block
  int bs() const { return cfg.policy == LCD_H2O && cfg.block_size > 1 ? cfg.block_size : 1; }
  std::vector<int> open_fill;
};

namespace {

lcd_status check_layer(const lcd_cache* c, int32_t layer) {
  if (!c) return fail(LCD_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers)
    return fail(LCD_EINVAL, "layer %d out of range [0, %d)", layer, c->cfg.n_layers);
  return LCD_OK;
}

}  // namespace

extern "C" {

int lcd_abi_version(void) { return LCD_ABI_VERSION; }

const char* lcd_last_error(void) { return g_err.c_str(); }

lcd_status lcd_cache_sizes(const lcd_cache_config* cfg, uint64_t* kv_bytes, uint64_t* aux_bytes,
                           uint64_t* ws_bytes) {
  Layout L;
  const lcd_status st = check_config(cfg, &L);
  if (st) return st;
  if (kv_bytes) *kv_bytes = L.kv_bytes;
  if (aux_bytes) *aux_bytes = L.aux_bytes;
  if (ws_bytes) *ws_bytes = L.ws_bytes;
  return ok();
}

lcd_status lcd_kv_cache_init(const lcd_cache_config* cfg, void* kv_mem, uint64_t kv_bytes, void* aux_mem,
                             uint64_t aux_bytes, void* stream, lcd_cache** out) {
  if (!out) return fail(LCD_EINVAL, "out is NULL");
  Layout L;
  const lcd_status st = check_config(cfg, &L);
  if (st) return st;
  if (!kv_mem) return fail(LCD_EINVAL, "kv_mem is NULL");
  if (!aligned16(kv_mem)) return fail(LCD_EALIGN, "kv_mem is not 16-byte aligned");
  if (kv_bytes < L.kv_bytes)
    return fail(LCD_ESIZE, "kv_bytes %llu < required %llu", (unsigned long long)kv_bytes,
                (unsigned long long)L.kv_bytes);
  if (!aux_mem) return fail(LCD_EINVAL, "aux_mem is NULL but %llu bytes are required",
                            (unsigned long long)L.aux_bytes);
  if (!aligned16(aux_mem)) return fail(LCD_EALIGN, "aux_mem is not 16-byte aligned");
  if (aux_bytes < L.aux_bytes)
    return fail(LCD_ESIZE, "aux_bytes %llu < required %llu", (unsigned long long)aux_bytes,
                (unsigned long long)L.aux_bytes);
  lcd_cache* c = new (std::nothrow) lcd_cache();
  if (!c) return fail(LCD_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->cfg.retrieval = nullptr;  // the head map lives in the layout (caller memory is read once)
  c->L = L;
  c->kv = static_cast<char*>(kv_mem);
  c->aux = static_cast<char*>(aux_mem);
  c->tokens.assign(cfg->n_layers, 0);
  c->filled.assign(cfg->n_layers, 0);
  c->open_fill.assign(cfg->n_layers, 0);
  const double scale = cfg->scale > 0 ? cfg->scale : 1.0 / std::sqrt((double)cfg->head_dim);
  c->qscale = (float)(scale * 1.4426950408889634074);  // scale * log2(e), rounded once
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = lcd::launch_fill_i32(c->arrivals(0), 0, (int64_t)cfg->n_layers * cfg->batch * cfg->n_kv_heads, s);
  if (e == hipSuccess && cfg->rope)
    e = lcd::launch_rope_table(c->cos_t(), c->sin_t(), std::max(L.C, 65), cfg->head_dim, cfg->rope_base, s);
  if (e == hipSuccess && cfg->policy == LCD_H2O) {
    const int64_t n = (int64_t)cfg->n_layers * c->per_layer_slots();
    e = lcd::launch_fill_i32(c->pos(0), -1, n, s);
    if (e == hipSuccess) e = lcd::launch_fill_f32(c->score(0), 0.f, n, s);
    if (e == hipSuccess) e = lcd::launch_fill_i32(c->victim(0), 0, (int64_t)cfg->n_layers * cfg->batch * cfg->n_kv_heads, s);
    if (e == hipSuccess) e = lcd::launch_fill_i32(c->open_block(0), 0, (int64_t)cfg->n_layers * cfg->batch * cfg->n_kv_heads, s);
  }
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "kv_cache_init launch");
  }
  *out = c;
  return ok();
}

void lcd_kv_cache_destroy(lcd_cache* cache) { delete cache; }

lcd_status lcd_kv_append(lcd_cache* c, int32_t layer, const void* k, const void* v, int32_t n_new, void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (!k || !v) return fail(LCD_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(LCD_EALIGN, "k or v is not 16-byte aligned");
  if (n_new < 1) return fail(LCD_EINVAL, "n_new must be >= 1");
  const lcd_cache_config& cfg = c->cfg;
  const int C = c->L.C;
  const int64_t t0 = c->tokens[layer];
  lcd::AppendParams p{};
  p.k_in = static_cast<const char*>(k);
  p.v_in = static_cast<const char*>(v);
  p.k_cache = c->k_layer(layer);
  p.v_cache = c->v_layer(layer);
  p.BHkv = cfg.batch * cfg.n_kv_heads;
  p.C = C;
  p.n_new = n_new;
  p.row_bytes = cfg.head_dim * c->L.esize;
  p.S = cfg.n_sink;
  p.W = cfg.window > 0 ? cfg.window : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t new_filled = c->filled[layer];
  if (cfg.policy == LCD_SINK_RING) {
    const int64_t S = cfg.n_sink, W = cfg.window;
    const int64_t t_end = t0 + n_new - 1;
    // sinks among the new tokens
    const int64_t sink_end = std::min<int64_t>(S, t0 + n_new);
    const int64_t n_sink_rows = sink_end > t0 ? sink_end - t0 : 0;
    // newest W tokens that are not sinks
    const int64_t a_first = std::max<int64_t>({S, t_end - W + 1, t0});
    const int64_t n_ring_rows = t_end >= a_first ? t_end - a_first + 1 : 0;
    hipError_t e = hipSuccess;
    if (n_sink_rows > 0) {
      lcd::AppendParams q = p;
      q.r0 = 0;
      q.n_rows = (int)n_sink_rows;
      q.r_split = (int)n_sink_rows;
      q.slot_lin = (int)t0;
      e = lcd::launch_append(q, s);
    }
    if (e == hipSuccess && n_ring_rows > 0) {
      lcd::AppendParams q = p;
      q.r0 = (int)(a_first - t0);
      q.n_rows = (int)n_ring_rows;
      q.r_split = q.r0;
      q.ring_off = (int)((a_first - S) % W);
      e = lcd::launch_append(q, s);
    }
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    new_filled = std::min<int64_t>(t0 + n_new, C);
  } else if (cfg.policy == LCD_APPEND) {
    if (c->filled[layer] + n_new > C)
      return fail(LCD_ECAPACITY, "append of %d rows to %lld filled of capacity %d", n_new,
                  (long long)c->filled[layer], C);
    p.r0 = 0;
    p.n_rows = n_new;
    p.r_split = n_new;
    p.slot_lin = (int)c->filled[layer];
    const hipError_t e = lcd::launch_append(p, s);
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    new_filled = c->filled[layer] + n_new;
  } else if (cfg.policy == LCD_DUO) {
    if (c->filled[layer] + n_new > C)
      return fail(LCD_ECAPACITY, "append of %d rows to %lld filled retrieval slots of capacity %d", n_new,
                  (long long)c->filled[layer], C);
    const int64_t S = cfg.n_sink, W = cfg.window;
    p.duo = 1;
    p.Hkv = cfg.n_kv_heads;
    p.Hret = c->L.duo_hret[layer];
    p.Hstr = cfg.n_kv_heads - p.Hret;
    p.C2 = c->L.C2;
    p.t0 = t0;
    p.a_first = std::max<int64_t>(S, t0 + n_new - W);  // oldest token of the final window
    p.k2_cache = p.k_cache + c->duo_str_off(layer);
    p.v2_cache = p.v_cache + c->duo_str_off(layer);
    for (int g = 0; g < cfg.n_kv_heads; ++g) p.duo_map[g] = c->L.duo_map[(size_t)layer * cfg.n_kv_heads + g];
    const hipError_t e = lcd::launch_append(p, s);
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    new_filled = c->filled[layer] + n_new;
  } else {  // H2O
    if (n_new != 1) return fail(LCD_EINVAL, "H2O appends one token per call (got %d)", n_new);
    if (t0 > INT32_MAX) return fail(LCD_ECAPACITY, "H2O token positions are int32");
    p.h2o = 1;
    p.fill = (int)c->filled[layer];
    p.victim = c->victim(layer);
    p.pos = c->pos(layer);
    p.score = c->score(layer);
    p.token = t0;
    const int bs = c->bs();
    p.bs = bs;
    p.open = c->open_block(layer);
    int next_fill = 0;  // slots used in the open block after this append
    if (p.fill < C) {
      next_fill = (p.fill % bs) + 1;
    } else if (c->open_fill[layer] >= bs) {  // a full cache needs a new block: the victim
      p.new_block = 1;
      next_fill = 1;
    } else {
      p.offset = c->open_fill[layer];
      next_fill = c->open_fill[layer] + 1;
    }
    const hipError_t e = lcd::launch_append(p, s);
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    new_filled = std::min<int64_t>(c->filled[layer] + 1, C);
    c->open_fill[layer] = next_fill;
  }
  c->tokens[layer] = t0 + n_new;
  c->filled[layer] = new_filled;
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by lcd_decode_attn and lcd_decode_step.
lcd_status check_decode_args(const lcd_cache* c, const void* q, const float* out, const void* ws,
                             uint64_t ws_bytes) {
  if (!q || !out || !ws) return fail(LCD_EINVAL, "q, out or ws is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return fail(LCD_EALIGN, "q, out or ws not 16-byte aligned");
  if (ws_bytes < c->L.ws_bytes)
    return fail(LCD_ESIZE, "ws_bytes %llu < required %llu", (unsigned long long)ws_bytes,
                (unsigned long long)c->L.ws_bytes);
  return LCD_OK;
}

// One decode launch over the layer's current state; with new_slot >= 0 the kernel also
// writes the token's rows k_new / v_new into that slot (fused append).
// H2O fused append: the new token's slot is chosen on the device unless the cache is
// still filling (new_slot >= 0); new_block / offset as in the H2O append.
struct FusedH2o {
  int on = 0, new_block = 0, offset = 0;
};

lcd_status launch_decode(lcd_cache* c, int32_t layer, const void* q, float* out, void* ws, void* stream,
                         const void* k_new, const void* v_new, int new_slot, FusedH2o h2o = FusedH2o()) {
  const lcd_cache_config& cfg = c->cfg;
  const Layout& L = c->L;
  const int n = (int)c->filled[layer];
  lcd::DecodeParams p{};
  p.k = c->k_layer(layer);
  p.v = c->v_layer(layer);
  p.q = q;
  p.cos_t = c->cos_t();
  p.sin_t = c->sin_t();
  char* w = static_cast<char*>(ws);
  p.part_o = reinterpret_cast<float*>(w);
  p.part_ml = reinterpret_cast<float*>(w + L.ws_off_ml);
  p.logits = cfg.policy == LCD_H2O ? reinterpret_cast<float*>(w + L.ws_off_logits) : nullptr;
  p.B = cfg.batch;
  p.Hq = cfg.n_q_heads;
  p.Hkv = cfg.n_kv_heads;
  p.C = L.C;
  p.n = n;
  if (cfg.policy == LCD_DUO) {
    // retrieval heads attend the n appended rows, streaming heads min(tokens, S + W);
    // the plan follows the retrieval heads (the bulk of the bytes) unless there are none
    p.duo = 1;
    p.Hret = L.duo_hret[layer];
    p.Hstr = cfg.n_kv_heads - p.Hret;
    p.C2 = L.C2;
    p.n2 = (int)std::min<int64_t>(c->tokens[layer], L.C2);
    p.k2 = c->k_layer(layer) + c->duo_str_off(layer);
    p.v2 = c->v_layer(layer) + c->duo_str_off(layer);
    for (int g = 0; g < cfg.n_kv_heads; ++g) {
      const int m = L.duo_map[(size_t)layer * cfg.n_kv_heads + g];
      p.duo_map[g] = (int16_t)m;
      if (m >= 0)
        p.duo_ret[m] = (int16_t)g;
      else
        p.duo_str[-1 - m] = (int16_t)g;
    }
    const int n_plan = p.Hret > 0 ? n : p.n2;
    plan_splits(L, n_plan, cfg.batch * (p.Hret > 0 ? p.Hret : cfg.n_kv_heads), &p.n_splits, &p.chunk);
    p.ret_splits = p.Hret > 0 ? (n + p.chunk - 1) / p.chunk : 0;
    p.str_splits = p.Hstr > 0 ? (p.n2 + p.chunk - 1) / p.chunk : 0;
    p.n_splits = std::max(p.ret_splits, p.str_splits);
  } else {
    plan_splits(L, n, cfg.batch * cfg.n_kv_heads, &p.n_splits, &p.chunk);
  }
  if (p.n_splits < 1 || p.n_splits > L.max_splits || p.chunk < 64 || p.chunk > L.chunk_cap)
    return fail(LCD_ESIZE, "split plan %d x %d outside the workspace bound %d", p.n_splits, p.chunk,
                L.max_splits);
  p.qscale = c->qscale;
  int mode = lcd::kModePlain;
  if (cfg.rope) {
    mode = lcd::kModeRope;
    const int64_t t = c->tokens[layer] - 1;
    p.S = cfg.n_sink;
    p.W = cfg.window;
    p.full = (t + 1 > L.C) ? 1 : 0;
    p.ring_head = p.full ? (int)((t - cfg.window + 1 - cfg.n_sink) % cfg.window) : 0;
    p.q_rank = n - 1;
  } else if (cfg.policy == LCD_H2O) {
    mode = c->bs() > 1 ? lcd::kModeMaskedLogits : lcd::kModePlainLogits;
  }
  p.out = out;
  p.arrivals = c->arrivals(layer);
  p.k_new = k_new;
  p.v_new = v_new;
  p.new_slot = new_slot;
  p.h2o_step = h2o.on;
  p.new_block = h2o.new_block;
  p.offset = h2o.offset;
  p.open = c->open_block(layer);
  p.token = c->tokens[layer] - 1;  // the appended token (the state is the one after the append)
  if (cfg.policy == LCD_H2O) {
    p.score = c->score(layer);
    p.pos = c->pos(layer);
    p.victim = c->victim(layer);
    // a victim is needed iff the next append finds the cache full and (blocks) the open
    // block full
    p.bs = c->bs();
    p.pick_victim = n == L.C && c->open_fill[layer] >= p.bs ? 1 : 0;
    p.max_pos = c->tokens[layer] - cfg.n_recent;  // next token id minus the protected count
    p.mask_pos = p.bs > 1 ? c->pos(layer) : nullptr;  // emptied slots of a reopened block
  }
  const hipError_t e =
      lcd::launch_decode_split(cfg.dtype, cfg.head_dim, L.G, mode, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

// lcd_decode_step and lcd_decode_step_noalloc: one token appended and attended in one launch.
lcd_status decode_step_impl(lcd_cache* c, int32_t layer, const void* k, const void* v, const void* q, float* out,
                            void* ws, uint64_t ws_bytes, void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (c->cfg.policy == LCD_DUO)
    return fail(LCD_EUNSUPPORTED, "decode_step is defined for the SINK_RING, APPEND and H2O caches");
  if (!k || !v) return fail(LCD_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(LCD_EALIGN, "k or v is not 16-byte aligned");
  if ((st = check_decode_args(c, q, out, ws, ws_bytes))) return st;
  const int64_t t = c->tokens[layer];
  const int C = c->L.C;
  int slot = -1;
  int64_t filled;
  FusedH2o h2o;
  int open_fill = c->open_fill[layer];
  if (c->cfg.policy == LCD_SINK_RING) {
    const int64_t S = c->cfg.n_sink, W = c->cfg.window;
    slot = (int)(t < S ? t : S + (t - S) % W);
    filled = std::min<int64_t>(t + 1, C);
  } else if (c->cfg.policy == LCD_APPEND) {
    if (c->filled[layer] + 1 > C)
      return fail(LCD_ECAPACITY, "append of 1 row to %lld filled of capacity %d", (long long)c->filled[layer], C);
    slot = (int)c->filled[layer];
    filled = c->filled[layer] + 1;
  } else {  // H2O: as lcd_kv_append, the slot of a full cache chosen on the device
    if (t > INT32_MAX) return fail(LCD_ECAPACITY, "H2O token positions are int32");
    const int bs = c->bs(), fill = (int)c->filled[layer];
    h2o.on = 1;
    if (fill < C) {
      slot = fill;
      open_fill = (fill % bs) + 1;
    } else if (open_fill >= bs) {  // a full cache needs a new block: the victim
      h2o.new_block = bs > 1 ? 1 : 0;
      open_fill = 1;
    } else {
      h2o.offset = open_fill;
      open_fill = open_fill + 1;
    }
    filled = std::min<int64_t>(fill + 1, C);
  }
  // the launch sees the state after the append
  const int64_t t_prev = c->tokens[layer], f_prev = c->filled[layer];
  const int o_prev = c->open_fill[layer];
  c->tokens[layer] = t + 1;
  c->filled[layer] = filled;
  c->open_fill[layer] = open_fill;
  st = launch_decode(c, layer, q, out, ws, stream, k, v, slot, h2o);
  if (st) {  // nothing was enqueued: keep the bookkeeping as it was
    c->tokens[layer] = t_prev;
    c->filled[layer] = f_prev;
    c->open_fill[layer] = o_prev;
  }
  return st;
}

// ---------------------------------------------------------------- device scratch
// The split partials of lcd_decode_step_noalloc live in a file-scope device array of
// scratch.hip (one copy per GPU); its device address comes from there.
lcd_status scratch_address(void** out) {
  const hipError_t e = lcd::scratch_device_address(out);
  if (e == hipErrorInvalidDevice) return fail(LCD_EUNSUPPORTED, "current device beyond the scratch table");
  if (e != hipSuccess) return hip_fail(e, "device scratch address");
  return LCD_OK;
}

}  // namespace

extern "C" {

lcd_status lcd_decode_attn(lcd_cache* c, int32_t layer, const void* q, float* out, void* ws, uint64_t ws_bytes,
                           void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if ((st = check_decode_args(c, q, out, ws, ws_bytes))) return st;
  if (c->tokens[layer] < 1 || c->filled[layer] < 1) return fail(LCD_EINVAL, "layer %d holds no token", layer);
  return launch_decode(c, layer, q, out, ws, stream, nullptr, nullptr, -1);
}

lcd_status lcd_decode_step(lcd_cache* c, int32_t layer, const void* k, const void* v, const void* q, float* out,
                           void* ws, uint64_t ws_bytes, void* stream) {
  return decode_step_impl(c, layer, k, v, q, out, ws, ws_bytes, stream);
}

lcd_status lcd_decode_step_noalloc(lcd_cache* c, int32_t layer, const void* k, const void* v, const void* q,
                                   float* out, void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (c->L.ws_bytes > lcd::kScratchBytes)
    return fail(LCD_ESIZE, "decode_step_noalloc: this cache needs %llu workspace bytes, above the %llu-byte "
                "device scratch buffer (use lcd_decode_step with a caller workspace)",
                (unsigned long long)c->L.ws_bytes, (unsigned long long)lcd::kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return decode_step_impl(c, layer, k, v, q, out, ws, lcd::kScratchBytes, stream);
}

int64_t lcd_kv_tokens(const lcd_cache* c, int32_t layer) {
  if (check_layer(c, layer)) return -1;
  return c->tokens[layer];
}

int64_t lcd_kv_filled(const lcd_cache* c, int32_t layer) {
  if (check_layer(c, layer)) return -1;
  return c->filled[layer];
}

int64_t lcd_kv_slot_of(const lcd_cache* c, int32_t layer, int64_t token) {
  if (check_layer(c, layer) || token < 0) return -1;
  const lcd_cache_config& cfg = c->cfg;
  if (cfg.policy == LCD_SINK_RING) {
    if (token < cfg.n_sink) return token;
    return cfg.n_sink + (token - cfg.n_sink) % cfg.window;
  }
  if (cfg.policy == LCD_APPEND) return token < c->filled[layer] ? token : -1;
  return -1;
}

int64_t lcd_kv_rank_of(const lcd_cache* c, int32_t layer, int64_t slot) {
  if (check_layer(c, layer) || slot < 0) return -1;
  const lcd_cache_config& cfg = c->cfg;
  if (cfg.policy != LCD_SINK_RING) return -1;
  const int64_t n = c->filled[layer];
  if (slot >= n) return -1;
  const int64_t t = c->tokens[layer] - 1;
  if (t + 1 <= c->L.C || slot < cfg.n_sink) return slot;
  const int64_t head = (t - cfg.window + 1 - cfg.n_sink) % cfg.window;
  int64_t r = slot - cfg.n_sink - head;
  if (r < 0) r += cfg.window;
  return cfg.n_sink + r;
}

lcd_status lcd_kv_layer_view(const lcd_cache* c, int32_t layer, void** k, void** v, int32_t** pos, float** score) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (c->cfg.policy == LCD_DUO)
    return fail(LCD_EUNSUPPORTED, "a mixed-head layer has no single [batch][heads][C][D] view");
  if (k) *k = c->k_layer(layer);
  if (v) *v = c->v_layer(layer);
  if (pos) *pos = c->pos(layer);
  if (score) *score = c->score(layer);
  return ok();
}

lcd_status lcd_kv_set_filled(lcd_cache* c, int32_t layer, int32_t n, int64_t next_token, void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (c->cfg.policy == LCD_SINK_RING || c->cfg.policy == LCD_DUO)
    return fail(LCD_EUNSUPPORTED, "set_filled applies to APPEND and H2O caches");
  if (n < 0 || n > c->L.C) return fail(LCD_ECAPACITY, "n=%d outside [0, %d]", n, c->L.C);
  if (next_token < n) return fail(LCD_EINVAL, "next_token must be >= n");
  if (c->cfg.policy == LCD_H2O && next_token > INT32_MAX) return fail(LCD_ECAPACITY, "H2O token positions are int32");
  const int bs = c->bs();
  if (c->cfg.policy == LCD_H2O && n == c->L.C) {
    const hipError_t e = lcd::launch_h2o_pick_victim(c->score(layer), c->pos(layer), c->victim(layer),
                                                     c->cfg.batch * c->cfg.n_kv_heads, c->L.C, n,
                                                     next_token - c->cfg.n_recent, bs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set_filled victim launch");
  }
  if (c->cfg.policy == LCD_H2O) c->open_fill[layer] = n % bs ? n % bs : (n ? bs : 0);
  c->filled[layer] = n;
  c->tokens[layer] = next_token;
  return ok();
}

int64_t lcd_kv_layer_bytes(const lcd_cache* c, int32_t layer) {
  if (check_layer(c, layer)) return -1;
  return (int64_t)(c->cfg.policy == LCD_DUO ? c->L.duo_bytes[layer] : c->L.layer_bytes);
}

}  // extern "C"

namespace {

// Checks shared by lcd_kv_save and lcd_kv_load: the buffers a layer's state needs.
lcd_status check_state_buffers(const lcd_cache* c, const void* k, const void* v, const void* pos,
                               const void* score, const void* victim, const void* open) {
  if (!k || !v) return fail(LCD_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(LCD_EALIGN, "k or v is not 16-byte aligned");
  if (c->cfg.policy == LCD_H2O) {
    if (!pos || !score || !victim || !open) return fail(LCD_EINVAL, "an H2O layer needs pos, score, victim and open");
  } else if (pos || score || victim || open) {
    return fail(LCD_EINVAL, "pos, score, victim and open are H2O state (pass NULL)");
  }
  return LCD_OK;
}

// Copies of one layer's device state between the cache and caller buffers, on the stream.
lcd_status copy_layer_state(const lcd_cache* c, int32_t layer, void* k, void* v, int32_t* pos, float* score,
                            int32_t* victim, int32_t* open, bool save, hipStream_t s) {
  const uint64_t kvb = c->cfg.policy == LCD_DUO ? c->L.duo_bytes[layer] : c->L.layer_bytes;
  struct Item {
    void* buf;
    void* dev;
    uint64_t bytes;
  };
  const uint64_t per_bg = (uint64_t)c->cfg.batch * c->cfg.n_kv_heads;
  std::vector<Item> items = {{k, c->k_layer(layer), kvb}, {v, c->v_layer(layer), kvb}};
  if (c->cfg.policy == LCD_H2O) {
    items.push_back({pos, c->pos(layer), per_bg * c->L.C * sizeof(int32_t)});
    items.push_back({score, c->score(layer), per_bg * c->L.C * sizeof(float)});
    items.push_back({victim, c->victim(layer), per_bg * sizeof(int32_t)});
    items.push_back({open, c->open_block(layer), per_bg * sizeof(int32_t)});
  }
  for (const Item& it : items) {
    const hipError_t e = save ? hipMemcpyAsync(it.buf, it.dev, it.bytes, hipMemcpyDeviceToDevice, s)
                              : hipMemcpyAsync(it.dev, it.buf, it.bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, save ? "kv_save copy" : "kv_load copy");
  }
  return LCD_OK;
}

}  // namespace

extern "C" {

lcd_status lcd_kv_save(const lcd_cache* c, int32_t layer, void* k, void* v, int32_t* pos, float* score,
                       int32_t* victim, int32_t* open, lcd_layer_state* state, void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (!state) return fail(LCD_EINVAL, "state is NULL");
  if ((st = check_state_buffers(c, k, v, pos, score, victim, open))) return st;
  if ((st = copy_layer_state(c, layer, k, v, pos, score, victim, open, true, static_cast<hipStream_t>(stream))))
    return st;
  state->tokens = c->tokens[layer];
  state->filled = c->filled[layer];
  state->open_fill = c->open_fill[layer];
  state->reserved = 0;
  return ok();
}

lcd_status lcd_kv_load(lcd_cache* c, int32_t layer, const void* k, const void* v, const int32_t* pos,
                       const float* score, const int32_t* victim, const int32_t* open, const lcd_layer_state* state,
                       void* stream) {
  lcd_status st = check_layer(c, layer);
  if (st) return st;
  if (!state) return fail(LCD_EINVAL, "state is NULL");
  if ((st = check_state_buffers(c, k, v, pos, score, victim, open))) return st;
  const lcd_cache_config& cfg = c->cfg;
  const int64_t C = c->L.C;
  if (state->filled < 0 || state->filled > C || state->tokens < state->filled)
    return fail(LCD_EINVAL, "state: need 0 <= filled <= capacity %lld and tokens >= filled", (long long)C);
  if (cfg.policy == LCD_SINK_RING && state->filled != std::min<int64_t>(state->tokens, C))
    return fail(LCD_EINVAL, "state: a sink + ring layer holds min(tokens, n_sink + window) slots");
  if (cfg.policy == LCD_DUO && state->filled != state->tokens)
    return fail(LCD_EINVAL, "state: a mixed-head layer's retrieval heads hold every token");
  const int bs = c->bs();
  if (state->open_fill < 0 || state->open_fill > bs || (cfg.policy != LCD_H2O && state->open_fill != 0))
    return fail(LCD_EINVAL, "state: open_fill outside [0, block size]");
  if (cfg.policy == LCD_H2O && state->tokens > INT32_MAX) return fail(LCD_ECAPACITY, "H2O token positions are int32");
  if ((st = copy_layer_state(c, layer, const_cast<void*>(k), const_cast<void*>(v), const_cast<int32_t*>(pos),
                             const_cast<float*>(score), const_cast<int32_t*>(victim), const_cast<int32_t*>(open),
                             false, static_cast<hipStream_t>(stream))))
    return st;
  c->tokens[layer] = state->tokens;
  c->filled[layer] = state->filled;
  c->open_fill[layer] = state->open_fill;
  return ok();
}

lcd_status lcd_snapkv_sizes(const lcd_snapkv_params* p, uint64_t* ws_bytes);
lcd_status lcd_snapkv_compress(const lcd_snapkv_params* p, const void* q_obs, const void* k, const void* v,
                               void* k_out, void* v_out, int32_t* idx_out, float* scores_out, void* ws,
                               uint64_t ws_bytes, void* stream);

}  // extern "C"

// ------------------------------------------------------------------------------ SnapKV
namespace {

lcd_status check_snapkv(const lcd_snapkv_params* p) {
  if (!p) return fail(LCD_EINVAL, "params is NULL");
  if (p->batch < 1 || p->n_heads < 1 || p->n_prompt < 1) return fail(LCD_ESHAPE, "batch, n_heads, n_prompt >= 1");
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(LCD_ESHAPE, "head_dim %d not in {64, 128, 256}", p->head_dim);
  const int max_obs = p->head_dim <= 128 ? 256 : 128;  // window queries staged in LDS beyond 64 rows
  if (p->l_obs < 1 || p->l_obs > max_obs || p->l_obs > p->n_prompt)
    return fail(LCD_ESHAPE, "l_obs %d outside [1, min(N, %d)]", p->l_obs, max_obs);
  if (p->kernel_size < 1 || p->kernel_size > 31 || p->kernel_size % 2 == 0)
    return fail(LCD_ESHAPE, "kernel_size must be odd and in [1, 31]");
  if (p->k_keep < 0 || p->k_keep > p->n_prompt - p->l_obs)
    return fail(LCD_ESHAPE, "k_keep %d outside [0, N - l_obs]", p->k_keep);
  if (p->pool != 0 && p->pool != 1) return fail(LCD_EINVAL, "pool must be 0 (avg) or 1 (max)");
  if (p->dtype != LCD_BF16) return fail(LCD_EUNSUPPORTED, "SnapKV scoring runs on bf16 inputs only");
  if (p->out_rows != 0 && p->out_rows < p->k_keep + p->l_obs)
    return fail(LCD_ESHAPE, "out_rows %d < k_keep + l_obs", p->out_rows);
  if ((int64_t)p->n_prompt - p->l_obs > 64 * 1024)
    return fail(LCD_ESHAPE, "n_prompt - l_obs must be <= 65536 (per-head selection is register-resident)");
  if (!(std::isfinite(p->scale) && p->scale >= 0.0)) return fail(LCD_EINVAL, "scale must be finite and >= 0");
  return LCD_OK;
}

}  // namespace

extern "C" lcd_status lcd_snapkv_sizes(const lcd_snapkv_params* p, uint64_t* ws_bytes) {
  const lcd_status st = check_snapkv(p);
  if (st) return st;
  if (ws_bytes) *ws_bytes = lcd::snapkv_ws_bytes(p->batch, p->n_heads, p->n_prompt, p->l_obs);
  return ok();
}

extern "C" lcd_status lcd_snapkv_compress(const lcd_snapkv_params* p, const void* q_obs, const void* k,
                                          const void* v, void* k_out, void* v_out, int32_t* idx_out,
                                          float* scores_out, void* ws, uint64_t ws_bytes, void* stream) {
  lcd_status st = check_snapkv(p);
  if (st) return st;
  if (!q_obs || !k || !v || !k_out || !v_out || !idx_out || !ws)
    return fail(LCD_EINVAL, "a required pointer is NULL");
  const void* ptrs[] = {q_obs, k, v, k_out, v_out, idx_out, ws};
  for (const void* x : ptrs)
    if (!aligned16(x)) return fail(LCD_EALIGN, "pointers must be 16-byte aligned");
  if (scores_out && !aligned16(scores_out)) return fail(LCD_EALIGN, "scores_out not 16-byte aligned");
  const uint64_t need = lcd::snapkv_ws_bytes(p->batch, p->n_heads, p->n_prompt, p->l_obs);
  if (ws_bytes < need)
    return fail(LCD_ESIZE, "ws_bytes %llu < required %llu", (unsigned long long)ws_bytes, (unsigned long long)need);
  lcd::SnapkvParams s{};
  s.q_obs = q_obs;
  s.k = k;
  s.v = v;
  s.k_out = k_out;
  s.v_out = v_out;
  s.idx_out = idx_out;
  s.scores_out = scores_out;
  s.B = p->batch;
  s.H = p->n_heads;
  s.D = p->head_dim;
  s.N = p->n_prompt;
  s.Lobs = p->l_obs;
  s.ksize = p->kernel_size;
  s.k_keep = p->k_keep;
  s.pool = p->pool;
  s.out_rows = p->out_rows ? p->out_rows : p->k_keep + p->l_obs;
  const double scale = p->scale > 0 ? p->scale : 1.0 / std::sqrt((double)p->head_dim);
  s.qscale = (float)(scale * 1.4426950408889634074);
  char* w = static_cast<char*>(ws);
  s.rowstat = reinterpret_cast<float*>(w);  // carved further inside launch_snapkv
  const hipError_t e = lcd::launch_snapkv(s, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "snapkv launch");
  return ok();
}

// ------------------------------------------------------------------ H2O prompt phase
namespace {

lcd_status check_h2o_prompt(const lcd_h2o_prompt_params* p) {
  if (!p) return fail(LCD_EINVAL, "params is NULL");
  if (p->batch < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1) return fail(LCD_ESHAPE, "batch and heads must be >= 1");
  if (p->n_q_heads % p->n_kv_heads)
    return fail(LCD_ESHAPE, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", p->n_q_heads, p->n_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(LCD_ESHAPE, "head_dim %d not in {64, 128, 256}", p->head_dim);
  if (p->n_prompt < 1 || p->n_prompt > 262144) return fail(LCD_ESHAPE, "n_prompt %d outside [1, 262144]", p->n_prompt);
  if (p->n_recent < 1 || p->budget < p->n_recent) return fail(LCD_ESHAPE, "need 1 <= n_recent <= budget");
  if (p->dtype != LCD_BF16) return fail(LCD_EUNSUPPORTED, "the prompt-phase scores run on bf16 MFMA (dtype must be bf16)");
  if (!(std::isfinite(p->scale) && p->scale >= 0.0)) return fail(LCD_EINVAL, "scale must be finite and >= 0");
  uint64_t e = (uint64_t)p->batch;
  if (!mul_ok(&e, p->n_q_heads) || !mul_ok(&e, p->n_prompt) || !mul_ok(&e, p->head_dim) || e > (uint64_t)1 << 40)
    return fail(LCD_ESIZE, "prompt tensors too large");
  return LCD_OK;
}

}  // namespace

extern "C" lcd_status lcd_h2o_prompt_sizes(const lcd_h2o_prompt_params* p, uint64_t* ws_bytes) {
  const lcd_status st = check_h2o_prompt(p);
  if (st) return st;
  if (ws_bytes) *ws_bytes = lcd::h2o_prompt_ws_bytes(p->batch, p->n_q_heads, p->n_kv_heads, p->n_prompt);
  return ok();
}

extern "C" lcd_status lcd_h2o_prompt_compress(const lcd_h2o_prompt_params* p, const void* q, const void* k,
                                              const void* v, void* k_out, void* v_out, int32_t* pos_out,
                                              float* score_out, float* scores_all, void* ws, uint64_t ws_bytes,
                                              void* stream) {
  lcd_status st = check_h2o_prompt(p);
  if (st) return st;
  if (!q || !k || !v || !k_out || !v_out || !pos_out || !score_out || !ws)
    return fail(LCD_EINVAL, "a required buffer is NULL");
  const void* bufs[] = {q, k, v, k_out, v_out, pos_out, score_out, ws};
  for (const void* b : bufs)
    if (!aligned16(b)) return fail(LCD_EALIGN, "buffers must be 16-byte aligned");
  if (scores_all && !aligned16(scores_all)) return fail(LCD_EALIGN, "scores_all must be 16-byte aligned");
  const uint64_t need = lcd::h2o_prompt_ws_bytes(p->batch, p->n_q_heads, p->n_kv_heads, p->n_prompt);
  if (ws_bytes < need)
    return fail(LCD_ESIZE, "ws_bytes %llu < required %llu", (unsigned long long)ws_bytes, (unsigned long long)need);
  lcd::H2oPromptParams h{};
  h.q = q;
  h.k = k;
  h.v = v;
  h.k_out = k_out;
  h.v_out = v_out;
  h.pos_out = pos_out;
  h.score_out = score_out;
  h.B = p->batch;
  h.Hq = p->n_q_heads;
  h.Hkv = p->n_kv_heads;
  h.D = p->head_dim;
  h.N = p->n_prompt;
  h.budget = p->budget;
  h.n_recent = p->n_recent;
  const double scale = p->scale > 0 ? p->scale : 1.0 / std::sqrt((double)p->head_dim);
  h.qscale = (float)(scale * 1.4426950408889634074);
  const hipError_t e = lcd::launch_h2o_prompt(h, ws, scores_all, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "h2o prompt launch");
  return ok();
}

// ------------------------------------------------------------------ PyramidKV budgets
extern "C" lcd_status lcd_pyramid_budgets(int32_t n_layers, int32_t b_base, int32_t b_target, int32_t* out) {
  if (!out) return fail(LCD_EINVAL, "budgets_out is NULL");
  if (n_layers < 1 || n_layers > 4096) return fail(LCD_EINVAL, "n_layers %d outside 1..4096", n_layers);
  const int32_t kMaxBudget = int32_t(1) << 24;
  if (b_base < 0 || b_base > kMaxBudget || b_target < 0 || b_target > kMaxBudget)
    return fail(LCD_EINVAL, "budgets must lie in 0..2^24");
  std::vector<int64_t> b(n_layers);
  if (n_layers == 1) {
    b[0] = b_target;
  } else {
    // B_l = b_base + floor(2 * (b_target - b_base) * (n_layers - 1 - l) / (n_layers - 1))
    const int64_t den = n_layers - 1;
    int64_t sum = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
      const int64_t num = 2 * (int64_t)(b_target - b_base) * (n_layers - 1 - l);
      const int64_t q = num >= 0 ? num / den : -((-num + den - 1) / den);  // floor division
      b[l] = b_base + q;
      sum += b[l];
    }
    const int64_t lost = (int64_t)n_layers * b_target - sum;  // 0 <= lost < n_layers
    for (int64_t l = 0; l < lost; ++l) b[l] += 1;
  }
  for (int32_t l = 0; l < n_layers; ++l)
    if (b[l] < 0) return fail(LCD_EINVAL, "layer %d budget would be negative (b_base > 2 * b_target)", l);
  for (int32_t l = 0; l < n_layers; ++l) out[l] = (int32_t)b[l];
  return ok();
}
