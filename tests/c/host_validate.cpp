// Drives every entry point of the C ABI through its validation and bookkeeping paths on
// the host alone (kernel launches and copies are stand-ins, see host_stubs.cpp), for a
// build under AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers are
// fake, aligned addresses that the host code must never dereference.  Prints "ok" and
// returns 0 when every status is as expected.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "lcd.h"

extern long g_launches;

namespace {

int g_fail = 0;

#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::printf("FAIL line %d: %s (last error: %s)\n", __LINE__, #cond,      \
                  lcd_last_error());                                            \
      ++g_fail;                                                                 \
    }                                                                           \
  } while (0)

void* dev(int k) { return reinterpret_cast<void*>((uintptr_t(0x100) + k) << 32); }  // fake, 4 GiB apart

lcd_cache_config base_cfg(int policy) {
  lcd_cache_config c;
  std::memset(&c, 0, sizeof c);
  c.batch = 2;
  c.n_layers = 2;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.dtype = LCD_BF16;
  c.policy = policy;
  c.n_sink = 4;
  c.window = 60;
  c.capacity = 96;
  c.n_recent = 8;
  c.rope = policy == LCD_SINK_RING ? 1 : 0;
  c.rope_base = 10000.0;
  return c;
}

struct Bound {
  lcd_cache* h = nullptr;
  uint64_t kv = 0, aux = 0, ws = 0;
};

Bound bind(const lcd_cache_config& c) {
  Bound b;
  EXPECT(lcd_cache_sizes(&c, &b.kv, &b.aux, &b.ws) == LCD_OK);
  EXPECT(lcd_kv_cache_init(&c, dev(1), b.kv, b.aux ? dev(2) : nullptr, b.aux, nullptr, &b.h) == LCD_OK);
  EXPECT(b.h != nullptr);
  return b;
}

void bad_config_cases() {
  uint64_t kv, aux, ws;
  EXPECT(lcd_cache_sizes(nullptr, &kv, &aux, &ws) != LCD_OK);
  lcd_cache_config z;
  std::memset(&z, 0, sizeof z);
  EXPECT(lcd_cache_sizes(&z, &kv, &aux, &ws) != LCD_OK);
  const int32_t big = std::numeric_limits<int32_t>::max();
  struct Case {
    const char* what;
    void (*edit)(lcd_cache_config&);
  };
  const Case cases[] = {
      {"head_dim 80", [](lcd_cache_config& c) { c.head_dim = 80; }},
      {"group of 3", [](lcd_cache_config& c) { c.n_q_heads = 6; }},
      {"q heads not a multiple", [](lcd_cache_config& c) { c.n_q_heads = 7; }},
      {"zero kv heads", [](lcd_cache_config& c) { c.n_kv_heads = 0; }},
      {"negative batch", [](lcd_cache_config& c) { c.batch = -1; }},
      {"zero layers", [](lcd_cache_config& c) { c.n_layers = 0; }},
      {"dtype 7", [](lcd_cache_config& c) { c.dtype = 7; }},
      {"policy 9", [](lcd_cache_config& c) { c.policy = 9; }},
      {"window 0", [](lcd_cache_config& c) { c.window = 0; }},
      {"negative sinks", [](lcd_cache_config& c) { c.n_sink = -3; }},
      {"rope base 1", [](lcd_cache_config& c) { c.rope_base = 1.0; }},
      {"rope base nan", [](lcd_cache_config& c) { c.rope_base = std::nan(""); }},
      {"scale -1", [](lcd_cache_config& c) { c.scale = -1.0; }},
      {"scale inf", [](lcd_cache_config& c) { c.scale = INFINITY; }},
      {"huge ring", [](lcd_cache_config& c) { c.window = std::numeric_limits<int32_t>::max() - 2; c.n_sink = 100; }},
      {"huge batch x layers", [](lcd_cache_config& c) { c.batch = std::numeric_limits<int32_t>::max(); c.n_layers = 4096; }},
  };
  for (const Case& k : cases) {
    lcd_cache_config c = base_cfg(LCD_SINK_RING);
    k.edit(c);
    const lcd_status st = lcd_cache_sizes(&c, &kv, &aux, &ws);
    if (st == LCD_OK) std::printf("accepted: %s\n", k.what);
    EXPECT(st != LCD_OK);
  }
  // policy-specific limits
  lcd_cache_config c = base_cfg(LCD_APPEND);
  c.rope = 1;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);  // rope is for SINK_RING only
  c = base_cfg(LCD_APPEND);
  c.capacity = 0;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
  c = base_cfg(LCD_H2O);
  c.n_recent = c.capacity + 1;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
  c = base_cfg(LCD_H2O);
  c.block_size = 16;
  c.capacity = 100;  // not a multiple of the block size
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
  c = base_cfg(LCD_H2O);
  c.block_size = 7;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
  c = base_cfg(LCD_H2O);
  c.capacity = big;
  c.batch = big;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
  c = base_cfg(LCD_DUO);
  c.retrieval = nullptr;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) != LCD_OK);
}

void decode_paths(lcd_cache_config c, bool step_ok) {
  Bound b = bind(c);
  const uint64_t qb = 1 << 20;
  // bad handles, layers and buffers
  EXPECT(lcd_kv_append(nullptr, 0, dev(3), dev(4), 1, nullptr) != LCD_OK);
  EXPECT(lcd_kv_append(b.h, -1, dev(3), dev(4), 1, nullptr) != LCD_OK);
  EXPECT(lcd_kv_append(b.h, c.n_layers, dev(3), dev(4), 1, nullptr) != LCD_OK);
  EXPECT(lcd_kv_append(b.h, 0, nullptr, dev(4), 1, nullptr) != LCD_OK);
  EXPECT(lcd_kv_append(b.h, 0, dev(3), dev(4), 0, nullptr) != LCD_OK);
  EXPECT(lcd_kv_append(b.h, 0, dev(3), dev(4), -5, nullptr) != LCD_OK);
  EXPECT(lcd_decode_attn(b.h, 0, dev(5), (float*)dev(6), dev(7), b.ws, nullptr) != LCD_OK);  // no token yet
  EXPECT(lcd_kv_tokens(b.h, 0) == 0 && lcd_kv_filled(b.h, 0) == 0);
  EXPECT(lcd_kv_tokens(b.h, 5) == -1 && lcd_kv_filled(nullptr, 0) == -1);
  const int steps = c.policy == LCD_APPEND || c.policy == LCD_DUO ? 90 : 130;
  for (int t = 0; t < steps; ++t) {
    for (int l = 0; l < c.n_layers; ++l) {
      if (step_ok && (t % 2 == 1)) {
        EXPECT(lcd_decode_step(b.h, l, dev(3), dev(4), dev(5), (float*)dev(6), dev(7), b.ws, nullptr) == LCD_OK);
      } else if (step_ok && t % 3 == 0) {
        EXPECT(lcd_decode_step_noalloc(b.h, l, dev(3), dev(4), dev(5), (float*)dev(6), nullptr) == LCD_OK);
      } else {
        EXPECT(lcd_kv_append(b.h, l, dev(3), dev(4), 1, nullptr) == LCD_OK);
        EXPECT(lcd_decode_attn(b.h, l, dev(5), (float*)dev(6), dev(7), b.ws, nullptr) == LCD_OK);
      }
    }
  }
  EXPECT(lcd_kv_tokens(b.h, 0) == steps);
  EXPECT(lcd_decode_attn(b.h, 0, dev(5), (float*)dev(6), dev(7), b.ws - 1, nullptr) == LCD_ESIZE);
  EXPECT(lcd_decode_attn(b.h, 0, nullptr, (float*)dev(6), dev(7), b.ws, nullptr) != LCD_OK);
  EXPECT(lcd_decode_attn(b.h, 0, dev(5), nullptr, dev(7), b.ws, nullptr) != LCD_OK);
  EXPECT(lcd_decode_attn(b.h, 0, (char*)dev(5) + 2, (float*)dev(6), dev(7), b.ws, nullptr) != LCD_OK);
  if (!step_ok) {
    EXPECT(lcd_decode_step(b.h, 0, dev(3), dev(4), dev(5), (float*)dev(6), dev(7), b.ws, nullptr) != LCD_OK);
  }
  for (int64_t tok = 0; tok < steps; tok += 7) (void)lcd_kv_slot_of(b.h, 0, tok);
  for (int64_t s = 0; s < 100; s += 3) (void)lcd_kv_rank_of(b.h, 0, s);
  EXPECT(lcd_kv_slot_of(b.h, 0, -1) == -1);
  EXPECT(lcd_kv_rank_of(b.h, 0, -1) == -1);
  void *k = nullptr, *v = nullptr;
  int32_t* pos = nullptr;
  float* score = nullptr;
  const lcd_status view = lcd_kv_layer_view(b.h, 1, &k, &v, &pos, &score);
  EXPECT(c.policy == LCD_DUO ? view != LCD_OK : view == LCD_OK);
  // checkpoint: save, then reload the counters into the same cache
  const int64_t lb = lcd_kv_layer_bytes(b.h, 1);
  EXPECT(lb > 0);
  EXPECT(lcd_kv_layer_bytes(b.h, 9) == -1);
  lcd_layer_state st;
  std::memset(&st, 0, sizeof st);
  const bool h2o = c.policy == LCD_H2O;
  int32_t* p32 = h2o ? (int32_t*)dev(8) : nullptr;
  float* f32 = h2o ? (float*)dev(9) : nullptr;
  int32_t* vic = h2o ? (int32_t*)dev(10) : nullptr;
  int32_t* opn = h2o ? (int32_t*)dev(11) : nullptr;
  EXPECT(lcd_kv_save(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, &st, nullptr) == LCD_OK);
  EXPECT(st.tokens == steps);
  EXPECT(lcd_kv_load(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, &st, nullptr) == LCD_OK);
  EXPECT(lcd_kv_save(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, nullptr, nullptr) != LCD_OK);
  lcd_layer_state bad = st;
  bad.filled = st.filled + 1000000;
  EXPECT(lcd_kv_load(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, &bad, nullptr) != LCD_OK);
  bad = st;
  bad.tokens = -1;
  EXPECT(lcd_kv_load(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, &bad, nullptr) != LCD_OK);
  bad = st;
  bad.open_fill = -4;
  EXPECT(lcd_kv_load(b.h, 1, dev(12), dev(13), p32, f32, vic, opn, &bad, nullptr) != LCD_OK);
  EXPECT(lcd_kv_tokens(b.h, 1) == steps);
  if (c.policy == LCD_APPEND) {
    EXPECT(lcd_kv_set_filled(b.h, 0, 10, 10, nullptr) == LCD_OK);
    EXPECT(lcd_kv_set_filled(b.h, 0, c.capacity + 1, c.capacity + 1, nullptr) != LCD_OK);
    EXPECT(lcd_kv_set_filled(b.h, 0, -1, 0, nullptr) != LCD_OK);
    // fill to capacity, then one more is refused
    EXPECT(lcd_kv_set_filled(b.h, 0, c.capacity, c.capacity, nullptr) == LCD_OK);
    EXPECT(lcd_kv_append(b.h, 0, dev(3), dev(4), 1, nullptr) == LCD_ECAPACITY);
  }
  if (h2o) EXPECT(lcd_kv_append(b.h, 0, dev(3), dev(4), 2, nullptr) != LCD_OK);
  lcd_kv_cache_destroy(b.h);
}

void init_cases() {
  lcd_cache_config c = base_cfg(LCD_SINK_RING);
  uint64_t kv, aux, ws;
  EXPECT(lcd_cache_sizes(&c, &kv, &aux, &ws) == LCD_OK);
  lcd_cache* h = nullptr;
  EXPECT(lcd_kv_cache_init(&c, dev(1), kv - 1, dev(2), aux, nullptr, &h) != LCD_OK);
  EXPECT(lcd_kv_cache_init(&c, dev(1), kv, dev(2), aux - 1, nullptr, &h) != LCD_OK);
  EXPECT(lcd_kv_cache_init(&c, (char*)dev(1) + 4, kv, dev(2), aux, nullptr, &h) != LCD_OK);
  EXPECT(lcd_kv_cache_init(&c, dev(1), kv, dev(2), aux, nullptr, nullptr) != LCD_OK);
  EXPECT(lcd_kv_cache_init(&c, nullptr, kv, dev(2), aux, nullptr, &h) != LCD_OK);
  EXPECT(h == nullptr);
  lcd_kv_cache_destroy(nullptr);
}

void compression_cases() {
  lcd_snapkv_params p;
  std::memset(&p, 0, sizeof p);
  p.batch = 1;
  p.n_heads = 4;
  p.head_dim = 128;
  p.n_prompt = 4096;
  p.l_obs = 32;
  p.kernel_size = 5;
  p.k_keep = 500;
  p.dtype = LCD_BF16;
  uint64_t ws = 0;
  EXPECT(lcd_snapkv_sizes(&p, &ws) == LCD_OK && ws > 0);
  EXPECT(lcd_snapkv_compress(&p, dev(1), dev(2), dev(3), dev(4), dev(5), (int32_t*)dev(6), nullptr, dev(7), ws,
                             nullptr) == LCD_OK);
  EXPECT(lcd_snapkv_compress(&p, dev(1), dev(2), dev(3), dev(4), dev(5), (int32_t*)dev(6), nullptr, dev(7), ws - 1,
                             nullptr) != LCD_OK);
  EXPECT(lcd_snapkv_compress(&p, nullptr, dev(2), dev(3), dev(4), dev(5), (int32_t*)dev(6), nullptr, dev(7), ws,
                             nullptr) != LCD_OK);
  EXPECT(lcd_snapkv_sizes(nullptr, &ws) != LCD_OK);
  lcd_snapkv_params q = p;
  q.l_obs = 0;
  EXPECT(lcd_snapkv_sizes(&q, &ws) != LCD_OK);
  q = p;
  q.kernel_size = 4;
  EXPECT(lcd_snapkv_sizes(&q, &ws) != LCD_OK);
  q = p;
  q.k_keep = p.n_prompt;
  EXPECT(lcd_snapkv_sizes(&q, &ws) != LCD_OK);
  q = p;
  q.n_prompt = std::numeric_limits<int32_t>::max();
  EXPECT(lcd_snapkv_sizes(&q, &ws) != LCD_OK);
  q = p;
  q.scale = std::nan("");
  EXPECT(lcd_snapkv_sizes(&q, &ws) != LCD_OK);

  lcd_h2o_prompt_params h;
  std::memset(&h, 0, sizeof h);
  h.batch = 2;
  h.n_q_heads = 8;
  h.n_kv_heads = 2;
  h.head_dim = 128;
  h.n_prompt = 3000;
  h.budget = 512;
  h.n_recent = 64;
  h.dtype = LCD_BF16;
  EXPECT(lcd_h2o_prompt_sizes(&h, &ws) == LCD_OK && ws > 0);
  EXPECT(lcd_h2o_prompt_compress(&h, dev(1), dev(2), dev(3), dev(4), dev(5), (int32_t*)dev(6), (float*)dev(7),
                                 nullptr, dev(8), ws, nullptr) == LCD_OK);
  EXPECT(lcd_h2o_prompt_compress(&h, dev(1), dev(2), dev(3), dev(4), dev(5), (int32_t*)dev(6), (float*)dev(7),
                                 nullptr, dev(8), ws - 1, nullptr) != LCD_OK);
  lcd_h2o_prompt_params g = h;
  g.n_recent = 0;
  EXPECT(lcd_h2o_prompt_sizes(&g, &ws) != LCD_OK);
  g = h;
  g.n_recent = h.budget + 1;
  EXPECT(lcd_h2o_prompt_sizes(&g, &ws) != LCD_OK);
  g = h;
  g.n_q_heads = 7;
  EXPECT(lcd_h2o_prompt_sizes(&g, &ws) != LCD_OK);
  g = h;
  g.n_prompt = 1 << 20;
  EXPECT(lcd_h2o_prompt_sizes(&g, &ws) != LCD_OK);

  std::vector<int32_t> bud(4096);
  EXPECT(lcd_pyramid_budgets(32, 256, 1024, bud.data()) == LCD_OK);
  int64_t sum = 0;
  for (int i = 0; i < 32; ++i) sum += bud[i];
  EXPECT(sum == 32 * 1024);
  EXPECT(lcd_pyramid_budgets(1, 100, 100, bud.data()) == LCD_OK && bud[0] == 100);
  EXPECT(lcd_pyramid_budgets(4096, 1 << 24, 1 << 24, bud.data()) == LCD_OK);
  EXPECT(lcd_pyramid_budgets(0, 1, 1, bud.data()) != LCD_OK);
  EXPECT(lcd_pyramid_budgets(8, 300, 100, bud.data()) != LCD_OK);
  EXPECT(lcd_pyramid_budgets(8, 10, 100, nullptr) != LCD_OK);
  EXPECT(lcd_pyramid_budgets(8, -1, 100, bud.data()) != LCD_OK);
}

}  // namespace

int main() {
  EXPECT(lcd_abi_version() == LCD_ABI_VERSION);
  bad_config_cases();
  init_cases();
  decode_paths(base_cfg(LCD_SINK_RING), true);
  lcd_cache_config f = base_cfg(LCD_SINK_RING);
  f.dtype = LCD_F32;
  f.rope = 0;
  f.n_q_heads = 2;  // G = 1
  decode_paths(f, true);
  decode_paths(base_cfg(LCD_APPEND), true);
  decode_paths(base_cfg(LCD_H2O), true);
  lcd_cache_config hb = base_cfg(LCD_H2O);
  hb.block_size = 16;
  hb.n_recent = 16;
  decode_paths(hb, true);
  lcd_cache_config d = base_cfg(LCD_DUO);
  const int32_t ret[4] = {1, 0, 0, 1};
  d.retrieval = ret;
  d.capacity = 200;
  decode_paths(d, false);
  compression_cases();
  if (g_fail) {
    std::printf("%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ok: %ld stand-in launches\n", g_launches);
  return 0;
}
