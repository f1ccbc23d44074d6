/*
 * lcd.h -- C ABI of the compressed-KV decode library for AMD MI355X (gfx950).
 *
 * Single-token decode attention over a compressed KV cache, and the SnapKV
 * prefill compression that produces one.  Sources, cited by title and section:
 *   [KVC]  "Compressão e Poda Dinâmica de KV Cache: StreamingLLM, SnapKV,
 *          PyramidKV e DuoAttention" (produtoramaxvision.com.br).
 *   [SINK] "attention sinks" (tonho.wtf encyclopedia entry).
 *   [KVL]  "O KV cache", lesson 7.2 (llmdeepdive.com).
 *
 * Conventions shared by every entry point
 *   Ownership   All device memory (cache, auxiliary state, workspaces, inputs,
 *               outputs) is allocated and owned by the caller.  The library
 *               allocates no device memory; a cache handle owns only host-side
 *               state (configuration, per-layer token counters) and
 *               lcd_kv_cache_destroy frees only that.  The one piece of device
 *               memory the library holds is the scratch array of
 *               lcd_decode_step_noalloc, a static array of its code object.
 *   Pointers    "device" pointers must be device memory of the current HIP
 *               device, 16-byte aligned, laid out exactly as documented
 *               (row-major, innermost dimension last, no padding).
 *   Streams     `stream` is a hipStream_t passed as void*; NULL is the null
 *               stream.  Every call only enqueues work on that stream and
 *               returns; the library never synchronises.  Ordering across
 *               streams is the caller's responsibility.
 *   Errors      Every argument is validated on the host before anything is
 *               enqueued.  On error the call returns a non-zero lcd_status,
 *               enqueues nothing, leaves the handle's state unchanged and sets a
 *               thread-local message readable with lcd_last_error().  A failed
 *               kernel launch returns LCD_EHIP; faults inside a kernel surface at
 *               the caller's next synchronisation.  No C++ exception crosses the
 *               ABI.
 *   Threads     A handle is not thread-safe; distinct handles are independent.
 *   Dtypes      LCD_BF16 tensors hold bfloat16 bit patterns (uint16); LCD_F32
 *               tensors hold IEEE float32.  Attention outputs are always float32
 *               and accumulation is float32.
 */
#ifndef LCD_H
#define LCD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCD_ABI_VERSION 5  /* 5: checkpoint calls (lcd_kv_save, lcd_kv_load, lcd_kv_layer_bytes) */

typedef enum lcd_status {
  LCD_OK = 0,
  LCD_EINVAL = 1,       /* invalid argument value or null pointer             */
  LCD_ESHAPE = 2,       /* unsupported or inconsistent shape                  */
  LCD_EALIGN = 3,       /* pointer not 16-byte aligned                        */
  LCD_ECAPACITY = 4,    /* operation would exceed the cache capacity          */
  LCD_ESIZE = 5,        /* a caller buffer is smaller than required          */
  LCD_EHIP = 6,         /* a HIP runtime call or kernel launch failed        */
  LCD_EUNSUPPORTED = 7  /* valid request the library does not implement         */
} lcd_status;

typedef enum lcd_dtype { LCD_F32 = 0, LCD_BF16 = 1 } lcd_dtype;

/* Cache policies.
 * LCD_SINK_RING  [KVC] "Attention Sinks e o StreamingLLM para fluxos contínuos";
 *                [SINK] "como funciona".  n_sink fixed attention-sink slots followed
 *                by a circular buffer of `window` slots.  The window counts the
 *                token being decoded: kv_append writes (evicting the oldest window
 *                entry once full) before decode_attn attends, so the newest token
 *                attends itself.  Token a lives in slot a if a < n_sink, else in
 *                slot n_sink + (a - n_sink) mod window.
 * LCD_APPEND     Fixed capacity, rows appended in order and never evicted: the
 *                layout of a SnapKV-compressed cache ([KVC] "SnapKV e a seleção de
 *                contexto no prefill") that decode continues from.
 * LCD_H2O        [KVC] "Heavy-Hitter Oracle (H2O) e a esparsidade de cauda pesada".
 *                Fixed budget = capacity; one accumulated attention score per slot;
 *                when full, each append overwrites the slot of the lowest score
 *                among tokens older than the n_recent newest (ties evict the newer
 *                token).  decode_attn adds the step's attention weights (summed
 *                over the query heads sharing the KV head) to the scores and picks
 *                the next victim.
 * LCD_DUO        [KVC] "Decomposição funcional com o DuoAttention".  Each KV head of
 *                each layer is a retrieval head (full history: APPEND rows in order
 *                up to `capacity`, never evicted) or a streaming head (the 4 sinks +
 *                64 recent tokens of the page, in general n_sink sinks + a ring of
 *                `window` slots exactly as LCD_SINK_RING), as `retrieval` says.
 *                Both kinds are served by one decode launch.  Keys are used as given
 *                (rope = 0). */
typedef enum lcd_policy { LCD_SINK_RING = 0, LCD_APPEND = 1, LCD_H2O = 2, LCD_DUO = 3 } lcd_policy;

typedef struct lcd_cache_config {
  int32_t batch;       /* B >= 1 (all rows advance in lockstep); B * H_q <= 2^24  */
  int32_t n_layers;    /* 1 <= L <= 65536 cached attention layers                  */
  int32_t n_q_heads;   /* H_q, a multiple of n_kv_heads; H_q / H_kv <= 8           */
  int32_t n_kv_heads;  /* H_kv >= 1; query head h reads KV head h / (H_q / H_kv)  */
  int32_t head_dim;    /* D in {64, 128, 256}                                      */
  int32_t dtype;       /* lcd_dtype of K, V and q                                  */
  int32_t policy;      /* lcd_policy                                               */
  int32_t n_sink;      /* SINK_RING, DUO streaming heads: sink slots S >= 0         */
  int32_t window;      /* SINK_RING, DUO streaming heads: ring slots W >= 1;
                          SINK_RING capacity C = S + W                              */
  int32_t capacity;    /* APPEND, H2O: slots C >= 1 per (layer, batch row, KV head);
                          DUO: slots of a retrieval head                            */
  int32_t n_recent;    /* H2O: protected newest tokens, 1 <= n_recent <= capacity;
                          includes the token being decoded                          */
  int32_t rope;        /* SINK_RING only: 1 = keys are stored un-rotated and q and
                          every key are rotated at decode time at their in-cache
                          positions ([SINK] "como funciona"), 0 = no rotation.
                          Must be 0 for APPEND and H2O (their inputs are used as
                          given).  Rotation pairs element i with i + D/2 and turns
                          pair i by position * rope_base^(-2i/D).                  */
  double rope_base;    /* > 1 when rope = 1                                        */
  double scale;        /* logit scale; 0 selects 1/sqrt(head_dim)                  */
  const int32_t* retrieval; /* DUO: host int32 [n_layers][n_kv_heads], 1 = retrieval
                          head, 0 = streaming head (n_kv_heads <= 128); read during
                          lcd_cache_sizes / lcd_kv_cache_init only (the handle keeps
                          a copy).  Ignored by the other policies (may be NULL).    */
  int32_t block_size;  /* H2O: 0 or 1 = token-level eviction; 16 or 32 = block-level
                          eviction ([KVC] "Implementação prática em vLLM e SGLang"):
                          slots form blocks of block_size consecutive slots (capacity a
                          multiple of it, n_recent <= capacity - block_size); tokens
                          fill the open block, and when a full cache needs a new block
                          the block with the lowest summed score among those holding
                          none of the n_recent newest tokens (ties: the newer block) is
                          freed whole and reused.  Ignored by the other policies.      */
} lcd_cache_config;

typedef struct lcd_cache lcd_cache; /* opaque host handle */

/* Version of this ABI (LCD_ABI_VERSION). */
int lcd_abi_version(void);

/* Message of the last error on the calling thread ("" if none).  The pointer is
 * valid until the next lcd_* call on this thread. */
const char* lcd_last_error(void);

/* Sizes of the caller-owned buffers a cache with this configuration needs.
 *   kv_bytes   K and V of every layer:
 *              2 * n_layers * n_kv_heads * head_dim * C * bytes_per_elem * batch,
 *              the size model of [KVC] "O gargalo de memória do KV Cache em
 *              contextos longos" and [KVL] "01 · Conceito" with C retained slots.
 *              Layout: for layer l, K at l*2*P and V at (l*2+1)*P bytes, each
 *              [batch][n_kv_heads][C][head_dim], P = kv_bytes / (2 * n_layers).
 *              DUO: per layer l with R_l retrieval and T_l streaming heads, K then
 *              V, each [batch][R_l][capacity][head_dim] (retrieval heads in head
 *              order) followed by [batch][T_l][n_sink + window][head_dim]
 *              (streaming heads in head order); layers follow each other.
 *   aux_bytes  Per-cache state: int32 arrival counters of the split merge (one
 *              per layer, batch row and KV head), the float32 cos/sin table of
 *              the in-cache positions (SINK_RING with rope), per-slot token
 *              positions and scores and per-(layer, row, head) victim slots
 *              (H2O).  Opaque.
 *   ws_bytes   Workspace one lcd_decode_attn call needs (split partials, and
 *              logits for H2O).  Opaque; may be reused across calls that are
 *              ordered on one stream.
 * Any output pointer may be NULL.  Pure host function, no HIP call. */
lcd_status lcd_cache_sizes(const lcd_cache_config* cfg, uint64_t* kv_bytes, uint64_t* aux_bytes,
                           uint64_t* ws_bytes);

/* kv_cache_init: bind a cache to caller memory ([KVC] "Attention Sinks e o
 * StreamingLLM..." two contiguous partitions; [KVL] "01 · Conceito" KV cache).
 * kv_mem (device, >= kv_bytes) holds K/V; aux_mem (device, >= aux_bytes, may be
 * NULL when aux_bytes is 0) is initialised on `stream` (cos/sin table computed
 * on the device in float64 and rounded to float32; H2O state cleared).  The
 * K/V contents are not touched: no slot is attended before it is written.  On
 * success *out receives a new handle with every layer empty. */
lcd_status lcd_kv_cache_init(const lcd_cache_config* cfg, void* kv_mem, uint64_t kv_bytes, void* aux_mem,
                             uint64_t aux_bytes, void* stream, lcd_cache** out);

/* Free the host handle (never touches device memory).  NULL is ignored. */
void lcd_kv_cache_destroy(lcd_cache* cache);

/* kv_append: write the K/V of n_new new tokens of one layer ([KVL] "01 ·
 * Conceito": each step appends its own k_t, v_t; [SINK] "como funciona": keys are
 * stored before rotation).
 *   k, v   device, [batch][n_kv_heads][n_new][head_dim] in the cache dtype.
 *   n_new  >= 1.  SINK_RING writes only the tokens that survive (the sinks among
 *          them and the newest `window`), exactly as n_new single appends would.
 *          APPEND requires tokens + n_new <= capacity (else LCD_ECAPACITY).  H2O
 *          requires n_new == 1 (bulk state goes through lcd_kv_layer_view and
 *          lcd_kv_set_filled); when the cache is full the row overwrites the
 *          victim slot chosen on the device by the previous lcd_decode_attn of
 *          this layer.  DUO writes every row of a retrieval head in order
 *          (tokens + n_new <= capacity, else LCD_ECAPACITY) and, for a streaming
 *          head, the rows that survive as SINK_RING does; one launch for both.
 * Advances the layer's token counter by n_new. */
lcd_status lcd_kv_append(lcd_cache* cache, int32_t layer, const void* k, const void* v, int32_t n_new,
                         void* stream);

/* decode_attn: one decode step of one layer ([KVL] "01 · Conceito": the newest
 * query attends every cached key and mixes the cached values; [KVC] "O gargalo de
 * memória...": a decode step reads the whole cache; [KVC] "Implementação
 * prática...": the work is split along the sequence, FlashDecoding-style).
 *   q    device, [batch][n_q_heads][head_dim], cache dtype: the query of the token
 *        appended last (its in-cache position is the newest one).
 *   out  device float32 [batch][n_q_heads][head_dim].
 *   ws   device workspace of ws_bytes >= lcd_cache_sizes' ws_bytes.
 * Attends all retained tokens of the layer, including the newest.  SINK_RING with
 * rope rotates q and every key at its in-cache position.  H2O also adds the step's
 * attention weights to the slot scores and selects the next victim; call it once
 * after each append.  DUO: retrieval heads attend every appended token, streaming
 * heads their sinks and window, in the same launch.  LCD_EINVAL if the layer
 * holds no token. */
lcd_status lcd_decode_attn(lcd_cache* cache, int32_t layer, const void* q, float* out, void* ws,
                           uint64_t ws_bytes, void* stream);

/* decode_step: lcd_kv_append of one token followed by lcd_decode_attn, in one
 * launch ([KVL] "01 · Conceito": a decode step appends the token's k_t, v_t and
 * attends its q_t over the cache that now holds them).
 *   k, v   device, [batch][n_kv_heads][head_dim] in the cache dtype: the new token's
 *          rows (un-rotated).
 *   q, out, ws  as lcd_decode_attn.
 * The workgroup whose slot range holds the new token's slot writes the rows from k and
 * v into that slot before attending; the cache contents and the output equal those of
 * the two calls (the same arithmetic in the same order).  SINK_RING, APPEND and H2O
 * (DUO: LCD_EUNSUPPORTED); APPEND needs a free slot (else LCD_ECAPACITY).  For a full
 * H2O cache the slot is the victim the previous step chose on the device ([KVC]
 * "Heavy-Hitter Oracle (H2O)...": evict, write, attend, accumulate in one launch), or the
 * next slot of the open block / a freed block (block_size 16 / 32), and the step picks
 * the next victim.  Advances the layer's token counter by one; on an error nothing is
 * enqueued and the counters are unchanged. */
lcd_status lcd_decode_step(lcd_cache* cache, int32_t layer, const void* k, const void* v, const void* q,
                           float* out, void* ws, uint64_t ws_bytes, void* stream);

/* decode_step_noalloc: lcd_decode_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * There is no workspace argument: the split partials go to a scratch buffer the library
 * holds on each GPU, a 32 MiB file-scope device array resident until the process ends.
 *   k, v, q, out  as lcd_decode_step; the scratch of the current device is used.
 * Returns LCD_ESIZE, enqueueing nothing, when the cache's workspace (lcd_cache_sizes'
 * ws_bytes) exceeds 32 MiB; otherwise the same checks, results and bookkeeping as
 * lcd_decode_step, bit for bit.  The call allocates no memory (no hipMalloc / hipFree;
 * the first call on a device resolves the array's address once).  Every call on a GPU
 * shares that GPU's scratch and the scratch keeps the last call's contents (nothing in
 * it needs clearing): calls that can overlap on one GPU (on different streams, or on
 * streams not ordered with each other) race, and the caller must serialise them. */
lcd_status lcd_decode_step_noalloc(lcd_cache* cache, int32_t layer, const void* k, const void* v, const void* q,
                                   float* out, void* stream);

/* Host-side queries (pure host functions, no HIP call; -1 on invalid arguments).
 *   lcd_kv_tokens   tokens appended so far to `layer` (int64 counter).
 *   lcd_kv_filled   slots currently holding a token (<= capacity; DUO: of a
 *                   retrieval head).
 *   lcd_kv_slot_of  SINK_RING: slot that holds / held token `token`; APPEND:
 *                   the row index of the token-th appended row; H2O, DUO: -1 (the
 *                   slot depends on the head).
 *   lcd_kv_rank_of  SINK_RING: in-cache position of the token in `slot` right now
 *                   (-1 if the slot is empty); others: -1. */
int64_t lcd_kv_tokens(const lcd_cache* cache, int32_t layer);
int64_t lcd_kv_filled(const lcd_cache* cache, int32_t layer);
int64_t lcd_kv_slot_of(const lcd_cache* cache, int32_t layer, int64_t token);
int64_t lcd_kv_rank_of(const lcd_cache* cache, int32_t layer, int64_t slot);

/* Device addresses of one layer's state, for callers that fill a cache in place
 * (e.g. SnapKV output written straight into an APPEND cache).  k/v point at
 * [batch][n_kv_heads][C][head_dim]; pos (int32) and score (float32) at
 * [batch][n_kv_heads][C] (H2O only, else NULL).  Any output may be NULL.
 * DUO: LCD_EUNSUPPORTED (heads of a layer have two layouts; see lcd_cache_sizes). */
lcd_status lcd_kv_layer_view(const lcd_cache* cache, int32_t layer, void** k, void** v, int32_t** pos,
                             float** score);

/* Seed a layer whose first n rows (per batch row and KV head) were already
 * written in place through lcd_kv_layer_view: sets the fill count to n and the
 * token counter to next_token (the position of the next appended token).  APPEND
 * and H2O only (n <= capacity; others LCD_EUNSUPPORTED).  For H2O the caller has also written pos (distinct
 * token positions < next_token) and score of those rows; when n == capacity the
 * victim of the next append is chosen on `stream` from those scores (lowest score
 * among positions <= next_token - n_recent, ties evicting the higher position).
 * Otherwise nothing is enqueued. */
lcd_status lcd_kv_set_filled(lcd_cache* cache, int32_t layer, int32_t n, int64_t next_token, void* stream);

/* Checkpoint / resume --------------------------------------------------------
 * A layer's whole state is its device arrays (K and V; for H2O also the slot positions
 * and scores, the per-(row, KV head) victim slot and open block) and three host counters.
 * lcd_kv_save copies the device arrays into caller buffers on `stream` and returns the
 * counters; lcd_kv_load copies them back into a cache of the same configuration and sets
 * the counters, after which the layer continues exactly as the saved one would have
 * (decode outputs and later state bit for bit).  The library keeps nothing else per
 * layer: the position table is a function of the configuration and the split-merge
 * counters are zero between calls.
 *   k, v          device, lcd_kv_layer_bytes(layer) bytes each: the layer's K and V blocks
 *                 in the cache layout ([batch][n_kv_heads][C][head_dim], or the DUO
 *                 per-layer layout of lcd_cache_sizes).
 *   pos, score    device int32 / float32 [batch][n_kv_heads][C] (H2O; NULL otherwise).
 *   victim, open  device int32 [batch][n_kv_heads] (H2O; NULL otherwise).
 *   state         host: tokens appended, slots filled, tokens in the open block (H2O
 *                 blocks).  lcd_kv_load checks it against the configuration (filled <=
 *                 capacity, tokens >= filled, SINK_RING: filled = min(tokens, n_sink +
 *                 window), DUO: filled = tokens, open_fill in [0, block size] and 0
 *                 without H2O blocks); LCD_EINVAL otherwise, nothing enqueued.  An H2O
 *                 layer past 2^31 - 1 tokens is refused with LCD_ECAPACITY.
 * Buffers must not overlap the cache.  Asynchronous: the copies are ordered on `stream`. */
typedef struct lcd_layer_state {
  int64_t tokens;
  int64_t filled;
  int32_t open_fill;
  int32_t reserved;  /* 0 */
} lcd_layer_state;

/* Bytes of one layer's K block (= its V block); -1 on invalid arguments.  Host-only. */
int64_t lcd_kv_layer_bytes(const lcd_cache* cache, int32_t layer);

lcd_status lcd_kv_save(const lcd_cache* cache, int32_t layer, void* k, void* v, int32_t* pos, float* score,
                       int32_t* victim, int32_t* open, lcd_layer_state* state, void* stream);
lcd_status lcd_kv_load(lcd_cache* cache, int32_t layer, const void* k, const void* v, const int32_t* pos,
                       const float* score, const int32_t* victim, const int32_t* open,
                       const lcd_layer_state* state, void* stream);

/* SnapKV ---------------------------------------------------------------------
 * [KVC] "SnapKV e a seleção de contexto no prefill": at the end of prefill each
 * head keeps the prompt positions with the highest smoothed observation-window
 * score.  Steps: (1) the last l_obs prompt queries attend the prompt causally
 * (row t is prompt token N - l_obs + t and sees keys 0..N - l_obs + t), softmax
 * over those keys; (2) s_i = mean over the rows of the weight of key i; (3) s
 * over the prefix i < N - l_obs is pooled with a centred window of kernel_size
 * (zero padding; average divides by kernel_size, max takes the maximum); (4) the
 * k_keep prefix positions of highest pooled score are kept, ties to the lower
 * index, decided on float32 scores.  The kept rows are the selected positions in
 * ascending order followed by the observation window N - l_obs .. N - 1. */
typedef struct lcd_snapkv_params {
  int32_t batch;        /* >= 1                                                  */
  int32_t n_heads;      /* >= 1 (q_obs, k and v have the same head count)         */
  int32_t head_dim;     /* D in {64, 128, 256}                                    */
  int32_t n_prompt;     /* N >= 1, N - l_obs <= 65536 (LCD_ESHAPE otherwise)       */
  int32_t l_obs;        /* 1 <= l_obs <= min(N, 256) (128 when head_dim = 256)    */
  int32_t kernel_size;  /* odd, 1 <= kernel_size <= 31                            */
  int32_t k_keep;       /* 0 <= k_keep <= N - l_obs                               */
  int32_t pool;         /* 0 = average, 1 = max                                   */
  int32_t dtype;        /* LCD_BF16 (the scoring contraction runs on bf16 MFMA)   */
  int32_t out_rows;     /* rows per head of k_out / v_out / idx_out; 0 selects
                           k_keep + l_obs; otherwise >= k_keep + l_obs (rows past
                           k_keep + l_obs are left untouched)                     */
  double scale;         /* logit scale; 0 selects 1/sqrt(head_dim)                */
} lcd_snapkv_params;

/* Workspace bytes lcd_snapkv_compress needs for these parameters. */
lcd_status lcd_snapkv_sizes(const lcd_snapkv_params* p, uint64_t* ws_bytes);

/* snapkv_compress:
 *   q_obs       device [batch][n_heads][l_obs][head_dim]: queries of the last l_obs
 *               prompt tokens (already position-encoded, used as given).
 *   k, v        device [batch][n_heads][N][head_dim] (position-encoded keys).
 *   k_out,v_out device [batch][n_heads][out_rows][head_dim]: kept rows.
 *   idx_out     device int32 [batch][n_heads][out_rows]: kept prompt positions.
 *   scores_out  device float32 [batch][n_heads][N - l_obs] pooled scores, or NULL.
 *   ws          device workspace of ws_bytes >= lcd_snapkv_sizes.
 * All buffers distinct (no aliasing between inputs and outputs). */
lcd_status lcd_snapkv_compress(const lcd_snapkv_params* p, const void* q_obs, const void* k, const void* v,
                               void* k_out, void* v_out, int32_t* idx_out, float* scores_out, void* ws,
                               uint64_t ws_bytes, void* stream);

/* H2O prompt-phase compression -------------------------------------------------
 * [KVC] "Heavy-Hitter Oracle (H2O) e a esparsidade de cauda pesada": token j's score
 * is the attention it receives, s_j = sum over steps t of alpha_{t,j}; when the budget
 * is reached the cache keeps a recent partition (the n_recent newest tokens) and the
 * heavy hitters (the highest s among the older tokens).  Applied to a whole prompt:
 * s_j = sum over the query heads h of the KV head's group and over the prompt rows
 * t >= j of the causal softmax weight alpha_{h,t,j} (row t attends keys 0..t, logit
 * scale * <q_{h,t}, k_j>); the cache keeps the budget - n_recent highest s_j among
 * j < N - n_recent (ties to the lower position, decided on float32 s) in ascending
 * position order, then the n_recent newest tokens.  The output is the state of a full
 * LCD_H2O layer: k_out / v_out / pos_out / score_out can be the arrays
 * lcd_kv_layer_view returns (capacity = budget), followed by
 * lcd_kv_set_filled(layer, min(budget, N), N). */
typedef struct lcd_h2o_prompt_params {
  int32_t batch;       /* >= 1                                                      */
  int32_t n_q_heads;   /* H_q, a multiple of n_kv_heads                             */
  int32_t n_kv_heads;  /* H_kv >= 1                                                 */
  int32_t head_dim;    /* D in {64, 128, 256}                                       */
  int32_t n_prompt;    /* N, 1 .. 262144                                            */
  int32_t budget;      /* kept rows per (batch row, KV head), n_recent <= budget;
                          a budget >= N keeps every token                          */
  int32_t n_recent;    /* >= 1                                                      */
  int32_t dtype;       /* LCD_BF16 (the score contractions run on bf16 MFMA)        */
  double scale;        /* logit scale; 0 selects 1/sqrt(head_dim)                   */
} lcd_h2o_prompt_params;

/* Workspace bytes lcd_h2o_prompt_compress needs for these parameters. */
lcd_status lcd_h2o_prompt_sizes(const lcd_h2o_prompt_params* p, uint64_t* ws_bytes);

/* h2o_prompt_compress:
 *   q           device [batch][n_q_heads][N][head_dim] prompt queries (as given)
 *   k, v        device [batch][n_kv_heads][N][head_dim]
 *   k_out,v_out device [batch][n_kv_heads][budget][head_dim]: kept rows; with
 *               budget > N rows N .. budget-1 are left untouched
 *   pos_out     device int32 [batch][n_kv_heads][budget]: kept prompt positions
 *   score_out   device float32 [batch][n_kv_heads][budget]: s of each kept token
 *   scores_all  device float32 [batch][n_kv_heads][N]: s of every token, or NULL
 *   ws          device workspace of ws_bytes >= lcd_h2o_prompt_sizes
 * All buffers distinct. */
lcd_status lcd_h2o_prompt_compress(const lcd_h2o_prompt_params* p, const void* q, const void* k, const void* v,
                                   void* k_out, void* v_out, int32_t* pos_out, float* score_out,
                                   float* scores_all, void* ws, uint64_t ws_bytes, void* stream);

/* PyramidKV per-layer budgets ---------------------------------------------------
 * [KVC] "Alocação piramidal com o PyramidKV": the budget of layer l falls linearly
 * with depth, B_l = b_base + dB * (n_layers - 1 - l) / (n_layers - 1), and the
 * budgets meet the global target, sum B_l = n_layers * b_target, which fixes
 * dB = 2 * (b_target - b_base).  Whole tokens: each B_l is rounded down and the
 * tokens that rounding lost (fewer than n_layers) go one each to the lowest layers
 * 0, 1, ..., so the sum is exact; one layer gets b_target.  Layer 0 is the lowest.
 * A budget counts every row a layer keeps per head: with SnapKV, k_keep = B_l - l_obs.
 *   n_layers     1 .. 4096
 *   b_base       budget of the top layer, 0 .. 2^24
 *   b_target     mean budget, 0 .. 2^24
 *   budgets_out  host int32 [n_layers], written on success only
 * Host-only (no device work, no stream).  LCD_EINVAL for a null pointer, values out
 * of range, or a layer budget that would be negative (b_base > 2 * b_target). */
lcd_status lcd_pyramid_budgets(int32_t n_layers, int32_t b_base, int32_t b_target, int32_t* budgets_out);

#ifdef __cplusplus
}
#endif

#endif /* LCD_H */
