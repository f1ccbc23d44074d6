// Internal launch interface between the host library (lcd_host.cpp) and the HIP
// kernels.  Plain structs of pointers and sizes; nothing here crosses the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcd {

// Decode workgroup: 4 waves of 64 lanes.
constexpr int kDecodeThreads = 256;
// Decode workgroups assumed resident at once (2 per CU on 256 CUs), for the split plan.
constexpr int kResidentWorkgroups = 512;

// kModeMaskedLogits: kModePlainLogits where slots with mask_pos[slot] < 0 are skipped
enum DecodeMode { kModeRope = 0, kModePlain = 1, kModePlainLogits = 2, kModeMaskedLogits = 3 };

// Most KV heads per layer of a mixed retrieval / streaming (DuoAttention) cache: the
// per-head map travels in the kernel arguments.
constexpr int kMaxDuoHeads = 128;

struct DecodeParams {
  void* k;             // layer K [B][Hkv][C][D] (cache dtype; written only by a fused append)
  void* v;             // layer V
  const void* q;       // [B][Hq][D]
  const float* cos_t;  // [C][D/2] (rope mode)
  const float* sin_t;
  float* out;          // [B][Hq][D] float32
  float* part_o;       // [splits][B][Hq][D]
  float* part_ml;      // [splits][B][Hq][2]  (max, sum) in the log2 domain
  float* logits;       // [B][Hq][C] per slot: log2-domain logit (one-pass kernel) or the
                       // split's weight 2^(x - m_s) (two-pass kernel) (logits mode)
  int* arrivals;       // layer [B][Hkv] arrival counters, zero between calls
  // H2O epilogue (logits mode)
  float* score;        // layer [B][Hkv][C]
  const int* pos;      // layer [B][Hkv][C]
  int* victim;         // layer [B][Hkv]
  int pick_victim;     // cache full: choose the slot the next append overwrites
  int64_t max_pos;     // victim candidates have pos <= max_pos
  int bs;              // H2O eviction granule: 1 = token, 16 / 32 = block of slots
  const int* mask_pos; // H2O blocks: slots with mask_pos[slot] < 0 are empty (not attended)
  int B, Hq, Hkv, C;
  int n;               // attended slots 0..n-1
  int chunk;           // slots per split (multiple of 64)
  int n_splits;
  int full;            // ring has wrapped: ranks follow the ring order
  int S, W;            // sinks and window (rope mode)
  // mixed heads (duo = 1): duo_map[g] >= 0 is KV head g's index among the Hret
  // retrieval heads (k / v, [B][Hret][C][D], n attended slots); duo_map[g] < 0 is
  // -1 - its index among the Hstr streaming heads (k2 / v2, [B][Hstr][C2][D], n2
  // attended slots).  n_splits is the larger split count of the two kinds.
  // The grid lists only real work: ret_splits x B x Hret retrieval items, then
  // str_splits x B x Hstr streaming items; duo_ret / duo_str give the KV head of each
  // retrieval / streaming index.
  int duo, Hret, Hstr, C2, n2, ret_splits, str_splits;
  const void* k2;
  const void* v2;
  int16_t duo_map[kMaxDuoHeads];
  int16_t duo_ret[kMaxDuoHeads];
  int16_t duo_str[kMaxDuoHeads];
  int ring_head;       // ring index of the oldest window token (rope mode, full)
  // fused append: the token's K / V rows ([B][Hkv][D], cache dtype) are read from k_new /
  // v_new and written into its slot by the workgroup whose range holds that slot.  The
  // slot is new_slot when >= 0; for an H2O cache (h2o_step = 1) with new_slot < 0 it is
  // chosen on the device per (row, KV head): victim[bg] (token granule), victim[bg] * bs (a
  // freed block, new_block = 1, whose other slots are emptied) or open[bg] * bs + offset.
  // The merging workgroup records the token's position and zero score (and the emptied
  // slots), so no slot of the position / score arrays has two writers in one launch.
  const void* k_new;
  const void* v_new;
  int new_slot;
  int h2o_step, new_block, offset;
  int* open;
  int64_t token;
  int q_rank;          // in-cache position of the query (rope mode)
  float qscale;        // logit scale * log2(e)
};

struct AppendParams {
  const char* k_in;    // [B][Hkv][n_new][D]
  const char* v_in;
  char* k_cache;       // layer [B][Hkv][C][D]
  char* v_cache;
  int BHkv, C, n_new, row_bytes;
  // rows [r0, r0 + n_rows) of the input are written; row r goes to
  //   slot_lin + (r - r0)                      if r <  r_split
  //   S + (ring_off + (r - r_split)) % W       if r >= r_split
  int r0, n_rows, r_split, slot_lin, ring_off, S, W;
  // H2O: one row per (b, kv head), slot = fill < C ? fill : victim[bh]; blocks of bs
  // slots: at a full cache a new block (new_block) takes victim[bh] (recorded in open[bh],
  // its other slots emptied), otherwise the row goes to slot open[bh] * bs + offset
  int h2o, fill, bs, new_block, offset;
  int* open;
  // mixed heads (duo = 1): rows of input token a = t0 + r go to a retrieval head's
  // slot a, or to a streaming head's sink / ring slot when a < S or a >= a_first
  int duo, Hkv, Hret, Hstr, C2;
  int64_t t0, a_first;
  char* k2_cache;
  char* v2_cache;
  int16_t duo_map[kMaxDuoHeads];
  const int* victim;
  int* pos;
  float* score;
  int64_t token;
};

hipError_t launch_decode_split(int dtype, int D, int G, int mode, const DecodeParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_h2o_pick_victim(const float* score, const int* pos, int* victim, int BHkv, int C, int n,
                                  int64_t max_pos, int bs, hipStream_t s);
hipError_t launch_rope_table(float* cos_t, float* sin_t, int C, int D, double base, hipStream_t s);
hipError_t launch_fill_i32(int* p, int value, int64_t n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float value, int64_t n, hipStream_t s);

// Device scratch of lcd_decode_step_noalloc (split partials): a file-scope array of
// kScratchBytes per GPU (scratch.hip).  scratch_device_address gives its address on the
// current device, resolved once per device with that device current:
// hipErrorInvalidDevice for a device id beyond the library's table, hipErrorInvalidValue
// if the address is not 256-byte aligned, otherwise the runtime's error.
constexpr uint64_t kScratchBytes = uint64_t(32) << 20;
hipError_t scratch_device_address(void** out);

bool decode_supported(int dtype, int D, int G);
// Most slots one decode workgroup may own for G query heads per KV head (a multiple of 64).
int decode_chunk_cap(int G);

// SnapKV
struct SnapkvParams {
  const void* q_obs;   // [B][H][Lobs][D] bf16
  const void* k;       // [B][H][N][D]
  const void* v;
  void* k_out;         // [B][H][out_rows][D]
  void* v_out;
  int* idx_out;        // [B][H][out_rows]
  float* scores_out;   // [B][H][N - Lobs] or null
  float* rowstat;      // ws: [B][H][tiles][Lobs][2]
  float* colscore;     // ws: [B][H][sstride] raw mean scores (N - Lobs used)
  float* pooled;       // ws: [B][H][sstride]
  int B, H, D, N, Lobs, ksize, k_keep, pool, out_rows, tiles;
  int sstride;         // row stride of colscore / pooled: N - Lobs rounded up to 4
  int h0;              // first head the scoring kernels cover (grid y covers the rest)
  float qscale;        // scale * log2(e)
};
size_t snapkv_ws_bytes(int B, int H, int N, int Lobs);
hipError_t launch_snapkv(const SnapkvParams& p, hipStream_t s);

// H2O prompt-phase compression (see h2o_prompt.hip).
struct H2oPromptParams {
  const void* q;       // [B][Hq][N][D] bf16
  const void* k;       // [B][Hkv][N][D]
  const void* v;
  void* k_out;         // [B][Hkv][budget][D]
  void* v_out;
  int* pos_out;        // [B][Hkv][budget]
  float* score_out;    // [B][Hkv][budget]
  float* rowstat;      // ws: [B][Hq][N] (max, 1/sum), log2 domain
  float* scores;       // [B][Hkv][N] accumulated scores (ws or the caller's buffer)
  int B, Hq, Hkv, D, N, budget, n_recent;
  float qscale;        // scale * log2(e)
};
size_t h2o_prompt_ws_bytes(int B, int Hq, int Hkv, int N);
hipError_t launch_h2o_prompt(const H2oPromptParams& p, void* ws, float* scores_all, hipStream_t s);

}  // namespace lcd
