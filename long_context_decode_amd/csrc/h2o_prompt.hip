// H2O prompt-phase compression for gfx950 ([KVC] "Heavy-Hitter Oracle (H2O) e a
// esparsidade de cauda pesada"): every prompt token's accumulated attention
// s_j = sum over the group's query heads h and rows t >= j of the causal softmax
// weight alpha_{h,t,j}, then the recent partition plus the heavy hitters, gathered
// into the layout of a full H2O cache.
//
// The score is a dense causal Q K^T over the whole prompt (N^2/2 * D * 2 flop per query
// head, twice: once for the row statistics, once for the column sums), so it runs on
// MFMA (v_mfma_f32_32x32x16_bf16) and is compute-bound: both kernels take the K tile as
// the A operand and the Q tile as the B operand, so the 32x32 result C[key][row] gives
// each lane 16 keys of one row (lane % 32), and the per-row softmax statistics of pass 1
// and the per-key sums of pass 2 need no cross-lane work inside the loop.
//
//   1. h2o_rowstats_kernel  per (256 prompt rows, query head; 128 at D = 256): Q rows
//                           held in registers, K streamed through LDS in blocks of 64
//                           keys, double buffered, over keys 0 .. last row; running (max,
//                           sum of 2^(x - max)) per row -> (M_t, 1/L_t).
//   2. h2o_colsum_kernel    per (256 keys, KV head; 128 at D = 256): K rows in registers,
//                           blocks of 64 rows of the group's query heads and their
//                           statistics streamed through LDS over rows t >= first key;
//                           weights 2^(x - M_t) / L_t summed per key in a fixed order -> s_j.
//   3. h2o_topk_kernel      per (batch row, KV head): exact selection of the heavy
//                           hitters on float32 s (radix select over range-relative
//                           bits, candidates streamed from memory), then an ascending,
//                           stable compaction by wave ballots; the recent tokens follow.
//   4. h2o_gather_kernel    kept K / V rows, positions and scores.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lcd_internal.h"

namespace lcd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile shapes at D <= 128, chosen by measurement on MI355X.
constexpr int kWaveTiles = 2;   // register tiles per wave
constexpr int kBlockTiles = 2;  // 32-row tiles per staged block

constexpr int kThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kMaxChunks = 256;  // prompt chunks of kTopkThreads positions: N <= 262144
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kHistCopies = 4;

// 2^x with the hardware instruction (v_exp_f32).  Arguments here are <= 0 (logit minus
// its row maximum); results below 2^-126, which the instruction may flush to zero, are
// negligible against the row sums they join.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline bf16x8 frag_global(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ inline bf16x8 frag_zero() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// LDS tile of 32 rows x D bf16, rows padded by 16 bytes (fragment reads, one row per
// lane, spread over the banks).
template <int D>
constexpr int tile_row_bytes() { return 2 * D + 16; }
template <int D>
constexpr int tile_bytes() { return 32 * tile_row_bytes<D>(); }

// Fragment of k-step s: row lane % 32, elements 16 s + 8 (lane / 32) .. + 7.
template <int D>
__device__ inline bf16x8 frag_lds(const char* lds, int s, int lane) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + (lane & 31) * tile_row_bytes<D>() +
                                                                    32 * s + 16 * (lane >> 5)));
}

// C register r of a 32x32 MFMA result: A-row 8 (r / 4) + 4 (lane / 32) + r % 4 (the key),
// B-column lane % 32 (the prompt row).
__device__ inline int c_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Keys (pass 1) or rows (pass 2) staged per iteration: two 32-row tiles (LDS buffers
// within 2 x 34 KiB, prefetch registers within 32 VGPRs).  With two register tiles per
// wave (D <= 128) every iteration gives each wave 32 MFMAs (16 at D = 256, each twice as
// long), enough to cover the global loads issued two iterations ahead.
template <int D>
constexpr int block_tiles() { return D == 256 ? 2 : kBlockTiles; }
template <int D>
constexpr int block_rows() { return 32 * block_tiles<D>(); }
template <int D>
constexpr int block_bytes() { return block_rows<D>() * tile_row_bytes<D>(); }
template <int D>
constexpr int block_pieces_per_thread() { return block_rows<D>() * D * 2 / 16 / kThreads; }

// Global -> registers for one block of rows (rows past n read as zero).
template <int D>
__device__ inline void block_load(const uint16_t* base, int row0, int n, uint4 (&r)[block_pieces_per_thread<D>()]) {
  constexpr int PPR = D * 2 / 16;  // pieces per row
#pragma unroll
  for (int i = 0; i < block_pieces_per_thread<D>(); ++i) {
    const int piece = i * kThreads + (int)threadIdx.x;
    const int row = piece / PPR, col = piece % PPR;
    r[i] = row0 + row < n ? *reinterpret_cast<const uint4*>(base + (size_t)(row0 + row) * D + col * 8)
                          : make_uint4(0, 0, 0, 0);
  }
}

// The same with every load issued (rows past n read row n - 1; callers mask them), for
// loops in which no branch may separate a load from its use: then the compiler's wait
// before the LDS store leaves the later prefetch in flight.
template <int D>
__device__ inline void block_load_all(const uint16_t* base, int row0, int n,
                                      uint4 (&r)[block_pieces_per_thread<D>()]) {
  constexpr int PPR = D * 2 / 16;  // pieces per row
#pragma unroll
  for (int i = 0; i < block_pieces_per_thread<D>(); ++i) {
    const int piece = i * kThreads + (int)threadIdx.x;
    const int row = min(row0 + piece / PPR, n - 1), col = piece % PPR;
    r[i] = *reinterpret_cast<const uint4*>(base + (size_t)row * D + col * 8);
  }
}

template <int D>
__device__ inline void block_store(char* lds, const uint4 (&r)[block_pieces_per_thread<D>()]) {
  constexpr int PPR = D * 2 / 16;
#pragma unroll
  for (int i = 0; i < block_pieces_per_thread<D>(); ++i) {
    const int piece = i * kThreads + (int)threadIdx.x;
    *reinterpret_cast<uint4*>(lds + (piece / PPR) * tile_row_bytes<D>() + (piece % PPR) * 16) = r[i];
  }
}

// Row (pass 1) or key (pass 2) tiles a wave keeps in registers: every fragment read from
// LDS then feeds that many MFMAs, which keeps the LDS reads below the MFMA rate.
template <int D>
constexpr int wave_tiles() { return D == 256 ? 1 : kWaveTiles; }

// ------------------------------------------------------------------ 1. row statistics
// Workgroup: 4 * 32 * TW prompt rows of one query head (Q fragments in registers).
// Iteration: a block of keys staged in LDS; each wave multiplies its rows with every key
// tile of the block (MFMA), then folds each tile into its rows' running (max, sum).
template <int D>
__global__ void __launch_bounds__(kThreads, 2) h2o_rowstats_kernel(H2oPromptParams p) {
  constexpr int KS = D / 16;  // MFMA k-steps
  constexpr int BT = block_tiles<D>(), BR = block_rows<D>();
  constexpr int TW = wave_tiles<D>();
  constexpr int WR = 4 * 32 * TW;  // rows per workgroup
  __shared__ __attribute__((aligned(16))) char kblk[2][block_bytes<D>()];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = (int)gridDim.x - 1 - (int)blockIdx.x;  // longest causal ranges first
  const int h = blockIdx.y, b = blockIdx.z, g = h / (p.Hq / p.Hkv);
  const int r0 = blk * WR + wave * 32 * TW;  // the wave's first row
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)b * p.Hq + h) * p.N * D;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k) + ((size_t)b * p.Hkv + g) * p.N * D;

  bf16x8 qf[TW][KS];
  float m[TW], l[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int row = r0 + i * 32 + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[i][s] = row < p.N ? frag_global(Q + (size_t)row * D + 16 * s + 8 * (lane >> 5)) : frag_zero();
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  const int n_keys = min(p.N, blk * WR + WR);
  const int n_blocks = (n_keys + BR - 1) / BR;
  // blocks are loaded two iterations ahead into alternating register sets (named, so
  // they stay in registers), stored to LDS one iteration ahead
  uint4 rawA[block_pieces_per_thread<D>()], rawB[block_pieces_per_thread<D>()];
  auto step = [&](auto all, int kb, uint4 (&load_into)[block_pieces_per_thread<D>()],
                  const uint4 (&store_from)[block_pieces_per_thread<D>()]) {
    if constexpr (decltype(all)::value)
      block_load_all<D>(K, (kb + 2) * BR, p.N, load_into);  // kb + 2 < n_blocks: no branch
    else if (kb + 2 < n_blocks)
      block_load<D>(K, (kb + 2) * BR, p.N, load_into);
    __syncthreads();  // block kb is in kblk[kb & 1]; every wave is done with block kb - 1
    const char* kl = kblk[kb & 1];
    const int k0 = kb * BR;
    // Blocks wholly past the wave's last row are skipped (a wave-uniform test per block).
    // Otherwise every tile is multiplied, with no test between the MFMAs so that the LDS
    // reads and MFMAs of the block pipeline; key tiles past a row tile's diagonal (at
    // most one block per wave) are masked to -inf by the fold like the diagonal itself.
    if (k0 <= r0 + 32 * TW - 1) {
      f32x16 acc[BT][TW];
#pragma unroll
      for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int i = 0; i < TW; ++i) acc[t][i] = f32x16{};
      // the next k-step's fragments are read while this step's MFMAs run
      bf16x8 fa[2][BT];
#pragma unroll
      for (int t = 0; t < BT; ++t) fa[0][t] = frag_lds<D>(kl + t * tile_bytes<D>(), 0, lane);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) {
#pragma unroll
          for (int t = 0; t < BT; ++t) fa[(s + 1) & 1][t] = frag_lds<D>(kl + t * tile_bytes<D>(), s + 1, lane);
        }
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
          for (int i = 0; i < TW; ++i)
            acc[t][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][t], qf[i][s], acc[t][i], 0, 0, 0);
      }
      // order: the reads of k-step s + 1 go ahead of the MFMAs of k-step s
      __builtin_amdgcn_sched_group_barrier(0x100, BT, 0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, BT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, BT * TW, 0);
      }
      // fold the block into each row's (max, sum): the maximum on the raw products (the
      // scale is positive), masked keys set to -inf, then 2^(acc * scale - max)
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int ri = r0 + i * 32;
        float bm = -INFINITY;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          const int kt0 = k0 + t * 32;
          if (kt0 + 31 > ri) {  // some key of the tile is past some row: key <= row <=> c_row <= row - first key
            const int dlt = ri + (lane & 31) - kt0;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (c_row(r, lane) > dlt) acc[t][i][r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) bm = fmaxf(bm, acc[t][i][r]);
        }
        const float mn = fmaxf(m[i], bm * p.qscale);
        if (mn > -INFINITY) {
          float add = 0.f;
#pragma unroll
          for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) add += exp2_hw(fmaf(acc[t][i][r], p.qscale, -mn));
          l[i] = l[i] * exp2_hw(m[i] - mn) + add;
          m[i] = mn;
        }
      }
    }
    if (kb + 1 < n_blocks) block_store<D>(kblk[(kb + 1) & 1], store_from);
  };
  block_load<D>(K, 0, p.N, rawA);
  if (n_blocks > 1) block_load<D>(K, BR, p.N, rawB);
  block_store<D>(kblk[0], rawA);
  int kb = 0;
  // loop split: while both steps prefetch a block that exists, the prefetches are unconditional
  for (; kb + 3 < n_blocks; kb += 2) {
    step(std::true_type{}, kb, rawA, rawB);
    step(std::true_type{}, kb + 1, rawB, rawA);
  }
  for (; kb < n_blocks; kb += 2) {
    step(std::false_type{}, kb, rawA, rawB);
    if (kb + 1 >= n_blocks) break;
    step(std::false_type{}, kb + 1, rawB, rawA);
  }
  // lanes l and l ^ 32 hold the same row (the two halves of every key tile)
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const float mo = __shfl_xor(m[i], 32, 64), lo = __shfl_xor(l[i], 32, 64);
    const float M = fmaxf(m[i], mo);
    const float Lsum = (m[i] > -INFINITY ? l[i] * exp2f(m[i] - M) : 0.f) + (mo > -INFINITY ? lo * exp2f(mo - M) : 0.f);
    const int row = r0 + i * 32 + (lane & 31);
    if (lane < 32 && row < p.N) {
      float2* st = reinterpret_cast<float2*>(p.rowstat) + ((size_t)b * p.Hq + h) * p.N + row;
      *st = make_float2(M, 1.f / Lsum);
    }
  }
}

// ------------------------------------------------------------------ 2. column sums
// Workgroup: 4 * 32 * TW keys of one KV head (K fragments in registers).
// Iteration: a block of prompt rows of one query head of the group (Q rows and their
// statistics staged in LDS), rows from the workgroup's first key to the end; each wave
// adds the weights 2^(x - M_t) / L_t of its keys over the block's rows.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) h2o_colsum_kernel(H2oPromptParams p) {
  constexpr int KS = D / 16;
  constexpr int BT = block_tiles<D>(), BR = block_rows<D>();
  constexpr int TW = wave_tiles<D>();
  constexpr int WK = 4 * 32 * TW;  // keys per workgroup
  __shared__ __attribute__((aligned(16))) char qblk[2][block_bytes<D>()];
  __shared__ float2 qstat[2][BR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int key0 = kb * WK + wave * 32 * TW;  // the wave's first key
  const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k) + ((size_t)b * p.Hkv + g) * p.N * D;
  bf16x8 kf[TW][KS];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int key = key0 + i * 32 + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[i][s] = key < p.N ? frag_global(K + (size_t)key * D + 16 * s + 8 * (lane >> 5)) : frag_zero();
  }
  float col[TW][16];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) col[i][r] = 0.f;

  // units: (row block, head j) from the row block holding the workgroup's first key
  const int rb_first = (kb * WK) / BR;
  const int n_rb = (p.N + BR - 1) / BR;
  const int units = (n_rb - rb_first) * G;
  // units are loaded two iterations ahead into alternating register sets (named, so
  // they stay in registers), stored to LDS one iteration ahead
  constexpr int P = block_pieces_per_thread<D>();
  uint4 rawA[P], rawB[P];
  float2 sA = make_float2(0.f, 0.f), sB = make_float2(0.f, 0.f);
  auto load_unit = [&](int u, uint4 (&raw)[P], float2& sraw) {
    const int row0 = (rb_first + u / G) * BR;
    const size_t bh = (size_t)b * p.Hq + g * G + u % G;
    block_load<D>(reinterpret_cast<const uint16_t*>(p.q) + bh * p.N * D, row0, p.N, raw);
    if ((int)threadIdx.x < BR)
      sraw = row0 + (int)threadIdx.x < p.N ? reinterpret_cast<const float2*>(p.rowstat)[bh * p.N + row0 + threadIdx.x]
                                           : make_float2(0.f, 0.f);
  };
  // every load issued: rows past N read row N - 1 and get the statistics (+inf, 0), so
  // their weights 2^(x - inf) * 0 are 0
  auto load_unit_all = [&](int u, uint4 (&raw)[P], float2& sraw) {
    const int row0 = (rb_first + u / G) * BR;
    const size_t bh = (size_t)b * p.Hq + g * G + u % G;
    block_load_all<D>(reinterpret_cast<const uint16_t*>(p.q) + bh * p.N * D, row0, p.N, raw);
    const int row = row0 + min((int)threadIdx.x, BR - 1);
    const float2 st = reinterpret_cast<const float2*>(p.rowstat)[bh * p.N + min(row, p.N - 1)];
    sraw = row < p.N ? st : make_float2(INFINITY, 0.f);
  };
  auto store_unit = [&](int buf, const uint4 (&raw)[P], float2 sraw) {
    block_store<D>(qblk[buf], raw);
    if ((int)threadIdx.x < BR) qstat[buf][threadIdx.x] = sraw;
  };
  auto step = [&](auto all, int u, uint4 (&load_into)[P], float2& s_into, const uint4 (&store_from)[P],
                  float2 s_from) {
    if constexpr (decltype(all)::value)
      load_unit_all(u + 2, load_into, s_into);  // u + 2 < units: no branch
    else if (u + 2 < units)
      load_unit(u + 2, load_into, s_into);
    __syncthreads();  // unit u is in buffer u & 1; every wave is done with unit u - 1
    const int row0 = (rb_first + u / G) * BR;
    const char* ql = qblk[u & 1];
    // Row blocks wholly before the wave's first key are skipped (a wave-uniform test per
    // block); otherwise every tile is multiplied with no test between the MFMAs, and the
    // fold masks rows before a key (the diagonal tiles and any tile before it).
    if (row0 + BR - 1 >= key0) {
      f32x16 acc[BT][TW];
#pragma unroll
      for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int i = 0; i < TW; ++i) acc[t][i] = f32x16{};
      bf16x8 fb[2][BT];
#pragma unroll
      for (int t = 0; t < BT; ++t) fb[0][t] = frag_lds<D>(ql + t * tile_bytes<D>(), 0, lane);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) {
#pragma unroll
          for (int t = 0; t < BT; ++t) fb[(s + 1) & 1][t] = frag_lds<D>(ql + t * tile_bytes<D>(), s + 1, lane);
        }
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
          for (int i = 0; i < TW; ++i)
            acc[t][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i][s], fb[s & 1][t], acc[t][i], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, BT, 0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, BT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, BT * TW, 0);
      }
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        const float2 st = qstat[u & 1][t * 32 + (lane & 31)];  // rows past N carry (0, 0) or (+inf, 0): weight 0
        const int rt0 = row0 + t * 32;
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const int ki = key0 + i * 32;
          if (rt0 >= ki + 31) {  // every key of the tile is <= every row (wave-uniform)
#pragma unroll
            for (int r = 0; r < 16; ++r) col[i][r] = fmaf(exp2_hw(fmaf(acc[t][i][r], p.qscale, -st.x)), st.y, col[i][r]);
          } else {  // key <= row <=> c_row <= row - first key (none where the tile is wholly before)
            const int dlt = rt0 + (lane & 31) - ki;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = exp2_hw(fmaf(acc[t][i][r], p.qscale, -st.x));
              col[i][r] = c_row(r, lane) <= dlt ? fmaf(e, st.y, col[i][r]) : col[i][r];
            }
          }
        }
      }
    }
    if (u + 1 < units) store_unit((u + 1) & 1, store_from, s_from);
  };
  load_unit(0, rawA, sA);
  if (units > 1) load_unit(1, rawB, sB);
  store_unit(0, rawA, sA);
  int u = 0;
  // loop split: while both steps prefetch a unit that exists, the prefetches are unconditional
  for (; u + 3 < units; u += 2) {
    step(std::true_type{}, u, rawA, sA, rawB, sB);
    step(std::true_type{}, u + 1, rawB, sB, rawA, sA);
  }
  for (; u < units; u += 2) {
    step(std::false_type{}, u, rawA, sA, rawB, sB);
    if (u + 1 >= units) break;
    step(std::false_type{}, u + 1, rawB, sB, rawA, sA);
  }
  // lanes of one half (lane / 32 fixed) hold the same 16 keys for different rows
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = col[i][r];
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) x += __shfl_xor(x, off, 64);
      col[i][r] = x;
    }
  if ((lane & 31) == 0) {
    float* sc = p.scores + ((size_t)b * p.Hkv + g) * p.N;
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + i * 32 + c_row(r, lane);
        if (key < p.N) sc[key] = col[i][r];
      }
  }
}

// ------------------------------------------------------------------ 3. selection
// Exclusive scan over the 1024 threads (per-wave shuffles, one barrier, every wave
// adds the totals of the waves before it); *total receives the sum.  Callers alternate
// the two halves of `buf` between consecutive scans.
__device__ inline int topk_scan(int v, int* buf, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int t = buf[w];
    before += w < wave ? t : 0;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// One workgroup per (batch row, KV head).  Candidates are positions [0, Np); chunk c
// covers positions c * 1024 .. c * 1024 + 1023 with position c * 1024 + threadIdx.x
// per thread, so every pass over the scores reads them coalesced.  Selection: the
// k-th largest float32 score T by radix select over v = bits - min(bits) (scores are
// >= 0, so bits order like values); kept = v > T plus the first positions with v == T
// up to k.  Compaction: per (chunk, wave) counts of both kinds, one scan over them,
// then ballots place each wave's kept positions in ascending order.
__global__ void __launch_bounds__(kTopkThreads) h2o_topk_kernel(H2oPromptParams p) {
  // the radix histogram, then (once the threshold is known) the per-piece counts
  static_assert(2 * kMaxChunks * kTopkWaves <= kHistCopies * kBins, "counts overlay the histogram");
  __shared__ int hist[kHistCopies * kBins];
  __shared__ int scan_buf[2][kTopkWaves];
  __shared__ uint32_t wmin[kTopkWaves], wmax[kTopkWaves];
  __shared__ int s_digit, s_krem;
  int* cnt_gt = hist;
  int* cnt_eq = hist + kMaxChunks * kTopkWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bg = blockIdx.x;
  const float* sc = p.scores + bg * p.N;
  int* idx = p.pos_out + bg * p.budget;
  const int N = p.N;
  const int kept_rows = min(p.budget, N);
  const int n_recent = min(p.n_recent, kept_rows);
  const int Np = N - n_recent;              // candidates of the heavy partition
  const int k = kept_rows - n_recent;       // heavy hitters kept (<= Np)
  const int chunks = (Np + kTopkThreads - 1) / kTopkThreads;
  int total;

  if (k >= Np) {  // every candidate is kept
    for (int i = threadIdx.x; i < Np; i += kTopkThreads) idx[i] = i;
  } else if (k > 0) {
    uint32_t lmin = 0xffffffffu, lmax = 0u;
    for (int c = 0; c < chunks; ++c) {
      const int i = c * kTopkThreads + threadIdx.x;
      if (i < Np) {
        const uint32_t u = __float_as_uint(sc[i]);
        lmin = min(lmin, u);
        lmax = max(lmax, u);
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      lmin = min(lmin, (uint32_t)__shfl_xor((int)lmin, off, 64));
      lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, off, 64));
    }
    if (lane == 0) {
      wmin[wave] = lmin;
      wmax[wave] = lmax;
    }
    __syncthreads();
    uint32_t umin = 0xffffffffu, umax = 0u;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      umin = min(umin, wmin[w]);
      umax = max(umax, wmax[w]);
    }
    const uint32_t range = umax - umin;
    const int Lb = range ? 32 - __clz((int)range) : 0;
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int hi = Lb; hi > 0; hi -= kDigitBits) {
      const int shift = hi > kDigitBits ? hi - kDigitBits : 0;
      const int bits = hi - shift;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = threadIdx.x; i < kHistCopies * kBins; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      int* hcopy = hist + (threadIdx.x & (kHistCopies - 1)) * kBins;
      for (int c = 0; c < chunks; ++c) {
        const int i = c * kTopkThreads + threadIdx.x;
        if (i < Np) {
          const uint32_t v = __float_as_uint(sc[i]) - umin;
          if ((v & mask) == prefix) atomicAdd(&hcopy[(v >> shift) & dmask], 1);
        }
      }
      __syncthreads();
      const int nb = 1 << bits;
      int cb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int bin = nb - 1 - (2 * (int)threadIdx.x + e);
        int v = 0;
        if (bin >= 0)
          for (int q = 0; q < kHistCopies; ++q) v += hist[q * kBins + bin];
        cb[e] = v;
      }
      const int before = topk_scan(cb[0] + cb[1], scan_buf[0], &total);
      if (before < krem && before + cb[0] + cb[1] >= krem) {
        const int e = before + cb[0] >= krem ? 0 : 1;
        s_digit = nb - 1 - (2 * (int)threadIdx.x + e);
        s_krem = krem - before - (e ? cb[0] : 0);
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= dmask << shift;
      krem = s_krem;
      __syncthreads();
    }
    const uint32_t T = prefix;  // v of the k-th largest score
    const int take_eq = krem;   // values equal to T that are kept
    // per (chunk, wave) counts of v > T and v == T
    for (int c = 0; c < chunks; ++c) {
      const int i = c * kTopkThreads + threadIdx.x;
      uint32_t v = 0;
      bool in = i < Np;
      if (in) v = __float_as_uint(sc[i]) - umin;
      const unsigned long long bgt = __ballot(in && v > T), beq = __ballot(in && v == T);
      if (lane == 0) {
        cnt_gt[c * kTopkWaves + wave] = __popcll(bgt);
        cnt_eq[c * kTopkWaves + wave] = __popcll(beq);
      }
    }
    __syncthreads();
    // exclusive prefix of both counts over (chunk, wave) in order: each thread sums a
    // contiguous run of the entries, then one scan over the threads
    const int n_ent = chunks * kTopkWaves;
    const int per = (n_ent + kTopkThreads - 1) / kTopkThreads;
    const int e0 = threadIdx.x * per;
    int sg = 0, se = 0;
    for (int e = e0; e < min(e0 + per, n_ent); ++e) {
      sg += cnt_gt[e];
      se += cnt_eq[e];
    }
    int run_eq = topk_scan(se, scan_buf[1], &total);
    int run_gt = topk_scan(sg, scan_buf[0], &total);
    __syncthreads();
    // turn the counts into the output offset of each (chunk, wave) piece: kept before
    // it = gt before + min(eq before, take_eq)
    for (int e = e0; e < min(e0 + per, n_ent); ++e) {
      const int g_here = cnt_gt[e], e_here = cnt_eq[e];
      cnt_gt[e] = run_gt + min(run_eq, take_eq);  // output offset of the piece
      cnt_eq[e] = run_eq;                          // equal values before the piece
      run_gt += g_here;
      run_eq += e_here;
    }
    __syncthreads();
    for (int c = 0; c < chunks; ++c) {
      const int i = c * kTopkThreads + threadIdx.x;
      uint32_t v = 0;
      bool in = i < Np;
      if (in) v = __float_as_uint(sc[i]) - umin;
      const bool gt = in && v > T, eq = in && v == T;
      const unsigned long long beq = __ballot(eq);
      const int eq_rank = cnt_eq[c * kTopkWaves + wave] + __popcll(beq & ((1ull << lane) - 1ull));
      const bool keep = gt || (eq && eq_rank < take_eq);
      const unsigned long long bk = __ballot(keep);
      if (keep) idx[cnt_gt[c * kTopkWaves + wave] + __popcll(bk & ((1ull << lane) - 1ull))] = i;
    }
  }
  for (int t = threadIdx.x; t < n_recent; t += kTopkThreads) idx[k + t] = Np + t;
}

// ------------------------------------------------------------------ 4. gather
template <int D>
__global__ void __launch_bounds__(kThreads) h2o_gather_kernel(H2oPromptParams p) {
  const size_t bg = blockIdx.y;
  const int rows = min(p.budget, p.N);
  constexpr int PPR = D * 2 / 16;
  const int* idx = p.pos_out + bg * p.budget;
  const char* k = reinterpret_cast<const char*>(p.k) + bg * p.N * D * 2;
  const char* v = reinterpret_cast<const char*>(p.v) + bg * p.N * D * 2;
  char* ko = reinterpret_cast<char*>(p.k_out) + bg * p.budget * D * 2;
  char* vo = reinterpret_cast<char*>(p.v_out) + bg * p.budget * D * 2;
  const int total = rows * PPR;
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < total; e += gridDim.x * kThreads) {
    const int row = e / PPR, c = e % PPR;
    const int src = idx[row];
    const size_t so = (size_t)src * D * 2 + (size_t)c * 16, dst = (size_t)row * D * 2 + (size_t)c * 16;
    *reinterpret_cast<uint4*>(ko + dst) = *reinterpret_cast<const uint4*>(k + so);
    *reinterpret_cast<uint4*>(vo + dst) = *reinterpret_cast<const uint4*>(v + so);
    if (c == 0) {
      const float s = p.scores[bg * p.N + src];
      p.score_out[bg * p.budget + row] = s;
    }
  }
}

template <int D>
hipError_t launch_d(const H2oPromptParams& p, hipStream_t s) {
  constexpr int W = 4 * 32 * wave_tiles<D>();  // rows / keys per workgroup
  const int wgs = (p.N + W - 1) / W;
  hipLaunchKernelGGL(h2o_rowstats_kernel<D>, dim3(wgs, p.Hq, p.B), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(h2o_colsum_kernel<D>, dim3(wgs, p.Hkv, p.B), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(h2o_topk_kernel, dim3(p.B * p.Hkv), dim3(kTopkThreads), 0, s, p);
  const int rows = p.budget < p.N ? p.budget : p.N;
  const int blocks = (rows * (D * 2 / 16) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(h2o_gather_kernel<D>, dim3(blocks < 1024 ? blocks : 1024, p.B * p.Hkv), dim3(kThreads), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t h2o_prompt_ws_bytes(int B, int Hq, int Hkv, int N) {
  const size_t stats = round256((size_t)B * Hq * N * 2 * sizeof(float));
  const size_t scores = round256((size_t)B * Hkv * N * sizeof(float));
  return stats + scores;
}

hipError_t launch_h2o_prompt(const H2oPromptParams& in, void* ws, float* scores_all, hipStream_t s) {
  H2oPromptParams p = in;
  char* w = static_cast<char*>(ws);
  p.rowstat = reinterpret_cast<float*>(w);
  p.scores = scores_all ? scores_all
                        : reinterpret_cast<float*>(w + round256((size_t)p.B * p.Hq * p.N * 2 * sizeof(float)));
  switch (p.D) {
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    case 256: return launch_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lcd
