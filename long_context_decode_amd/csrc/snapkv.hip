// SnapKV prefill compression for gfx950 ([KVC] "SnapKV e a seleção de contexto no
// prefill"): observation-window attention scores, their mean over the window rows,
// 1-D pooling, per-head top-k and the gather of the kept K/V rows.
//
// Pipeline on one stream, no host round trip:
//   1. snapkv_rowstats   per (512-key tile, head, row): logits of the L_obs window
//                        queries against the tile's keys on MFMA (bf16 in, fp32
//                        accumulate), causal mask, per-row (max, sum of 2^(x-max)).
//   2. snapkv_colscore   per tile of prefix keys: merges the head's tile statistics into
//                        (M_t, 1/L_t), then the same MFMA product, weights
//                        2^(x - M_t) / L_t summed over the window rows -> s_i
//                        (times 1/L_obs: the mean over the window).
//   3. snapkv_select     one workgroup per head: pooled scores (kernel_size > 9: pooled
//                        by snapkv_pool_kernel first), radix select (11-bit
//                        digits over the range-relative float bits; scores are >= 0,
//                        so the bit patterns order like the values) of the k-th
//                        largest, then a stable compaction that lists the kept
//                        positions in ascending order (ties at the threshold keep the
//                        lower indices), followed by the observation window.
//   4. snapkv_gather     copy the kept K and V rows.
// The contraction is L_obs x N x D per head: 32 rows against every key, i.e. 32 flops
// per byte of K read.  It is a dense product, so it runs on MFMA, but it remains
// HBM-bound (K is read twice: steps 1 and 2).
#include <hip/hip_runtime.h>

#include "lcd_internal.h"

namespace lcd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveBlocks = 4;  // 32-key blocks per wave in the scoring kernels (by measurement)
constexpr int kTileKeys = 4 * kWaveBlocks * 32;  // keys per scoring workgroup

constexpr int kSelectThreads = 1024;

__device__ inline bf16x8 load_frag(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ inline bf16x8 zero_frag() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Observation-query fragments of row block rb: lane l holds row rb*32 + l%32, elements
// 16*s + 8*(l/32) .. +7 of step s.  Rows past L_obs are zero.
template <int D>
__device__ inline void load_q_frags(const uint16_t* q, int Lobs, int rb, int lane, bf16x8 (&qf)[D / 16]) {
  const int row = rb * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = row < Lobs ? load_frag(q + (size_t)row * D + 16 * s + 8 * (lane >> 5)) : zero_frag();
}

// K rows are staged through LDS so that global loads are fully coalesced: a 32-key
// block is read in column chunks of CW = min(D, 128) elements as 16-byte pieces, 64
// consecutive pieces per load instruction, then the MFMA fragments of that chunk are
// read back from LDS.  Rows are padded by 16 bytes so that the fragment reads (one
// row per lane) spread over the LDS banks.
template <int D>
constexpr int chunk_w() { return D < 128 ? D : 128; }
template <int D>
constexpr int lds_row_bytes() { return chunk_w<D>() * 2 + 16; }
template <int D>
constexpr int block_lds_bytes() { return 32 * lds_row_bytes<D>(); }
template <int D>
constexpr int chunk_pieces() { return chunk_w<D>() / 16; }  // 16-byte pieces per lane per chunk

// NT: non-temporal loads (the last read of these rows); otherwise plain loads, which
// leave the rows in the caches for the second pass.
template <int D, bool NT>
__device__ inline void chunk_load(const uint16_t* k, int N, int key0, int c, int lane,
                                  u32x4 (&raw)[chunk_pieces<D>()]) {
  constexpr int PPR = chunk_w<D>() * 2 / 16;  // pieces per row of the chunk
#pragma unroll
  for (int i = 0; i < chunk_pieces<D>(); ++i) {
    const int piece = i * 64 + lane;
    const int row = piece / PPR, col = piece % PPR;
    const int key = key0 + row;
    const u32x4* src = reinterpret_cast<const u32x4*>(k + (size_t)key * D + c * chunk_w<D>() + col * 8);
    if (key < N)
      raw[i] = NT ? __builtin_nontemporal_load(src) : *src;
    else
      raw[i] = u32x4{0, 0, 0, 0};
  }
}

template <int D>
__device__ inline void chunk_store_lds(char* lds, int lane, const u32x4 (&raw)[chunk_pieces<D>()]) {
  constexpr int PPR = chunk_w<D>() * 2 / 16;
#pragma unroll
  for (int i = 0; i < chunk_pieces<D>(); ++i) {
    const int piece = i * 64 + lane;
    *reinterpret_cast<u32x4*>(lds + (piece / PPR) * lds_row_bytes<D>() + (piece % PPR) * 16) = raw[i];
  }
}

// Fragment s (within the chunk) of row lane%32: chunk elements 16*s + 8*(lane/32) .. +7.
template <int D>
__device__ inline void chunk_frags_lds(const char* lds, int lane, bf16x8 (&kf)[chunk_w<D>() / 16]) {
#pragma unroll
  for (int s = 0; s < chunk_w<D>() / 16; ++s)
    kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + (lane & 31) * lds_row_bytes<D>() +
                                                                       32 * s + 16 * (lane >> 5)));
}

// LDS accesses of one wave execute in program order; this keeps the compiler from
// moving them across the hand-off between the staging store and the fragment reads.
__device__ inline void wave_lds_order() { __asm__ volatile("" ::: "memory"); }

// Result element r of a 32x32 MFMA tile sits at A-row 8*(r/4) + 4*(lane/32) + r%4 and
// B-column lane%32.
__device__ inline int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------- window queries
// The observation rows are RB blocks of 32.  Up to two blocks (L_obs <= 64) the query
// fragments stay in registers for the whole pass; beyond that the workgroup stages the
// window queries in LDS once (rows padded by 16 bytes, zero past L_obs) and each K block
// loops over the row blocks, reading their fragments from LDS, RG blocks' accumulators at
// a time (RG = min(RB, 4)).
template <int D>
constexpr int q_row_bytes() { return 2 * D + 16; }

template <int D, int RB>
struct QRows {
  static constexpr bool kRegs = RB <= 2;
  static constexpr int kRG = RB < 4 ? RB : 4;  // row blocks whose accumulators are live at once
  static constexpr int kLdsBytes = kRegs ? 16 : RB * 32 * q_row_bytes<D>();
};

// Chunks of K a scoring wave keeps in flight (two while the window queries fit registers;
// wider windows keep one so as not to lose occupancy), and the occupancy asked of the
// compiler for the narrow shapes (three waves per SIMD, which the second set fits into).
template <int D, int RB>
constexpr int prefetch_depth() { return QRows<D, RB>::kRegs && D <= 128 ? 2 : 1; }
template <int D, int RB>
constexpr int scoring_min_waves() { return RB == 1 && D <= 128 ? 3 : 1; }

template <int D, int RB>
__device__ inline void stage_q_rows(const uint16_t* q, int Lobs, char* qs) {
  constexpr int PPR = D * 2 / 16;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < RB * 32 * PPR; i += 256) {
    const int row = i / PPR, col = i % PPR;
    const u32x4 v = row < Lobs ? *reinterpret_cast<const u32x4*>(q + (size_t)row * D + col * 8) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(qs + row * q_row_bytes<D>() + col * 16) = v;
  }
}

// Fragment of row block rb, k-step s (over the whole row): lane l holds row rb * 32 + l % 32,
// elements 16 s + 8 (l / 32) .. + 7.
template <int D>
__device__ inline bf16x8 q_frag_lds(const char* qs, int rb, int s, int lane) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qs + (rb * 32 + (lane & 31)) * q_row_bytes<D>() +
                                                                     32 * s + 16 * (lane >> 5)));
}

// ---------------------------------------------------------------------------- 1. rowstats
template <int D, int RB>
__global__ void __launch_bounds__(256, (scoring_min_waves<D, RB>())) snapkv_rowstats_kernel(SnapkvParams p) {
  using QR = QRows<D, RB>;
  constexpr int R = RB * 32, RG = QR::kRG;
  __shared__ float sm[4][R], sl[4][R];
  __shared__ __attribute__((aligned(16))) char stage[4][block_lds_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char qs[QR::kLdsBytes];
  const int tile = blockIdx.x, h = p.h0 + blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)b * p.H + h;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q_obs) + bh * p.Lobs * D;
  const uint16_t* k = reinterpret_cast<const uint16_t*>(p.k) + bh * (size_t)p.N * D;
  const int last_visible0 = p.N - p.Lobs;  // row t sees keys <= last_visible0 + t
  const int wkey0 = tile * kTileKeys + wave * kWaveBlocks * 32;
  bf16x8 qf[QR::kRegs ? RB : 1][D / 16];
  if constexpr (QR::kRegs) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) load_q_frags<D>(q, p.Lobs, rb, lane, qf[rb]);
  } else {
    stage_q_rows<D, RB>(q, p.Lobs, qs);
    __syncthreads();
  }
  auto qfrag = [&](int rb, int s) {
    if constexpr (QR::kRegs) return qf[rb][s];
    else return q_frag_lds<D>(qs, rb, s, lane);
  };
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
  }
  constexpr int NC = D / chunk_w<D>();
  constexpr int FS = chunk_w<D>() / 16;  // fragments per chunk
  static_assert(NC == 1 || RG == RB, "a row of two column chunks keeps every row block's accumulator");
  // fold of row block rb's 32 x 32 tile (acc[r]: key key0 + mfma_row(r), row rb * 32 + lane % 32)
  // into the row's running (max, sum of 2^(x - max)), the max kept on the raw products (the
  // scale is positive) and each weight one FMA and one exp2.  Keys past the prompt or after
  // the row's own position are masked, tested only on tiles that reach either.
  auto fold = [&](int rb, const f32x16& acc, int key0) {
    const int t = rb * 32 + (lane & 31);
    float a[16];
    const bool edge = key0 + 31 >= p.N || key0 + 31 > last_visible0;  // wave-uniform
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + mfma_row(r, lane);
        a[r] = key < p.N && key <= last_visible0 + t ? acc[r] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = acc[r];
    }
    float bm = a[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bm = fmaxf(bm, a[r]);
    const float mn = fmaxf(m[rb], bm);  // raw units
    if (mn > -INFINITY && t < p.Lobs) {
      const float off = -mn * p.qscale;
      float add = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) add += exp2f(fmaf(a[r], p.qscale, off));
      l[rb] = fmaf(l[rb], exp2f((m[rb] - mn) * p.qscale), add);
      m[rb] = mn;
    }
  };
  // the wave's kWaveBlocks * NC chunks in order, PF in flight: chunk i + PF is requested
  // into the register set that chunk i leaves when it moves to LDS
  constexpr int T = kWaveBlocks * NC, PF = prefetch_depth<D, RB>();
  u32x4 raw[PF][chunk_pieces<D>()];
#pragma unroll
  for (int i = 0; i < PF && i < T; ++i) chunk_load<D, true>(k, p.N, wkey0 + 32 * (i / NC), i % NC, lane, raw[i]);
#pragma unroll
  for (int blk = 0; blk < kWaveBlocks; ++blk) {
    const int key0 = wkey0 + blk * 32;
    if (key0 >= p.N) break;  // wave-uniform
    f32x16 acc[RG];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = blk * NC + c;
      chunk_store_lds<D>(stage[wave], lane, raw[i % PF]);
      if (i + PF < T) chunk_load<D, true>(k, p.N, wkey0 + 32 * ((i + PF) / NC), (i + PF) % NC, lane, raw[i % PF]);
      wave_lds_order();
      bf16x8 kf[FS];
      chunk_frags_lds<D>(stage[wave], lane, kf);
      wave_lds_order();
#pragma unroll
      for (int g0 = 0; g0 < RB; g0 += RG) {
        if (NC == 1 || c == 0) {
#pragma unroll
          for (int r = 0; r < RG; ++r) acc[r] = f32x16{};
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
#pragma unroll
          for (int s = 0; s < FS; ++s)
            acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qfrag(g0 + r, c * FS + s), acc[r], 0, 0, 0);
        }
        if (NC == 1 || c == NC - 1) {
#pragma unroll
          for (int r = 0; r < RG; ++r) fold(g0 + r, acc[r], key0);
        }
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] *= p.qscale;  // log2 units from here on (the -inf of an empty row stays -inf)
    // lanes l and l ^ 32 hold the same row
    const float mo = __shfl_xor(m[rb], 32, 64), lo = __shfl_xor(l[rb], 32, 64);
    const float mm = fmaxf(m[rb], mo);
    float ll = 0.f;
    if (mm > -INFINITY) ll = l[rb] * exp2f(m[rb] - mm) + lo * exp2f(mo - mm);
    if (lane < 32) {
      sm[wave][rb * 32 + lane] = mm;
      sl[wave][rb * 32 + lane] = ll;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < R; t += 256) {
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm[w][t]);
    float ll = 0.f;
    if (mm > -INFINITY)
      for (int w = 0; w < 4; ++w) ll += sl[w][t] * exp2f(sm[w][t] - mm);
    float* out = p.rowstat + ((bh * p.tiles + tile) * R + t) * 2;
    out[0] = mm;
    out[1] = ll;
  }
}

// ---------------------------------------------------------------------------- 2. colscore
template <int D, int RB>
__global__ void __launch_bounds__(256, (scoring_min_waves<D, RB>())) snapkv_colscore_kernel(SnapkvParams p) {
  using QR = QRows<D, RB>;
  constexpr int R = RB * 32, RG = QR::kRG;
  __shared__ float sM[R], sI[R];
  __shared__ __attribute__((aligned(16))) char stage[4][block_lds_bytes<D>()];
  __shared__ __attribute__((aligned(16))) char qs[QR::kLdsBytes];
  // Walk K in the reverse of the row-statistics pass: the rows read last there are the
  // likeliest still cached.
  const int tile = gridDim.x - 1 - blockIdx.x, h = p.h0 + (int)(gridDim.y - 1 - blockIdx.y),
            b = gridDim.z - 1 - blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)b * p.H + h;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q_obs) + bh * p.Lobs * D;
  const uint16_t* k = reinterpret_cast<const uint16_t*>(p.k) + bh * (size_t)p.N * D;
  const int Np = p.N - p.Lobs;  // prefix keys: visible to every observation row
  const float inv_rows = 1.f / (float)p.Lobs;
  const int wkey0 = tile * kTileKeys + wave * kWaveBlocks * 32;
  // the wave's first K chunk is requested before the statistics merge below, so that its
  // latency overlaps the merge's loads (keys past the prefix load nothing)
  constexpr int NCK = D / chunk_w<D>(), T = kWaveBlocks * NCK, PF = prefetch_depth<D, RB>();
  u32x4 raw[PF][chunk_pieces<D>()];
#pragma unroll
  for (int i = 0; i < PF && i < T; ++i) chunk_load<D, true>(k, Np, wkey0 + 32 * (i / NCK), i % NCK, lane, raw[i]);
  // the rows' (M_t, 1/L_t) from the row-statistics partials of every tile of the head:
  // thread = (row t, part); each part merges every PARTS-th tile, 8 tiles' loads issued
  // together, then the parts are merged through LDS
  {
    constexpr int PARTS = R < 256 ? 256 / R : 1, TU = 8;
    __shared__ float pm[256], pl[256];
    const int t = threadIdx.x % R, part = threadIdx.x / R;
    float M = -INFINITY, L = 0.f;
    if (t < R && part < PARTS) {
      for (int i0 = part; i0 < p.tiles; i0 += PARTS * TU) {
        float2 st[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          const int i = min(i0 + u * PARTS, p.tiles - 1);  // in range; extra tiles are dropped below
          st[u] = *reinterpret_cast<const float2*>(p.rowstat + ((bh * p.tiles + i) * R + t) * 2);
        }
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          const float m = i0 + u * PARTS < p.tiles ? st[u].x : -INFINITY;
          const float mn = fmaxf(M, m);
          if (mn > -INFINITY) {
            L = L * exp2f(M - mn) + (m > -INFINITY ? st[u].y * exp2f(m - mn) : 0.f);
            M = mn;
          }
        }
      }
    }
    pm[threadIdx.x] = M;
    pl[threadIdx.x] = L;
    __syncthreads();
    if (threadIdx.x < R) {
      float mm = -INFINITY, ll = 0.f;
      for (int q = 0; q < PARTS; ++q) mm = fmaxf(mm, pm[q * R + threadIdx.x]);
      if (mm > -INFINITY)
        for (int q = 0; q < PARTS; ++q) ll += pl[q * R + threadIdx.x] * exp2f(pm[q * R + threadIdx.x] - mm);
      // rows past L_obs get zero weight
      const bool real = (int)threadIdx.x < p.Lobs && ll > 0.f;
      sM[threadIdx.x] = real ? mm : 0.f;
      sI[threadIdx.x] = real ? 1.f / ll : 0.f;
    }
  }
  bf16x8 qf[QR::kRegs ? RB : 1][D / 16];
  if constexpr (QR::kRegs) {
    __syncthreads();  // sM / sI complete
    if (wkey0 >= Np) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) load_q_frags<D>(q, p.Lobs, rb, lane, qf[rb]);
  } else {
    stage_q_rows<D, RB>(q, p.Lobs, qs);
    __syncthreads();  // sM / sI and the staged rows complete
    if (wkey0 >= Np) return;
  }
  auto qfrag = [&](int rb, int s) {
    if constexpr (QR::kRegs) return qf[rb][s];
    else return q_frag_lds<D>(qs, rb, s, lane);
  };
  constexpr int NC = D / chunk_w<D>();
  constexpr int FS = chunk_w<D>() / 16;
  static_assert(NC == 1 || RG == RB, "a row of two column chunks keeps every row block's accumulator");
#pragma unroll
  for (int blk = 0; blk < kWaveBlocks; ++blk) {
    const int key0 = wkey0 + blk * 32;
    if (key0 >= Np) break;  // wave-uniform
    float sc = 0.f;
    f32x16 acc[RG];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = blk * NC + c;  // PF chunks in flight, as in the row-statistics pass
      chunk_store_lds<D>(stage[wave], lane, raw[i % PF]);
      if (i + PF < T) chunk_load<D, true>(k, Np, wkey0 + 32 * ((i + PF) / NC), (i + PF) % NC, lane, raw[i % PF]);
      wave_lds_order();
      bf16x8 kf[FS];
      chunk_frags_lds<D>(stage[wave], lane, kf);
      wave_lds_order();
#pragma unroll
      for (int g0 = 0; g0 < RB; g0 += RG) {
        if (NC == 1 || c == 0) {
#pragma unroll
          for (int r = 0; r < RG; ++r) acc[r] = f32x16{};
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
#pragma unroll
          for (int st = 0; st < FS; ++st)
            acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfrag(g0 + r, c * FS + st), kf[st], acc[r], 0, 0, 0);
        }
        if (NC == 1 || c == NC - 1) {
          // acc[r][e]: observation row (g0 + r) * 32 + mfma_row(e), key key0 + lane % 32;
          // weight 2^(acc * scale - M_t) / L_t as FMA, exp2, FMA
#pragma unroll
          for (int r = 0; r < RG; ++r) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int t = (g0 + r) * 32 + mfma_row(e, lane);
              sc = fmaf(exp2f(fmaf(acc[r][e], p.qscale, -sM[t])), sI[t], sc);
            }
          }
        }
      }
    }
    sc += __shfl_xor(sc, 32, 64);
    const int key = key0 + (lane & 31);
    if (lane < 32 && key < Np) p.colscore[bh * p.sstride + key] = sc * inv_rows;
  }
}

// ---------------------------------------------------------------------------- 3. select
// Exclusive prefix sum over the 1024 threads of the block; *total receives the sum.
// Each wave scans its lanes with DPP-free shuffles, publishes its total, and after one
// barrier every wave adds the totals of the waves before it itself (16 broadcast LDS
// reads, no serial pass).  warp_tot must not be reused before every thread has
// returned: callers alternate two buffers.
__device__ int block_exclusive_scan(int v, int* warp_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) warp_tot[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    const int t = warp_tot[w];
    before += w < wave ? t : 0;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// Pooling of the prefix scores: centred window of kernel_size, zero padding; the
// average divides by kernel_size everywhere.  Fixed summation order (-r .. r).
__global__ void snapkv_pool_kernel(SnapkvParams p) {
  const int Np = p.N - p.Lobs;
  const size_t total = (size_t)p.B * p.H * Np;
  const int rad = p.ksize / 2;
  const float inv_k = 1.f / (float)p.ksize;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = e / Np;
    const int i = (int)(e % Np);
    const float* s = p.colscore + bh * p.sstride;
    float acc = 0.f;  // scores are >= 0: also the identity of max
    for (int d = -rad; d <= rad; ++d) {
      const int j = i + d;
      if (j < 0 || j >= Np) continue;
      acc = p.pool ? fmaxf(acc, s[j]) : acc + s[j];
    }
    const float v = p.pool ? acc : acc * inv_k;
    p.pooled[bh * p.sstride + i] = v;
    if (p.scores_out) p.scores_out[e] = v;
  }
}

// Radix select of the k-th largest pooled score of one head, with the scores held in
// registers: thread t owns the contiguous positions [t*PER, (t+1)*PER).
//
// With HALO = 4 the pooling is done here (kernel_size <= 9): each thread reads its raw
// column scores with HALO neighbours on each side as 16-byte loads and pools them in
// registers, in the same order and with the same zero padding as snapkv_pool_kernel;
// with HALO = 0 the input is the pooled scores.
//
// Scores are >= 0, so their float bit patterns order like the values.  The select runs
// on v = bits - min(bits) over the head: its bit length Lb is set by the spread of the
// scores (a few octaves), so the first 11-bit digit already separates values that the
// raw exponent bits would lump into a handful of bins (fewer LDS atomic conflicts).
// Digits are taken from bit Lb down in 11-bit steps; each pass histograms the
// candidates that match the prefix fixed so far (4 interleaved copies of the histogram
// cut conflicts further), then a block scan over the bins, highest digit first, finds
// the digit where the count of larger values reaches k.
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kHistCopies = 4;

// Pooled scores of the thread's PER positions from its window w (HALO raw scores on each
// side, zero past the ends): the 2 RAD + 1 taps in ascending order, then 1/kernel_size
// for the average.  Scores are >= 0, so 0 is also the identity of the maximum.
template <int PER, int HALO, int RAD, bool MAX>
__device__ inline void pool_taps(const float (&w)[PER + 2 * HALO], uint32_t (&u)[PER], float inv_k) {
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int d = -RAD; d <= RAD; ++d) acc = MAX ? fmaxf(acc, w[j + HALO + d]) : acc + w[j + HALO + d];
    u[j] = __float_as_uint(MAX ? acc : acc * inv_k);
  }
}

template <int PER, int HALO>
__global__ void __launch_bounds__(kSelectThreads) snapkv_select_kernel(SnapkvParams p) {
  static_assert(PER % 4 == 0 && HALO % 4 == 0, "16-byte pieces");
  __shared__ int hist[kHistCopies * kBins];
  __shared__ int warp_tot[2][kSelectThreads / 64];  // alternated between consecutive scans
  __shared__ uint32_t wmin[kSelectThreads / 64], wmax[kSelectThreads / 64];
  int total;
  __shared__ int s_digit, s_krem;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)b * p.H + h;
  const int Np = p.N - p.Lobs;
  const float* src = (HALO > 0 ? p.colscore : p.pooled) + bh * p.sstride;
  const int i0 = threadIdx.x * PER;

  // ---- the thread's scores as bit patterns (rows are padded to a multiple of 4 floats)
  uint32_t u[PER];
  {
    constexpr int NW = PER + 2 * HALO;
    float w[NW];
    // every load in range (clamped to the row's first and last 16-byte pieces; a row
    // holds at least one), positions outside [0, Np) zeroed after the load
    const int last = Np > 0 ? ((Np - 1) & ~3) : 0;
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const int e0 = i0 - HALO + 4 * q;  // a multiple of 4
      const float4 v = *reinterpret_cast<const float4*>(src + min(max(e0, 0), last));
      const bool lo = e0 >= 0;
      w[4 * q] = lo && e0 < Np ? v.x : 0.f;
      w[4 * q + 1] = lo && e0 + 1 < Np ? v.y : 0.f;
      w[4 * q + 2] = lo && e0 + 2 < Np ? v.z : 0.f;
      w[4 * q + 3] = lo && e0 + 3 < Np ? v.w : 0.f;
    }
    if constexpr (HALO > 0) {
      const float inv_k = 1.f / (float)p.ksize;
      // one branch on the (uniform) radius and kind, then straight-line taps
#define LCD_POOL(R)                                                                  \
  do {                                                                               \
    if (p.pool)                                                                      \
      pool_taps<PER, HALO, (R) < HALO ? (R) : HALO, true>(w, u, inv_k);             \
    else                                                                             \
      pool_taps<PER, HALO, (R) < HALO ? (R) : HALO, false>(w, u, inv_k);            \
  } while (0)
      switch (p.ksize / 2) {
        case 0: LCD_POOL(0); break;
        case 1: LCD_POOL(1); break;
        case 2: LCD_POOL(2); break;
        case 3: LCD_POOL(3); break;
        default: LCD_POOL(4); break;
      }
#undef LCD_POOL
      if (p.scores_out) {
        float* so = p.scores_out + bh * Np;
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (i0 + j < Np) so[i0 + j] = __uint_as_float(u[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) u[j] = __float_as_uint(w[j]);
    }
  }
  uint32_t lmin = 0xffffffffu, lmax = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (i0 + j < Np) {
      lmin = min(lmin, u[j]);
      lmax = max(lmax, u[j]);
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
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    umin = min(umin, wmin[w]);
    umax = max(umax, wmax[w]);
  }
  const int k = p.k_keep;
  const uint32_t range = umax >= umin ? umax - umin : 0u;
  const int Lb = range ? 32 - __clz((int)range) : 0;
  // from here on u holds v = bits - umin (order-preserving over the valid positions;
  // positions past Np are excluded by index everywhere)
#pragma unroll
  for (int j = 0; j < PER; ++j) u[j] -= umin;
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  if (k > 0) {
    for (int hi = Lb; hi > 0; hi -= kDigitBits) {
      const int shift = hi > kDigitBits ? hi - kDigitBits : 0;
      const int bits = hi - shift;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = threadIdx.x; i < kHistCopies * kBins; i += kSelectThreads) hist[i] = 0;
      __syncthreads();
      int* hcopy = hist + (threadIdx.x & (kHistCopies - 1)) * kBins;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (i0 + j < Np && (u[j] & mask) == prefix) atomicAdd(&hcopy[(u[j] >> shift) & dmask], 1);
      __syncthreads();
      // bins in descending digit order, two per thread
      const int nb = 1 << bits;
      int c[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int bin = nb - 1 - (2 * (int)threadIdx.x + e);
        int v = 0;
        if (bin >= 0)
          for (int q = 0; q < kHistCopies; ++q) v += hist[q * kBins + bin];
        c[e] = v;
      }
      const int before = block_exclusive_scan(c[0] + c[1], warp_tot[0], &total);
      if (before < krem && before + c[0] + c[1] >= krem) {
        const int e = before + c[0] >= krem ? 0 : 1;
        s_digit = nb - 1 - (2 * (int)threadIdx.x + e);
        s_krem = krem - before - (e ? c[0] : 0);
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= dmask << shift;
      krem = s_krem;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;                   // v of the k-th largest score
  const int take_eq_total = k > 0 ? krem : 0;  // how many values equal to T are kept
  int n_gt = 0, n_eq = 0;
  if (k > 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool in = i0 + j < Np;
      n_gt += in && u[j] > T;
      n_eq += in && u[j] == T;
    }
  }
  const int eq_before = block_exclusive_scan(n_eq, warp_tot[1], &total);
  const int take_eq = max(0, min(n_eq, take_eq_total - eq_before));
  const int off = block_exclusive_scan(n_gt + take_eq, warp_tot[0], &total);
  int* idx = p.idx_out + bh * p.out_rows;
  if (k > 0) {
    int o = off, seen = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (i0 + j >= Np) break;
      bool keep = u[j] > T;
      if (u[j] == T) {
        keep = seen < take_eq;
        ++seen;
      }
      if (keep) idx[o++] = i0 + j;
    }
  }
  for (int t = threadIdx.x; t < p.Lobs; t += kSelectThreads) idx[k + t] = Np + t;
}

// ---------------------------------------------------------------------------- 4. gather
// Row copies of the kept K and V rows as 16-byte pieces: each thread moves kGatherU
// pieces of K and of V per iteration, all loads issued before the stores (plain loads
// and stores: non-temporal ones measured no faster on MI355X).
constexpr int kGatherU = 1;
__global__ void __launch_bounds__(256) snapkv_gather_kernel(SnapkvParams p, int rows) {
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * p.H + h;
  const int chunks = p.D * 2 / 16;  // 16-byte pieces per row
  const int* idx = p.idx_out + bh * p.out_rows;
  const char* k = reinterpret_cast<const char*>(p.k) + bh * (size_t)p.N * p.D * 2;
  const char* v = reinterpret_cast<const char*>(p.v) + bh * (size_t)p.N * p.D * 2;
  char* ko = reinterpret_cast<char*>(p.k_out) + bh * (size_t)p.out_rows * p.D * 2;
  char* vo = reinterpret_cast<char*>(p.v_out) + bh * (size_t)p.out_rows * p.D * 2;
  const int total = rows * chunks;
  for (int e0 = blockIdx.x * 256 * kGatherU + threadIdx.x; e0 < total; e0 += gridDim.x * 256 * kGatherU) {
    u32x4 kr[kGatherU], vr[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
      const int e = e0 + u * 256;
      if (e < total) {
        const size_t src = (size_t)idx[e / chunks] * p.D * 2 + (size_t)(e % chunks) * 16;
        kr[u] = *reinterpret_cast<const u32x4*>(k + src);
        vr[u] = *reinterpret_cast<const u32x4*>(v + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
      const int e = e0 + u * 256;
      if (e < total) {
        const size_t dst = (size_t)(e / chunks) * p.D * 2 + (size_t)(e % chunks) * 16;
        *reinterpret_cast<u32x4*>(ko + dst) = kr[u];
        *reinterpret_cast<u32x4*>(vo + dst) = vr[u];
      }
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t rowstat, colscore, pooled, total;
};

// Rows of the column-score and pooled buffers are padded to a multiple of 4 floats
// (16-byte loads in the select kernel).
size_t score_stride(int N, int Lobs) {
  const size_t np = (size_t)(N - Lobs);
  return np ? (np + 3) / 4 * 4 : 4;
}

// Observation row blocks of 32 the scoring kernels run: 1, 2, 4 or 8.
int row_blocks(int Lobs) {
  const int rb = (Lobs + 31) / 32;
  return rb <= 1 ? 1 : rb <= 2 ? 2 : rb <= 4 ? 4 : 8;
}

WsLayout ws_layout(int B, int H, int N, int Lobs) {
  const size_t bh = (size_t)B * H;
  const size_t tiles = (size_t)(N + kTileKeys - 1) / kTileKeys;
  const size_t st = score_stride(N, Lobs);
  const size_t rows = (size_t)row_blocks(Lobs) * 32;  // per-tile row statistics, padded rows
  WsLayout w;
  w.rowstat = 0;
  w.colscore = align256(w.rowstat + bh * tiles * rows * 2 * sizeof(float));
  w.pooled = align256(w.colscore + bh * st * sizeof(float));
  w.total = align256(w.pooled + bh * st * sizeof(float));
  return w;
}

template <int D, int RB>
void launch_scores(const SnapkvParams& p, int np, hipStream_t s) {
  const dim3 sgrid(p.tiles, p.H, p.B);
  hipLaunchKernelGGL((snapkv_rowstats_kernel<D, RB>), sgrid, dim3(256), 0, s, p);
  if (np > 0) {
    const dim3 cgrid((np + kTileKeys - 1) / kTileKeys, p.H, p.B);
    hipLaunchKernelGGL((snapkv_colscore_kernel<D, RB>), cgrid, dim3(256), 0, s, p);
  }
}

template <int D>
hipError_t launch_d(SnapkvParams p, hipStream_t s) {
  const int np = p.N - p.Lobs;
  p.h0 = 0;
  switch (row_blocks(p.Lobs)) {
    case 1: launch_scores<D, 1>(p, np, s); break;
    case 2: launch_scores<D, 2>(p, np, s); break;
    case 4: launch_scores<D, 4>(p, np, s); break;
    default:
      if constexpr (D <= 128) launch_scores<D, 8>(p, np, s);  // (the host admits 256 rows at D <= 128 only)
      else return hipErrorInvalidValue;
      break;
  }
  // pooling is fused into the select kernel for kernel_size <= 9
  const bool fused = p.ksize <= 9;
  if (np > 0 && !fused) {
    const size_t work = (size_t)p.B * p.H * np;
    const size_t blocks = (work + 255) / 256;
    hipLaunchKernelGGL(snapkv_pool_kernel, dim3(blocks < 8192 ? blocks : 8192), dim3(256), 0, s, p);
  }
  const int per = (np + kSelectThreads - 1) / kSelectThreads;
  const dim3 sel_grid(p.H, p.B);
#define LCD_SELECT(PER)                                                                    \
  do {                                                                                     \
    if (fused)                                                                             \
      hipLaunchKernelGGL((snapkv_select_kernel<PER, 4>), sel_grid, dim3(kSelectThreads), 0, s, p); \
    else                                                                                   \
      hipLaunchKernelGGL((snapkv_select_kernel<PER, 0>), sel_grid, dim3(kSelectThreads), 0, s, p); \
  } while (0)
  if (per <= 8)
    LCD_SELECT(8);
  else if (per <= 16)
    LCD_SELECT(16);
  else if (per <= 32)
    LCD_SELECT(32);
  else
    LCD_SELECT(64);
#undef LCD_SELECT
  const int rows = p.k_keep + p.Lobs;
  const int chunks = p.D * 2 / 16;
  const int blocks_x = (rows * chunks + 256 * kGatherU - 1) / (256 * kGatherU);
  hipLaunchKernelGGL(snapkv_gather_kernel, dim3(blocks_x < 1024 ? blocks_x : 1024, p.H, p.B), dim3(256), 0, s, p,
                     rows);
  return hipGetLastError();
}

}  // namespace

size_t snapkv_ws_bytes(int B, int H, int N, int Lobs) { return ws_layout(B, H, N, Lobs).total; }

hipError_t launch_snapkv(const SnapkvParams& in, hipStream_t s) {
  SnapkvParams p = in;
  const WsLayout w = ws_layout(p.B, p.H, p.N, p.Lobs);
  char* base = reinterpret_cast<char*>(p.rowstat);
  p.rowstat = reinterpret_cast<float*>(base + w.rowstat);
  p.colscore = reinterpret_cast<float*>(base + w.colscore);
  p.pooled = reinterpret_cast<float*>(base + w.pooled);
  p.tiles = (p.N + kTileKeys - 1) / kTileKeys;
  p.sstride = (int)score_stride(p.N, p.Lobs);
  switch (p.D) {
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    case 256: return launch_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lcd
