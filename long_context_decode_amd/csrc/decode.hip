// Split-K decode attention over a compressed KV cache, for gfx950 (wave64).
//
// One workgroup owns one (split, KV head g, batch row b): a contiguous range of
// `chunk` cache slots and the G query heads that share KV head g (grouped-query
// attention, [KVL] "01 · Conceito": 24 query heads share 4 KV heads).  The decode
// step reads the whole cache once ([KVC] "O gargalo de memória do KV Cache...":
// decode is a matrix-vector product over the cache, 1-2 flop per byte), and the
// cache is split along the sequence ([KVC] "Implementação prática em vLLM e
// SGLang": FlashDecoding parallelises along time), so the kernel is HBM-bound.
//
// Per workgroup:
//   K pass  every key of the range is loaded once (two 16-byte loads per lane,
//           one from each half of the row), rotated in registers at its in-cache
//           position when keys are stored un-rotated ([SINK] "como funciona"),
//           and dotted with the G pre-rotated, pre-scaled queries; the dot is
//           reduced across the LPK lanes that share the key.  Logits go to LDS.
//   softmax the range maximum per query head, p = 2^(x - m) in LDS, l = sum p.
//   V pass  every value row is loaded once and accumulated with the G weights.
//   merge   with one split the workgroup normalises and writes the output;
//           otherwise it publishes (o, m, l) to the workspace and the last
//           workgroup of its (b, g) to arrive merges all splits in split order
//           (deterministic) and, for H2O, runs the score / eviction epilogue.
// Logits are kept in the log2 domain (the query carries scale * log2 e) so the
// exponentials are single exp2 instructions.
#include <hip/hip_runtime.h>

#include "lcd_internal.h"

namespace lcd {

struct bf16_t {
  uint16_t bits;
};

// K/V rows are streamed once per decode step; their loads are non-temporal so they
// do not displace the position table in L2 (LCD_NT_KV=0 builds plain loads).
#ifndef LCD_NT_KV
#define LCD_NT_KV 1
#endif

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint4 load16(const void* p) {
#if LCD_NT_KV
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#endif
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Element formats.  HALF elements fill one 16-byte load; cvt widens to float32.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int HALF = 4;
  __device__ static inline void cvt(const uint4 v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ static inline void load(const void* p, float (&x)[4]) { cvt(load16(p), x); }
};

template <>
struct Elem<bf16_t> {
  static constexpr int HALF = 8;
  __device__ static inline void cvt(const uint4 v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline void load(const void* p, float (&x)[8]) { cvt(load16(p), x); }
};

// DPP lane moves inside 16-lane rows (no LDS traffic).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64); every
// lane of the group receives the total.  Groups up to 16 lanes use DPP.
template <int N>
__device__ inline float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
#pragma unroll
  for (int off = 16; off < N; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Cross-workgroup hand-off of split partials.  The L2 of one XCD is not coherent
// with the others, and a device-scope fence writes back / invalidates the whole L2,
// so partials are written and read with device-scope relaxed atomic accesses
// (coherent at the device level, no cache-wide maintenance) and ordered before the
// arrival counter by waiting for the stores to complete.
__device__ inline void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(kDecodeThreads) decode_split_kernel(DecodeParams p) {
  constexpr bool ROPE = MODE == kModeRope;
  constexpr bool LOGITS = MODE == kModePlainLogits;
  constexpr int HALF = Elem<T>::HALF;
  constexpr int EPL = 2 * HALF;    // elements per lane (HALF pairs)
  constexpr int LPK = D / EPL;     // lanes per key
  constexpr int KPW = 64 / LPK;    // keys per wave per iteration
  constexpr int KPI = 4 * KPW;     // keys per workgroup per iteration
  constexpr int D2 = D / 2;
  static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "lane mapping");

  extern __shared__ float smem[];
  float* xs = smem;                       // [chunk][G] logits, then weights
  float* red = xs + p.chunk * G;          // [4][G] cross-wave reductions, then [G] sums
  float* ored = red + 5 * G;              // [4][G][D] cross-wave output sums

  // Workgroups are dealt round-robin to the 8 XCDs, so linear id w runs on XCD
  // w % 8.  Give each XCD a contiguous run of (split, kv-head, batch) items, split
  // slowest: the workgroups resident on one XCD then share a slot range and its
  // slice of the position table stays in that XCD's L2.
  const int per_xcd = (int)((gridDim.x + 7) / 8);
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int n_bg = p.B * p.Hkv;
  if (item >= p.n_splits * n_bg) return;  // padding of the grid to a multiple of 8
  const int split = item / n_bg;
  const int g = (item % n_bg) % p.Hkv, b = (item % n_bg) / p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kg = lane / LPK;
  const int i0 = sub * HALF;  // first pair index owned by this lane
  const int s_begin = split * p.chunk;
  const int cnt = min(p.n - s_begin, p.chunk);

  const size_t bg = (size_t)b * p.Hkv + g;
  const char* kbase = reinterpret_cast<const char*>(p.k) + bg * p.C * D * sizeof(T);
  const char* vbase = reinterpret_cast<const char*>(p.v) + bg * p.C * D * sizeof(T);
  const size_t lo_off = (size_t)i0 * sizeof(T);
  const size_t hi_off = (size_t)(D2 + i0) * sizeof(T);

  // ---- queries of the group: load, rotate at the query's position, pre-scale
  float qf[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const char* qrow = reinterpret_cast<const char*>(p.q) + ((size_t)b * p.Hq + g * G + j) * D * sizeof(T);
    float lo[HALF], hi[HALF];
    Elem<T>::load(qrow + lo_off, lo);
    Elem<T>::load(qrow + hi_off, hi);
    if constexpr (ROPE) {
      const float* cr = p.cos_t + (size_t)p.q_rank * D2 + i0;
      const float* sr = p.sin_t + (size_t)p.q_rank * D2 + i0;
#pragma unroll
      for (int e = 0; e < HALF; ++e) {
        const float c = cr[e], s = sr[e];
        const float a = lo[e], bb = hi[e];
        lo[e] = a * c - bb * s;
        hi[e] = a * s + bb * c;
      }
    }
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      qf[j][e] = lo[e] * p.qscale;
      qf[j][HALF + e] = hi[e] * p.qscale;
    }
  }

  // ---- K pass: U keys per lane group per iteration, every load issued first.
  // With RoPE, the lane's U keys of one iteration sit KPI slots apart; where their
  // in-cache positions are also KPI apart (everywhere except across the ring's wrap
  // point and the sink boundary) the cos/sin of key u+1 follow from key u's by one
  // angle addition with the per-lane constant rotation (cos, sin)(KPI * theta_i), so
  // only one table row is read per iteration.  Waves that straddle a discontinuity
  // read every key's row from the table instead.
  constexpr int U = (G <= 2) ? 4 : 2;
  float mx[G];
#pragma unroll
  for (int j = 0; j < G; ++j) mx[j] = -INFINITY;
  float dc[HALF], ds[HALF];
  if constexpr (ROPE) {
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      dc[e] = p.cos_t[(size_t)KPI * D2 + i0 + e];
      ds[e] = p.sin_t[(size_t)KPI * D2 + i0 + e];
    }
  }
  auto rank_of = [&](int slot) {
    int rank = slot;
    if (p.full && slot >= p.S) {
      int r = slot - p.S - p.ring_head;
      if (r < 0) r += p.W;
      rank = p.S + r;
    }
    return rank;
  };
  auto load_cs = [&](int rank, float (&c)[HALF], float (&sn)[HALF]) {
    const float4* cr = reinterpret_cast<const float4*>(p.cos_t + (size_t)rank * D2 + i0);
    const float4* sr = reinterpret_cast<const float4*>(p.sin_t + (size_t)rank * D2 + i0);
#pragma unroll
    for (int e = 0; e < HALF / 4; ++e) {
      const float4 c4 = cr[e], s4 = sr[e];
      c[4 * e] = c4.x; c[4 * e + 1] = c4.y; c[4 * e + 2] = c4.z; c[4 * e + 3] = c4.w;
      sn[4 * e] = s4.x; sn[4 * e + 1] = s4.y; sn[4 * e + 2] = s4.z; sn[4 * e + 3] = s4.w;
    }
  };

  for (int base = 0; base < cnt; base += KPI * U) {
    const int key0 = base + wave * KPW + kg;
    uint4 rlo[U], rhi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = key0 + u * KPI;
      if (key < cnt) {
        const char* row = kbase + (size_t)(s_begin + key) * D * sizeof(T);
        rlo[u] = load16(row + lo_off);
        rhi[u] = load16(row + hi_off);
      } else {
        rlo[u] = make_uint4(0, 0, 0, 0);
        rhi[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float c[HALF], sn[HALF];
    bool stepwise = false;  // this wave straddles a rank discontinuity
    int rank0 = 0;
    if constexpr (ROPE) {
      rank0 = rank_of(s_begin + min(key0, cnt - 1));
      bool disc = false;
#pragma unroll
      for (int u = 1; u < U; ++u) {
        const int key = key0 + u * KPI;
        disc |= key < cnt && rank_of(s_begin + key) != rank0 + u * KPI;
      }
      stepwise = __any(disc);
      load_cs(rank0, c, sn);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = key0 + u * KPI;
      const bool valid = key < cnt;
      float kf[EPL];
      {
        float lo[HALF], hi[HALF];
        Elem<T>::cvt(rlo[u], lo);
        Elem<T>::cvt(rhi[u], hi);
        if constexpr (ROPE) {
          if (u > 0) {
            if (stepwise) {
              load_cs(rank_of(s_begin + min(key, cnt - 1)), c, sn);
            } else {
#pragma unroll
              for (int e = 0; e < HALF; ++e) {
                const float cc = c[e] * dc[e] - sn[e] * ds[e];
                sn[e] = sn[e] * dc[e] + c[e] * ds[e];
                c[e] = cc;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            kf[e] = lo[e] * c[e] - hi[e] * sn[e];
            kf[HALF + e] = lo[e] * sn[e] + hi[e] * c[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            kf[e] = lo[e];
            kf[HALF + e] = hi[e];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[j][e], kf[e], d);
        d = group_sum<LPK>(d);
        if (valid) {
          mx[j] = fmaxf(mx[j], d);
          if (sub == 0) {
            xs[key * G + j] = d;
            if constexpr (LOGITS) store_dev(&p.logits[((size_t)b * p.Hq + g * G + j) * p.C + s_begin + key], d);
          }
        }
      }
    }
  }

  // first V rows are requested before the softmax barriers (their latency overlaps them)
  constexpr int UV = 4;
  uint4 vlo[UV], vhi[UV];
  auto load_v = [&](int base) {
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int key = base + u * KPI + wave * KPW + kg;
      if (key < cnt) {
        const char* row = vbase + (size_t)(s_begin + key) * D * sizeof(T);
        vlo[u] = load16(row + lo_off);
        vhi[u] = load16(row + hi_off);
      } else {
        vlo[u] = make_uint4(0, 0, 0, 0);
        vhi[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  load_v(0);

  // ---- range maximum per query head
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float m = wave_max(mx[j]);
    if (lane == 0) red[wave * G + j] = m;
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    M[j] = fmaxf(fmaxf(red[j], red[G + j]), fmaxf(red[2 * G + j], red[3 * G + j]));
  __syncthreads();  // red is reused below

  // ---- weights p = 2^(x - m) and their sums
  float ls[G];
#pragma unroll
  for (int j = 0; j < G; ++j) ls[j] = 0.f;
  for (int key = threadIdx.x; key < cnt; key += kDecodeThreads) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float e = exp2f(xs[key * G + j] - M[j]);
      xs[key * G + j] = e;
      ls[j] += e;
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float s = wave_sum(ls[j]);
    if (lane == 0) red[wave * G + j] = s;
  }
  __syncthreads();

  // ---- V pass: UV rows per lane group per iteration; the next iteration's rows are
  // requested before this iteration's arithmetic (software pipelining)
  float o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;

  for (int base = 0; base < cnt; base += KPI * UV) {
    uint4 clo[UV], chi[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      clo[u] = vlo[u];
      chi[u] = vhi[u];
    }
    if (base + KPI * UV < cnt) load_v(base + KPI * UV);
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int key = base + u * KPI + wave * KPW + kg;
      if (key < cnt) {
        float lo[HALF], hi[HALF];
        Elem<T>::cvt(clo[u], lo);
        Elem<T>::cvt(chi[u], hi);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float w = xs[key * G + j];
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            o[j][e] = fmaf(w, lo[e], o[j][e]);
            o[j][HALF + e] = fmaf(w, hi[e], o[j][HALF + e]);
          }
        }
      }
    }
  }

  // ---- merge the key groups of the wave, then the 4 waves
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = o[j][e];
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      o[j][e] = x;
    }
  if (kg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < HALF; ++e) {
        ored[(wave * G + j) * D + i0 + e] = o[j][e];
        ored[(wave * G + j) * D + D2 + i0 + e] = o[j][HALF + e];
      }
  }
  __syncthreads();
  const size_t bh0 = (size_t)b * p.Hq + g * G;
  float* wsum = red + 4 * G;  // this workgroup's l per head (aliases nothing live)
  if (threadIdx.x < G) {
    const int j = threadIdx.x;
    wsum[j] = red[j] + red[G + j] + red[2 * G + j] + red[3 * G + j];
  }
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int j = idx / D, d = idx % D;
    ored[idx] = ored[(0 * G + j) * D + d] + ored[(1 * G + j) * D + d] + ored[(2 * G + j) * D + d] +
                ored[(3 * G + j) * D + d];
  }
  __syncthreads();
  // ored[0 .. G*D) now holds this range's unnormalised output, wsum its l, M its max.

  __shared__ float Mtot[G], Linv[G];
  __shared__ int is_last;
  if (p.n_splits == 1) {
    if (threadIdx.x < G) {
      Mtot[threadIdx.x] = M[threadIdx.x];
      Linv[threadIdx.x] = 1.f / wsum[threadIdx.x];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads)
      p.out[(bh0 + idx / D) * D + idx % D] = ored[idx] * Linv[idx / D];
  } else {
    // publish this split's partial, then count arrivals for (b, g)
    const size_t BH = (size_t)p.B * p.Hq;
    for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads)
      store_dev(&p.part_o[((size_t)split * BH + bh0 + idx / D) * D + idx % D], ored[idx]);
    if (threadIdx.x < G) {
      float* ml = p.part_ml + ((size_t)split * BH + bh0 + threadIdx.x) * 2;
      store_dev(&ml[0], M[threadIdx.x]);
      store_dev(&ml[1], wsum[threadIdx.x]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = __hip_atomic_fetch_add(&p.arrivals[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                p.n_splits - 1;
    __syncthreads();
    if (!is_last) return;
    // last arrival: merge every split in split order (deterministic)
    if (threadIdx.x < G) {
      const int j = threadIdx.x;
      float mt = -INFINITY;
      for (int s = 0; s < p.n_splits; ++s) mt = fmaxf(mt, load_dev(&p.part_ml[((size_t)s * BH + bh0 + j) * 2]));
      float lt = 0.f;
      for (int s = 0; s < p.n_splits; ++s) {
        const float* ml = p.part_ml + ((size_t)s * BH + bh0 + j) * 2;
        lt += load_dev(&ml[1]) * exp2f(load_dev(&ml[0]) - mt);
      }
      Mtot[j] = mt;
      Linv[j] = 1.f / lt;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
      const int j = idx / D, d = idx % D;
      float acc = 0.f;
      for (int s = 0; s < p.n_splits; ++s)
        acc += load_dev(&p.part_o[((size_t)s * BH + bh0 + j) * D + d]) *
               exp2f(load_dev(&p.part_ml[((size_t)s * BH + bh0 + j) * 2]) - Mtot[j]);
      p.out[(bh0 + j) * D + d] = acc * Linv[j];
    }
    if (threadIdx.x == 0)  // ready for the next call
      __hip_atomic_store(&p.arrivals[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (LOGITS) {
    // H2O: add this step's weights (summed over the group's query heads) to every
    // filled slot's score and pick the slot the next append overwrites: the lowest
    // score among slots with pos <= max_pos, ties evicting the higher position.
    __shared__ unsigned long long wbest[4];
    float* score = p.score + bg * p.C;
    const int* pos = p.pos + bg * p.C;
    unsigned long long best = ~0ull;
    for (int i = threadIdx.x; i < p.n; i += kDecodeThreads) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) a += exp2f(load_dev(&p.logits[(bh0 + j) * p.C + i]) - Mtot[j]) * Linv[j];
      const float sc = score[i] + a;
      score[i] = sc;
      const int ps = pos[i];
      if (p.pick_victim && (int64_t)ps <= p.max_pos) {
        const unsigned long long key =
            ((unsigned long long)__float_as_uint(sc) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)ps);
        best = key < best ? key : best;
      }
    }
    if (p.pick_victim) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long other = __shfl_xor(best, off, 64);
        best = other < best ? other : best;
      }
      if (lane == 0) wbest[wave] = best;
      __syncthreads();
      best = wbest[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) best = wbest[w] < best ? wbest[w] : best;
      if (best != ~0ull) {
        const int win_pos = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        for (int i = threadIdx.x; i < p.n; i += kDecodeThreads)
          if (pos[i] == win_pos) p.victim[bg] = i;
      }
    }
  }
}

// Victim choice for a seeded H2O layer (no decode step has run yet): the lowest score
// among slots whose token position is <= max_pos, ties evicting the higher position.
__global__ void __launch_bounds__(256) h2o_pick_victim_kernel(const float* score, const int* pos, int* victim, int C,
                                                              int n, int64_t max_pos) {
  __shared__ unsigned long long wbest[4];
  const size_t bg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long best = ~0ull;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int ps = pos[bg * C + i];
    if ((int64_t)ps <= max_pos) {
      const unsigned long long key = ((unsigned long long)__float_as_uint(score[bg * C + i]) << 32) |
                                     (unsigned long long)(0xffffffffu - (uint32_t)ps);
      best = key < best ? key : best;
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long other = __shfl_xor(best, off, 64);
    best = other < best ? other : best;
  }
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  best = wbest[0];
  for (int w = 1; w < 4; ++w) best = wbest[w] < best ? wbest[w] : best;
  if (best == ~0ull) return;
  const int win_pos = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
  for (int i = threadIdx.x; i < n; i += 256)
    if (pos[bg * C + i] == win_pos) victim[bg] = i;
}

hipError_t launch_h2o_pick_victim(const float* score, const int* pos, int* victim, int BHkv, int C, int n,
                                  int64_t max_pos, hipStream_t s) {
  hipLaunchKernelGGL(h2o_pick_victim_kernel, dim3(BHkv), dim3(256), 0, s, score, pos, victim, C, n, max_pos);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- dispatch
template <typename T, int D, int G>
static hipError_t launch_tdg(int mode, const DecodeParams& p, hipStream_t s) {
  const int items = p.n_splits * p.B * p.Hkv;
  const dim3 grid(((items + 7) / 8) * 8);
  const size_t lds = ((size_t)p.chunk * G + 5 * G + 4 * G * D) * sizeof(float);
  switch (mode) {
    case kModeRope:
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, kModeRope>), grid, dim3(kDecodeThreads), lds, s, p);
      break;
    case kModePlain:
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, kModePlain>), grid, dim3(kDecodeThreads), lds, s, p);
      break;
    case kModePlainLogits:
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, kModePlainLogits>), grid, dim3(kDecodeThreads), lds, s,
                         p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_td(int G, int mode, const DecodeParams& p, hipStream_t s) {
  switch (G) {
    case 1: return launch_tdg<T, D, 1>(mode, p, s);
    case 2: return launch_tdg<T, D, 2>(mode, p, s);
    case 4: return launch_tdg<T, D, 4>(mode, p, s);
    case 6: return launch_tdg<T, D, 6>(mode, p, s);
    case 8: return launch_tdg<T, D, 8>(mode, p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_t(int D, int G, int mode, const DecodeParams& p, hipStream_t s) {
  switch (D) {
    case 64: return launch_td<T, 64>(G, mode, p, s);
    case 128: return launch_td<T, 128>(G, mode, p, s);
    case 256: return launch_td<T, 256>(G, mode, p, s);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int dtype, int D, int G) {
  const bool d_ok = D == 64 || D == 128 || D == 256;
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 6 || G == 8;
  return (dtype == 0 || dtype == 1) && d_ok && g_ok;
}

hipError_t launch_decode_split(int dtype, int D, int G, int mode, const DecodeParams& p, hipStream_t s) {
  return dtype == 0 ? launch_t<float>(D, G, mode, p, s) : launch_t<bf16_t>(D, G, mode, p, s);
}

}  // namespace lcd
