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
// Per workgroup, one pass over the range: every lane group of LPK lanes owns one key
// (and its value) at a time; the lanes load one LB-byte piece from each half of the
// row, so each lane holds whole RoPE pairs (i, i + D/2) and rotates the key in
// registers at its in-cache position when keys are stored un-rotated ([SINK] "como
// funciona").  The group reduces the G dot products with DPP moves and keeps its own
// running softmax state (max m, sum l, output o) over its keys (online softmax):
// K and V rows of the next iteration are requested before the current one's
// arithmetic, and nothing in the loop waits for another wave.  At the end the lane
// groups of a wave, then the 4 waves, merge their (m, l, o).  With one split the
// workgroup normalises and writes the output; otherwise it publishes (o, m, l) to the
// workspace and the last workgroup of its (b, g) to arrive merges all splits in split
// order (deterministic) and, for H2O, runs the score / eviction epilogue.
// Logits are kept in the log2 domain (the query carries scale * log2 e) so the
// exponentials are single exp2 instructions.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>

#include "lcd_internal.h"

namespace lcd {

struct bf16_t {
  uint16_t bits;
};

// Constants chosen by measurement on MI355X.
// Keys per lane group per iteration: the one-pass kernel for G <= 2 (two iterations in
// flight) and for larger G; the two-pass kernel's K pass sets its own (see its Geo).
constexpr int kUnrollG2 = 2;
constexpr int kUnrollOnepassBig = 1;
constexpr int kOnepassMaxG = 2;  // largest G served by the one-pass kernel
// H2O epilogue: slots per thread per iteration (token-level and block-level eviction).  Four
// measured fastest at a budget of 4096 slots (1, 2, 6, 8, 12 and 16 were 0.5-3 us slower per
// launch, at the same register count).
constexpr int kH2oEu = 4;
constexpr int kH2oEuBlk = 4;
template <bool BLOCKS>
constexpr int EU_OF() { return BLOCKS ? kH2oEuBlk : kH2oEu; }
constexpr int kMergeSu = 4;  // split merge: splits whose loads are issued together

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// W 32-bit words of one row piece, loaded in one instruction (W = 4: 16 bytes, W = 2: 8).
template <int W>
struct Words {
  uint32_t w[W];
};

// K/V rows are streamed once per decode step; their loads are non-temporal so they do
// not displace the position table in L2.
template <int W>
__device__ inline Words<W> load_words(const void* p) {
  Words<W> r;
  if constexpr (W == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    static_assert(W == 2, "row pieces are 8 or 16 bytes");
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

template <int W>
__device__ inline Words<W> zero_words() {
  Words<W> r;
#pragma unroll
  for (int i = 0; i < W; ++i) r.w[i] = 0u;
  return r;
}

// Element formats: N elements per W-word piece, widened to float32.
template <typename T, int W>
struct Elem;

template <int W>
struct Elem<float, W> {
  static constexpr int N = W;
  __device__ static inline void cvt(const Words<W>& v, float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < W; ++i) x[i] = __uint_as_float(v.w[i]);
  }
};

template <int W>
struct Elem<bf16_t, W> {
  static constexpr int N = 2 * W;
  __device__ static inline void cvt(const Words<W>& v, float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      x[2 * i] = __uint_as_float(v.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(v.w[i] & 0xffff0000u);
    }
  }
};

// N consecutive floats (N = 2, 4 or 8) with 8- or 16-byte loads.
template <int N>
__device__ inline void load_floats(const float* p, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int e = 0; e < N / 4; ++e) {
      const float4 v = reinterpret_cast<const float4*>(p)[e];
      x[4 * e] = v.x; x[4 * e + 1] = v.y; x[4 * e + 2] = v.z; x[4 * e + 3] = v.w;
    }
  } else {
    static_assert(N == 2, "table pieces are 2, 4 or 8 floats");
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  }
}

// Waits for every outstanding vector-memory load of this wave (s_waitcnt vmcnt(0), other
// counters untouched).  Placed inside a rarely taken branch that loads registers the
// code after the branch reads, it keeps the compiler from waiting for all loads (those of
// the next iteration included) on the common path, where it merges the branch's state.
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// DPP lane moves inside 16-lane rows (no LDS traffic).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppRowShr4 = 0x114;  // lane i <- i - 4 within each 16 lanes
constexpr int kDppRowRor4 = 0x124;  // lane i <- (i + 4) mod 16 within each 16 lanes
constexpr int kDppRowRor8 = 0x128;  // lane i <- (i + 8) mod 16 within each 16 lanes

// Sums over aligned groups of N consecutive lanes (N in {4, 8, 16, 32}) of M values (M a
// multiple of 4), leaving each lane M/4 of the totals.  The first two steps transpose:
// partners (lanes i and i^1, then i and i^2) each keep half of their values and add the
// partner's copy of that half, so a step costs half the adds of a plain butterfly step
// (plus two selects per add); the remaining lane bits are summed in full.  Afterwards, with
// b0 = lane & 1 and b1 = (lane >> 1) & 1, slot i < M/4 holds the group total of value
// i + b0 * M/2 + b1 * M/4, in every lane for N = 4, 16 and 32 and in the lanes with bit 2
// set for N = 8 (there the last step writes only those lanes).  Totals are identical in
// every lane that holds them (each step adds a commutative pair).
template <int N, int M>
__device__ inline void group_sum_transposed(float (&x)[M], int lane) {
  static_assert(M % 4 == 0 && (N == 4 || N == 8 || N == 16 || N == 32), "shape");
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  constexpr int H1 = M / 2, H2 = M / 4;
#pragma unroll
  for (int i = 0; i < H1; ++i) {
    const float keep = b0 ? x[i + H1] : x[i];
    const float send = b0 ? x[i] : x[i + H1];
    x[i] = keep + dpp_mov<kDppXor1>(send);
  }
#pragma unroll
  for (int i = 0; i < H2; ++i) {
    const float keep = b1 ? x[i + H2] : x[i];
    const float send = b1 ? x[i] : x[i + H2];
    x[i] = keep + dpp_mov<kDppXor2>(send);
  }
  if constexpr (N == 8) {
#pragma unroll
    for (int i = 0; i < H2; ++i)  // lanes 4..7 (and 12..15) add lanes 0..3 (8..11)
      x[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x[i]), kDppRowShr4,
                                                                    0xF, 0xA, false));
  } else if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < H2; ++i) x[i] += dpp_mov<kDppRowRor4>(x[i]);
#pragma unroll
    for (int i = 0; i < H2; ++i) x[i] += dpp_mov<kDppRowRor8>(x[i]);
    if constexpr (N == 32) {
#pragma unroll
      for (int i = 0; i < H2; ++i) x[i] += __shfl_xor(x[i], 16, 64);
    }
  }
}

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64) of M
// independent values, one reduction step for all of them before the next, so the DPP
// moves of different values fill each other's hazards.  Every lane of a group receives
// the group's total, bit-identical across the group (each step adds a commutative pair).
template <int N, int M>
__device__ inline void group_sum_n(float (&x)[M]) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] += dpp_mov<kDppXor1>(x[m]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] += dpp_mov<kDppXor2>(x[m]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] += dpp_mov<kDppRowHalfMirror>(x[m]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] += dpp_mov<kDppRowMirror>(x[m]);
  }
#pragma unroll
  for (int off = 16; off < N; off <<= 1) {
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] += __shfl_xor(x[m], off, 64);
  }
}

// 2^x by the hardware instruction alone (v_exp_f32) for the softmax weights, x <= 0: it
// differs from exp2f only where the result is below 2^-126, which exp2f rescales to get
// subnormal results right; weights that small add nothing to a sum that holds a 1.
__device__ inline float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Geometry of the one-pass kernel: 16-byte pieces (W = 4 words).
template <typename T, int D, int G>
struct Geo {
  static constexpr int W = 4;
  static constexpr int HALF = Elem<T, W>::N;  // elements per piece = pairs per lane
  static constexpr int EPL = 2 * HALF;        // elements per lane
  static constexpr int LPK = D / EPL;         // lanes per key
  static constexpr int KPW = 64 / LPK;        // keys per wave per sub-step
  static constexpr int KPI = 4 * KPW;         // keys per workgroup per sub-step
  static constexpr int U = G <= 2 ? kUnrollG2 : kUnrollOnepassBig;
  static constexpr int STEP = KPI * U;        // keys per workgroup per iteration
  static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "lane mapping");
};

// Dynamic LDS of the one-pass kernel: the 4 waves' outputs [4][G][D], their (m, l)
// [2][4][G], the wave weights [4][G] and the workgroup's (m, l) [2][G].
template <int D, int G>
constexpr size_t onepass_lds_bytes() {
  return ((size_t)4 * G * D + 14 * G) * sizeof(float);
}

// Dynamic LDS of the two-pass kernel: the logits [G][chunk + kXsPad] (reused for the
// output after the V pass: [4][G][D] for float32 caches, [G][D] for bf16), cross-wave
// reductions [4][G] and the workgroup's (m, l) [2][G].  The padding shifts each query
// head's row by 16 bytes, so the V pass's reads of G rows at one key fall in distinct banks.
constexpr int kTwopassRed = 64;  // cross-wave reduction floats: 4 waves x (U * G <= 16)
constexpr int kXsPad = 4;
template <int D, int G>
inline size_t twopass_lds_floats(int chunk) {
  const size_t a = (size_t)(chunk + kXsPad) * G, o = (size_t)4 * G * D;
  return (a > o ? a : o) + kTwopassRed + 2 * G;
}

// The work item of linear index `item` (split, KV head g, batch row b), split slowest;
// split = -1 past the end.  Mixed heads: retrieval items first, then streaming ones.
struct WorkItem {
  int split, g, b;
};

__device__ inline WorkItem work_item(const DecodeParams& p, int item) {
  if (p.duo) {
    const int nr = p.B * p.Hret, ns = p.B * p.Hstr;
    const int items_ret = p.ret_splits * nr;
    if (item < items_ret) {
      const int r = item % nr;
      return {item / nr, p.duo_ret[r % p.Hret], r / p.Hret};
    }
    item -= items_ret;
    if (item >= p.str_splits * ns) return {-1, 0, 0};
    const int r = item % ns;
    return {item / ns, p.duo_str[r % p.Hstr], r / p.Hstr};
  }
  const int n_bg = p.B * p.Hkv;
  if (item >= p.n_splits * n_bg) return {-1, 0, 0};
  const int r = item % n_bg;
  return {item / n_bg, r % p.Hkv, r / p.Hkv};
}

// The cache rows one workgroup's (b, g) reads: K / V bases and attended slot count.
// Uniform caches: [B][Hkv][C][D] and n.  Mixed retrieval / streaming heads: the
// retrieval or streaming region of the head, each with its own count.
struct HeadView {
  const char* k;
  const char* v;
  int n;
};

template <typename T, int D>
__device__ inline HeadView head_view(const DecodeParams& p, int b, int g) {
  constexpr size_t row = (size_t)D * sizeof(T);
  if (p.duo) {
    const int m = p.duo_map[g];
    if (m >= 0) {
      const size_t off = ((size_t)b * p.Hret + m) * p.C * row;
      return {reinterpret_cast<const char*>(p.k) + off, reinterpret_cast<const char*>(p.v) + off, p.n};
    }
    const size_t off = ((size_t)b * p.Hstr + (-1 - m)) * p.C2 * row;
    return {reinterpret_cast<const char*>(p.k2) + off, reinterpret_cast<const char*>(p.v2) + off, p.n2};
  }
  const size_t off = ((size_t)b * p.Hkv + g) * p.C * row;
  return {reinterpret_cast<const char*>(p.k) + off, reinterpret_cast<const char*>(p.v) + off, p.n};
}

// H2O eviction candidates.  A candidate's key is (score bits << 32 | ~position): the
// minimum is the lowest score, ties to the newer token; positions are unique, so the
// minimum is unique and carries the index to evict.  Scores are >= 0, so their bits order
// like the values.
struct Victim {
  unsigned long long key = ~0ull;  // ~0: no candidate
  int at = 0;                      // slot (token granule) or block index of key
};

// Folds one slot per lane (score s, position ps, slot index i, in range) into v.  Token
// granule (bs <= 1): every slot with ps <= max_pos.  Blocks of bs = 16 or 32 slots (bs
// consecutive lanes starting at a multiple of bs, every lane active): the block's summed
// score and newest position, a candidate only if all its slots hold tokens with
// ps <= max_pos; lane 0 of the block folds it.
__device__ inline void fold_victim(Victim& v, float s, int ps, int i, bool in, int64_t max_pos, int bs, int lane) {
  if (bs <= 1) {
    if (in && (int64_t)ps <= max_pos) {
      const unsigned long long key =
          ((unsigned long long)__float_as_uint(s) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)ps);
      if (key < v.key) {
        v.key = key;
        v.at = i;
      }
    }
    return;
  }
  float sum = in ? s : 0.f;
  int mpos = in ? ps : -1;
  int bad = (!in || ps < 0 || (int64_t)ps > max_pos) ? 1 : 0;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {  // a fixed trip count keeps the callers' loops unrolled
    if (off < bs) {
      sum += __shfl_xor(sum, off, 64);
      mpos = max(mpos, __shfl_xor(mpos, off, 64));
      bad = max(bad, __shfl_xor(bad, off, 64));
    }
  }
  if ((lane & (bs - 1)) == 0 && !bad) {
    const unsigned long long key =
        ((unsigned long long)__float_as_uint(sum) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)mpos);
    if (key < v.key) {
      v.key = key;
      v.at = i / bs;
    }
  }
}

// The workgroup's minimum (256 threads; every thread calls it; wk / wa: 4 LDS entries each).
__device__ inline Victim reduce_victim(Victim v, unsigned long long* wk, int* wa) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long ok = __shfl_xor(v.key, off, 64);
    const int oa = __shfl_xor(v.at, off, 64);
    if (ok < v.key) {
      v.key = ok;
      v.at = oa;
    }
  }
  if (lane == 0) {
    wk[wave] = v.key;
    wa[wave] = v.at;
  }
  __syncthreads();
  Victim r;
  r.key = wk[0];
  r.at = wa[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (wk[w] < r.key) {
      r.key = wk[w];
      r.at = wa[w];
    }
  return r;
}

// Fused append: the workgroup whose slot range [s_begin, s_begin + cnt) holds the new
// token's slot writes its K and V rows into the cache (16-byte pieces, one per thread).
// The launch never reads that slot from the cache: its loads take the input rows.
// The slot a fused append writes for (row, KV head) bg (-1: none).
__device__ inline int new_slot_of(const DecodeParams& p, size_t bg) {
  if (!p.h2o_step || p.new_slot >= 0) return p.new_slot;
  if (p.bs <= 1) return p.victim[bg];
  return p.new_block ? p.victim[bg] * p.bs : p.open[bg] * p.bs + p.offset;
}

template <typename T, int D>
__device__ inline void write_new_rows(const DecodeParams& p, int b, int g, int slot, int s_begin, int cnt) {
  if (slot < s_begin || slot >= s_begin + cnt) return;
  constexpr int PIECES = D * (int)sizeof(T) / 16;  // per row
  const size_t src = ((size_t)b * p.Hkv + g) * D * sizeof(T);
  const size_t dst = (((size_t)b * p.Hkv + g) * p.C + slot) * D * sizeof(T);
  for (int i = threadIdx.x; i < 2 * PIECES; i += kDecodeThreads) {
    const bool is_v = i >= PIECES;
    const int piece = is_v ? i - PIECES : i;
    const char* from = reinterpret_cast<const char*>(is_v ? p.v_new : p.k_new) + src + 16 * piece;
    char* to = reinterpret_cast<char*>(is_v ? p.v : p.k) + dst + 16 * piece;
    *reinterpret_cast<u32x4*>(to) = *reinterpret_cast<const u32x4*>(from);
  }
}

// ---------------------------------------------------------------- split finish
// The end of a decode workgroup: ored[0 .. G*D) (LDS, at least 64 * G floats) holds its
// range's unnormalised output and Mh / Lh (LDS) its maximum and sum per query head.  With
// one split the output is normalised and written; otherwise the partial is published and
// the last workgroup of (b, g) to arrive merges every split (deterministic), reusing ored
// for per-split weights.  In
// logits mode the merging workgroup then runs the H2O epilogue, evicting whole blocks of
// p.bs slots when BLOCKS is set, from what each split stored per slot and query head: its
// weight 2^(x - m_s) relative to the split's maximum (WEIGHTS: the two-pass kernel, after its
// V pass) or the logit x itself (the one-pass kernel, which keeps no weights).
template <int D, int G, bool LOGITS, bool BLOCKS, bool WEIGHTS>
__device__ inline void split_finish(const DecodeParams& p, float* ored, const float* Mh, const float* Lh,
                                    int split, int n_splits, int b, int g) {
  const int lane = threadIdx.x & 63;
  const size_t bg = (size_t)b * p.Hkv + g;
  const size_t bh0 = (size_t)b * p.Hq + g * G;
  __shared__ float Mtot[G], Linv[G];
  __shared__ int is_last;
  if (n_splits == 1) {
    if (threadIdx.x < G) {
      Mtot[threadIdx.x] = Mh[threadIdx.x];
      Linv[threadIdx.x] = 1.f / Lh[threadIdx.x];
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
      store_dev(&ml[0], Mh[threadIdx.x]);
      store_dev(&ml[1], Lh[threadIdx.x]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = __hip_atomic_fetch_add(&p.arrivals[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                n_splits - 1;
    __syncthreads();
    if (!is_last) return;
    // last arrival: merge every split (fixed order, so deterministic).  The totals per
    // query head come from wave-wide reductions with one split per lane; the outputs
    // from per-split weights staged in LDS, 64 splits at a time, with the loads of
    // SU splits of each thread's EPT elements issued before their arithmetic.
    const int wave = threadIdx.x >> 6;
    float* wsp = ored;  // [64][G] weights of the current group of splits (the partial is published)
    const bool one_group = n_splits <= 64;
    if (one_group) {
      // each lane loads its split's (m, l) once, unconditionally (lanes past the splits
      // read the last one and drop it): totals and weights come from the same registers,
      // one round trip instead of three
      for (int j = wave; j < G; j += kDecodeThreads / 64) {
        const bool in = lane < n_splits;
        const float* ml = p.part_ml + ((size_t)min(lane, n_splits - 1) * BH + bh0 + j) * 2;
        const float m = load_dev(&ml[0]), l = load_dev(&ml[1]);
        const float mx = wave_max(in ? m : -INFINITY);
        const float e = in ? exp2f(m - mx) : 0.f;
        const float lt = wave_sum(in ? l * e : 0.f);
        const float linv = 1.f / lt;
        if (in) wsp[lane * G + j] = e * linv;
        if (lane == 0) {
          Mtot[j] = mx;
          Linv[j] = linv;
        }
      }
    } else {
      for (int j = wave; j < G; j += kDecodeThreads / 64) {
        float mx = -INFINITY;
        for (int s = lane; s < n_splits; s += 64) mx = fmaxf(mx, load_dev(&p.part_ml[((size_t)s * BH + bh0 + j) * 2]));
        mx = wave_max(mx);
        float lt = 0.f;
        for (int s = lane; s < n_splits; s += 64) {
          const float* ml = p.part_ml + ((size_t)s * BH + bh0 + j) * 2;
          lt += load_dev(&ml[1]) * exp2f(load_dev(&ml[0]) - mx);
        }
        lt = wave_sum(lt);
        if (lane == 0) {
          Mtot[j] = mx;
          Linv[j] = 1.f / lt;
        }
      }
    }
    __syncthreads();
    constexpr int EPT = (G * D + kDecodeThreads - 1) / kDecodeThreads;  // output elements per thread
    constexpr int SU = kMergeSu;
    float acc[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) acc[k] = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
      const int ns = min(64, n_splits - s0);
      if (!one_group) {  // (one group: staged above)
        for (int e = threadIdx.x; e < ns * G; e += kDecodeThreads) {
          const int j = e % G;
          wsp[e] = exp2f(load_dev(&p.part_ml[((size_t)(s0 + e / G) * BH + bh0 + j) * 2]) - Mtot[j]) * Linv[j];
        }
        __syncthreads();
      }
      for (int s1 = 0; s1 < ns; s1 += SU) {
        // every load in range and unconditional (past the splits: the last split's partial,
        // dropped below), so none waits for another: a load under a branch would make the
        // compiler wait for it at the branch's end
        float x[SU][EPT];
#pragma unroll
        for (int u = 0; u < SU; ++u)
#pragma unroll
          for (int k = 0; k < EPT; ++k) {
            const int idx = min((int)threadIdx.x + k * kDecodeThreads, G * D - 1);
            const int sp = min(s0 + s1 + u, n_splits - 1);
            x[u][k] = load_dev(&p.part_o[((size_t)sp * BH + bh0) * D + idx]);
          }
#pragma unroll
        for (int u = 0; u < SU; ++u)
#pragma unroll
          for (int k = 0; k < EPT; ++k) {
            const int idx = min((int)threadIdx.x + k * kDecodeThreads, G * D - 1);
            const int su = min(s1 + u, ns - 1);  // an in-range weight (the select drops it)
            const float t = fmaf(x[u][k], wsp[su * G + idx / D], acc[k]);
            acc[k] = s1 + u < ns ? t : acc[k];
          }
      }
      __syncthreads();  // wsp is rewritten by the next group
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int idx = threadIdx.x + k * kDecodeThreads;
      if (idx < G * D) p.out[bh0 * D + idx] = acc[k];
    }
    if (threadIdx.x == 0)  // ready for the next call
      __hip_atomic_store(&p.arrivals[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (LOGITS) {
    // H2O: add this step's weights (summed over the group's query heads) to every
    // filled slot's score and pick what the next append overwrites: the lowest score
    // among slots (or blocks of slots) of tokens with pos <= max_pos, ties evicting the
    // newer token.  The loop bound is wave-uniform so block reductions see whole waves.
    __shared__ unsigned long long wkey[4];
    __shared__ int wat[4];
    // The stored values are the splits' weights 2^(x - m_s) (WEIGHTS) or the logits x.
    // Split s's weight for query head j, 2^(m_s - M) / L, is read from LDS at
    // ored[(s - s_lo) * G + j]: the merge left those of up to 64 splits there (s_lo = 0);
    // one split has 1 / L; with more than 64 each iteration stages those of its own slots'
    // splits (at most 65) from the published (m, l).
    constexpr int IT = kDecodeThreads * EU_OF<BLOCKS>();  // slots per iteration
    if (n_splits == 1) {
      __builtin_amdgcn_s_waitcnt(0);  // this workgroup's stores of the values have completed
      __syncthreads();                // (and every thread is done with ored)
      if constexpr (WEIGHTS) {
        if (threadIdx.x < G) ored[threadIdx.x] = Linv[threadIdx.x];
        __syncthreads();
      }
    }
    float* score = p.score + bg * p.C;
    int* pos = const_cast<int*>(p.pos) + bg * p.C;
    // a fused append's slot holds the new token (score 0 before this step's weight) and a
    // reopened block's other slots are empty: this workgroup is the only writer of the
    // position and score arrays in the launch, so it takes those values as known
    const int nslot = p.h2o_step ? new_slot_of(p, bg) : -1;
    const int emp_end = p.h2o_step && p.new_block ? nslot + p.bs : -1;
    Victim best;
    const int bs = BLOCKS ? p.bs : 1;  // eviction granule
    constexpr int EU = EU_OF<BLOCKS>();  // slots per thread per iteration, all loads issued first
    // the iteration count is the workgroup's (waves past n run with every slot out of range),
    // so that weight staging can use barriers and block reductions see whole waves
    for (int it0 = 0; it0 < p.n; it0 += IT) {
      const int base = it0 + (int)threadIdx.x - lane;
      const int i0 = base + lane;
      int s_lo = 0;
      if constexpr (WEIGHTS) {
        if (n_splits > 64) {  // workgroup-uniform
          s_lo = it0 / p.chunk;
          const int ns = min(n_splits, (it0 + IT - 1) / p.chunk + 1) - s_lo;
          const size_t BHq = (size_t)p.B * p.Hq;
          __syncthreads();  // the previous iteration's reads are done
          for (int e = threadIdx.x; e < ns * G; e += kDecodeThreads) {
            const int sp = s_lo + e / G, j = e % G;
            ored[e] = exp2f(load_dev(&p.part_ml[((size_t)sp * BHq + bh0 + j) * 2]) - Mtot[j]) * Linv[j];
          }
          __syncthreads();
        }
      }
      float x[EU][G], sc[EU];
      int ps[EU];
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        // unconditional loads (slots past n read slot n - 1; their values are not used),
        // so that no branch separates a load from its use
        const int ic = min(i0 + u * kDecodeThreads, p.n - 1);
#pragma unroll
        for (int j = 0; j < G; ++j) x[u][j] = load_dev(&p.logits[(bh0 + j) * p.C + ic]);
        sc[u] = score[ic];
        ps[u] = pos[ic];
      }
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        const int ic = i0 + u * kDecodeThreads;
        const bool fresh = ic == nslot, emptied = ic > nslot && ic < emp_end;
        sc[u] = fresh || emptied ? 0.f : sc[u];
        ps[u] = fresh ? (int)p.token : emptied ? -1 : ps[u];
      }
      // arithmetic and victim folds first, the score stores last: a store issued before
      // a later branch would make the compiler's wait at that branch cover it too
      float snew[EU];
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        const bool in = i0 + u * kDecodeThreads < p.n;
        float a = 0.f;
        if constexpr (WEIGHTS) {
          const float* w = ored + (min(i0 + u * kDecodeThreads, p.n - 1) / p.chunk - s_lo) * G;
#pragma unroll
          for (int j = 0; j < G; ++j) a += x[u][j] * w[j];
        } else {
#pragma unroll
          for (int j = 0; j < G; ++j) a += exp2f(x[u][j] - Mtot[j]) * Linv[j];
        }
        snew[u] = in ? sc[u] + a : 0.f;
      }
      if (p.pick_victim) {
#pragma unroll
        for (int u = 0; u < EU; ++u) {
          const int i = i0 + u * kDecodeThreads;
          if (base + u * kDecodeThreads < p.n)  // wave-uniform
            fold_victim(best, snew[u], ps[u], i, i < p.n, p.max_pos, bs, lane);
        }
      }
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        const int i = i0 + u * kDecodeThreads;
        if (i < p.n) score[i] = snew[u];
      }
    }
    if (p.pick_victim) {
      const Victim v = reduce_victim(best, wkey, wat);
      if (threadIdx.x == 0 && v.key != ~0ull) p.victim[bg] = v.at;
    }
    if (p.h2o_step) {  // the fused append's position record (and a reopened block's)
      if (threadIdx.x == 0) {
        pos[nslot] = (int)p.token;
        if (p.new_block) p.open[bg] = nslot / p.bs;
      }
      if (p.new_block && threadIdx.x > 0 && (int)threadIdx.x < p.bs) pos[nslot + threadIdx.x] = -1;
    }
  }
}

// ---------------------------------------------------------------- one-pass kernel
// For up to 2 query heads per KV head (registers hold the queries and the outputs
// together).
template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(kDecodeThreads) decode_onepass_kernel(DecodeParams p) {
  constexpr bool ROPE = MODE == kModeRope;
  constexpr bool LOGITS = MODE == kModePlainLogits || MODE == kModeMaskedLogits;
  constexpr bool MASKED = MODE == kModeMaskedLogits;
  using GE = Geo<T, D, G>;
  constexpr int W = GE::W, HALF = GE::HALF, EPL = GE::EPL, LPK = GE::LPK, KPW = GE::KPW, KPI = GE::KPI;
  constexpr int U = GE::U, STEP = GE::STEP;
  constexpr int D2 = D / 2;
  using E = Elem<T, W>;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* ored = smem;                 // [4][G][D] the waves' outputs, then [G][D] their merge
  float* wm = ored + 4 * G * D;       // [4][G] the waves' maxima
  float* wl = wm + 4 * G;             // [4][G] the waves' sums
  float* wsc = wl + 4 * G;            // [4][G] the waves' weights 2^(m_w - m)
  float* Mh = wsc + 4 * G;            // [G] the workgroup's maxima
  float* Lh = Mh + G;                 // [G] the workgroup's sums

  // Workgroups are dealt round-robin to the 8 XCDs, so linear id w runs on XCD
  // w % 8.  Give each XCD a contiguous run of (split, kv-head, batch) items, split
  // slowest: the workgroups resident on one XCD then share a slot range and its
  // slice of the position table stays in that XCD's L2.
  const int per_xcd = (int)((gridDim.x + 7) / 8);
  const WorkItem wi = work_item(p, (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8));
  if (wi.split < 0) return;  // padding of the grid to a multiple of 8
  const int split = wi.split, g = wi.g, b = wi.b;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kg = lane / LPK;
  const int i0 = sub * HALF;  // first pair index owned by this lane
  const HeadView hv = head_view<T, D>(p, b, g);
  const int s_begin = split * p.chunk;
  if (s_begin >= hv.n) return;  // never taken: every listed item holds at least one slot
  const int n_splits = (hv.n + p.chunk - 1) / p.chunk;
  const int cnt = min(hv.n - s_begin, p.chunk);
  const char* kbase = hv.k;
  const char* vbase = hv.v;
  const size_t lo_off = (size_t)i0 * sizeof(T);
  const size_t hi_off = (size_t)(D2 + i0) * sizeof(T);
  // fused append: the new token's rows come from the input (the slot is written below)
  const int nslot = new_slot_of(p, (size_t)b * p.Hkv + g);
  const int new_key = nslot - s_begin;  // key index of the new slot (outside 0..cnt-1 if none here)
  const size_t new_row = ((size_t)b * p.Hkv + g) * D * sizeof(T);
  write_new_rows<T, D>(p, b, g, nslot, s_begin, cnt);
  // H2O blocks: a freed block reopened by this step holds only the new token
  const int emp_lo = p.new_block ? new_key : INT_MAX, emp_hi = p.new_block ? new_key + p.bs : INT_MIN;

  // ---- queries of the group: load, rotate at the query's position, pre-scale (without
  // RoPE, bf16 queries stay packed for v_dot2_f32_bf16, as in the two-pass kernel)
  constexpr bool DOT2 = !ROPE && sizeof(T) == 2;
  float qf[G][EPL];
  Words<W> qlo[G], qhi[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const char* qrow = reinterpret_cast<const char*>(p.q) + ((size_t)b * p.Hq + g * G + j) * D * sizeof(T);
    if constexpr (DOT2) {
      qlo[j] = load_words<W>(qrow + lo_off);
      qhi[j] = load_words<W>(qrow + hi_off);
      continue;
    }
    float lo[HALF], hi[HALF];
    E::cvt(load_words<W>(qrow + lo_off), lo);
    E::cvt(load_words<W>(qrow + hi_off), hi);
    if constexpr (ROPE) {
      float c[HALF], s[HALF];
      load_floats<HALF>(p.cos_t + (size_t)p.q_rank * D2 + i0, c);
      load_floats<HALF>(p.sin_t + (size_t)p.q_rank * D2 + i0, s);
#pragma unroll
      for (int e = 0; e < HALF; ++e) {
        const float a = lo[e], bb = hi[e];
        lo[e] = a * c[e] - bb * s[e];
        hi[e] = a * s[e] + bb * c[e];
      }
    }
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      qf[j][e] = lo[e] * p.qscale;
      qf[j][HALF + e] = hi[e] * p.qscale;
    }
  }

  // ---- RoPE angles of the keys.  With few query heads (G <= 2, where the kernel is
  // far from ALU-bound) a lane group's keys sit KPI slots apart, and where their in-cache
  // positions are also KPI apart (everywhere except across the ring's wrap point and the
  // sink boundary) the cos/sin of a key follow from the previous key's by one angle
  // addition with the per-lane constant rotation (cos, sin)(KPI * theta_i), across
  // iterations too: a table row is read only in every other iteration (an anchor), and
  // waves whose keys break the rank sequence read every key's row.  With more query heads
  // every key reads its own row (the split's table slice stays in its XCD's L2).
  constexpr bool REC = ROPE && G <= 2;
  constexpr int NCS = ROPE ? (REC ? 1 : U) : 1;  // table rows held per iteration
  float dc[HALF], ds[HALF];
  if constexpr (REC) {
    load_floats<HALF>(p.cos_t + (size_t)KPI * D2 + i0, dc);
    load_floats<HALF>(p.sin_t + (size_t)KPI * D2 + i0, ds);
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
    load_floats<HALF>(p.cos_t + (size_t)rank * D2 + i0, c);
    load_floats<HALF>(p.sin_t + (size_t)rank * D2 + i0, sn);
  };
  auto advance = [&](float (&c)[HALF], float (&sn)[HALF]) {  // by KPI ranks
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      const float cc = c[e] * dc[e] - sn[e] * ds[e];
      sn[e] = sn[e] * dc[e] + c[e] * ds[e];
      c[e] = cc;
    }
  };

  // one iteration's registers: the raw K and V pieces of U keys, and the table rows
  struct Buf {
    Words<W> klo[U], khi[U], vlo[U], vhi[U];
    float c[NCS][HALF], sn[NCS][HALF];
    int mp[U];  // H2O blocks: the slots' positions (< 0: empty)
  };
  // TABLE: an anchor iteration, which also loads its first key's table row
  auto load_iter = [&](int base, Buf& bf, auto table) {
    constexpr bool TABLE = decltype(table)::value;
    const int key0 = base + wave * KPW + kg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // keys past the range load the range's last row (their logits are masked and their
      // weights are 0): no branch around the loads, so the compiler counts this set's
      // loads exactly and leaves them in flight while the previous set is consumed
      const int key = min(key0 + u * KPI, cnt - 1);
      const bool fresh = key == new_key;
      const char* krow = fresh ? reinterpret_cast<const char*>(p.k_new) + new_row
                               : kbase + (size_t)(s_begin + key) * D * sizeof(T);
      const char* vrow = fresh ? reinterpret_cast<const char*>(p.v_new) + new_row
                               : vbase + (size_t)(s_begin + key) * D * sizeof(T);
      bf.klo[u] = load_words<W>(krow + lo_off);
      bf.khi[u] = load_words<W>(krow + hi_off);
      bf.vlo[u] = load_words<W>(vrow + lo_off);
      bf.vhi[u] = load_words<W>(vrow + hi_off);
    }
    if constexpr (MASKED) {  // an in-range index for every lane, then a select on the value
      const int* mrow = p.mask_pos + ((size_t)b * p.Hkv + g) * p.C + s_begin;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = key0 + u * KPI;
        const int v = mrow[min(key, cnt - 1)];
        // the new token's slot is filled; the rest of a reopened block is empty
        bf.mp[u] = key >= cnt ? -1 : key == new_key ? 0 : (key > emp_lo && key < emp_hi) ? -1 : v;
      }
    }
    if constexpr (ROPE && (TABLE || !REC)) {
#pragma unroll
      for (int u = 0; u < NCS; ++u) load_cs(rank_of(s_begin + min(key0 + u * KPI, cnt - 1)), bf.c[u], bf.sn[u]);
    }
  };
  // REC: the table row of the lane group's current key and its rank
  float rc[HALF], rs[HALF];
  int rrank = 0;

  // running softmax state of this lane group (identical in its LPK lanes)
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
  }

  auto compute_iter = [&](int base, Buf& bf, auto anchor) {
    constexpr bool ANCHOR = decltype(anchor)::value;
    const int key0 = base + wave * KPW + kg;
    bool stepwise = false;  // REC: this wave's keys break the rank sequence
    int rk[U];              // REC: the keys' ranks
    if constexpr (REC) {
      // an anchor starts at its loaded row; otherwise the first key continues the previous
      // iteration's last one
      const int rank0 = ANCHOR ? rank_of(s_begin + min(key0, cnt - 1)) : rrank + KPI;
      bool disc = false;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = key0 + u * KPI;
        rk[u] = rank_of(s_begin + min(key, cnt - 1));
        if (u > 0 || !ANCHOR) disc |= key < cnt && rk[u] != rank0 + u * KPI;
      }
      stepwise = __any(disc);
    }
    // dot products of the U keys with the G queries, then their lane-group sums in one
    // interleaved pass
    float d[U * G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (DOT2) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qlo[j].w[w]),
                                                  __builtin_bit_cast(bf16x2, bf.klo[u].w[w]), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qhi[j].w[w]),
                                                  __builtin_bit_cast(bf16x2, bf.khi[u].w[w]), acc, false);
          }
          d[u * G + j] = acc;
        }
        continue;
      }
      float kf[EPL];
      {
        float lo[HALF], hi[HALF];
        E::cvt(bf.klo[u], lo);
        E::cvt(bf.khi[u], hi);
        if constexpr (REC) {
          if (u == 0 && ANCHOR) {
#pragma unroll
            for (int e = 0; e < HALF; ++e) {
              rc[e] = bf.c[0][e];
              rs[e] = bf.sn[0][e];
            }
          } else if (stepwise) {
            load_cs(rk[u], rc, rs);
            wait_loads();  // complete here, so the common path keeps the next set's loads in flight
          } else if (u > 0) {
            advance(rc, rs);
          }  // (u = 0 otherwise: advanced after the previous iteration)
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            kf[e] = lo[e] * rc[e] - hi[e] * rs[e];
            kf[HALF + e] = lo[e] * rs[e] + hi[e] * rc[e];
          }
        } else if constexpr (ROPE) {
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            kf[e] = lo[e] * bf.c[u][e] - hi[e] * bf.sn[u][e];
            kf[HALF + e] = lo[e] * bf.sn[u][e] + hi[e] * bf.c[u][e];
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
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[j][e], kf[e], acc);
        d[u * G + j] = acc;
      }
    }
    if constexpr (REC) {  // the row of the next iteration's first key
      advance(rc, rs);
      rrank = (stepwise ? rk[U - 1] : (ANCHOR ? rk[0] : rrank + KPI) + (U - 1) * KPI);
    }
    group_sum_n<LPK, U * G>(d);
    if constexpr (DOT2) {
#pragma unroll
      for (int i = 0; i < U * G; ++i) d[i] *= p.qscale;
    }

    // mask the keys past the range, record logits (H2O), new running maxima
    float mn[G];
#pragma unroll
    for (int j = 0; j < G; ++j) mn[j] = m[j];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = key0 + u * KPI;
      bool valid = key < cnt;
      if constexpr (MASKED) valid = valid && bf.mp[u] >= 0;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        d[u * G + j] = valid ? d[u * G + j] : -INFINITY;
        mn[j] = fmaxf(mn[j], d[u * G + j]);
      }
      if constexpr (LOGITS) {  // masked (empty) slots store -inf: their weight is 0
        if (key < cnt && sub == 0) {
#pragma unroll
          for (int j = 0; j < G; ++j)
            store_dev(&p.logits[((size_t)b * p.Hq + g * G + j) * p.C + s_begin + key], d[u * G + j]);
        }
      }
    }
    // rescale the running sums only when some maximum of the wave grew (rare after the
    // first iterations); a group that has seen no key yet keeps m = -inf and scale 1
    bool grow = false;
#pragma unroll
    for (int j = 0; j < G; ++j) grow |= mn[j] > m[j];
    if (__any(grow)) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float corr = mn[j] == -INFINITY ? 1.f : exp2_weight(m[j] - mn[j]);
        m[j] = mn[j];
        l[j] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] *= corr;
      }
    }
    // weights p = 2^(x - m) (0 for masked keys) and the V accumulation
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float x = d[u * G + j];
        const float pw = x == -INFINITY ? 0.f : exp2_weight(x - m[j]);
        d[u * G + j] = pw;
        l[j] += pw;
      }
      float lo[HALF], hi[HALF];
      E::cvt(bf.vlo[u], lo);
      E::cvt(bf.vhi[u], hi);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float pw = d[u * G + j];
#pragma unroll
        for (int e = 0; e < HALF; ++e) {
          o[j][e] = fmaf(pw, lo[e], o[j][e]);
          o[j][HALF + e] = fmaf(pw, hi[e], o[j][HALF + e]);
        }
      }
    }
  };

  // ---- the pass: two register sets alternate, the next iteration's loads are issued
  // before this iteration's arithmetic (a third set measured no faster)
  {
    const std::true_type yes{};  // A's iterations are the anchors
    const std::false_type no{};
    Buf A, B;
    load_iter(0, A, yes);
    for (int base = 0; base < cnt; base += 2 * STEP) {
      load_iter(base + STEP, B, no);  // unconditional (past the range: clamped rows)
      compute_iter(base, A, yes);
      if (base + STEP >= cnt) break;
      load_iter(base + 2 * STEP, A, yes);
      compute_iter(base + STEP, B, no);
    }
  }

  // ---- merge the lane groups of each wave at the wave's maximum, then the 4 waves
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mw = m[j];
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off, 64));
    const float sc = m[j] == -INFINITY ? 0.f : exp2f(m[j] - mw);
    float lw = l[j] * sc;
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) lw += __shfl_xor(lw, off, 64);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = o[j][e] * sc;
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      o[j][e] = x;
    }
    if (lane == 0) {
      wm[wave * G + j] = mw;
      wl[wave * G + j] = lw;
    }
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
  // the workgroup's (m, l) per head and the waves' weights, then the merged output
  if (threadIdx.x < G) {
    const int j = threadIdx.x;
    const float M = fmaxf(fmaxf(wm[j], wm[G + j]), fmaxf(wm[2 * G + j], wm[3 * G + j]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mwv = wm[w * G + j];
      const float s = mwv == -INFINITY ? 0.f : exp2f(mwv - M);
      wsc[w * G + j] = s;
      L += wl[w * G + j] * s;
    }
    Mh[j] = M;
    Lh[j] = L;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {  // each thread reads only its idx
    const int j = idx / D;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += ored[w * G * D + idx] * wsc[w * G + j];
    ored[idx] = acc;
  }
  __syncthreads();
  split_finish<D, G, LOGITS, MASKED, false>(p, ored, Mh, Lh, split, n_splits, b, g);
}

// ---------------------------------------------------------------- two-pass kernel
// For 4 or more query heads per KV head.  K pass: every key of the range is loaded
// once, rotated, dotted with the G queries; logits go to LDS.  Softmax: the range
// maximum per query head, p = 2^(x - m) in LDS, l = sum p.  V pass: every value row is
// loaded once and accumulated with the G weights, on the matrix cores for bf16 values.
// Registers then hold either the queries (K pass) or the outputs (V pass), never both,
// which keeps G * D-sized state within two waves per SIMD at 16-byte pieces.
//
// The K pass takes G multiply-adds per key element (against one byte loaded per 1/2
// element), which makes it VALU-heavy, so its loop carries no per-key
// work beyond that arithmetic: rows are addressed by 32-bit offsets from the range's
// uniform base, a fused append's rows are written to the cache before the passes (so no
// load selects between cache and input), in-cache positions come from the range's two
// precomputed rank breakpoints, and only the last, partial iteration of each pass tests
// keys against the end of the range.
template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(kDecodeThreads) decode_twopass_kernel(DecodeParams p) {
  constexpr bool ROPE = MODE == kModeRope;
  constexpr bool LOGITS = MODE == kModePlainLogits || MODE == kModeMaskedLogits;
  constexpr bool MASKED = MODE == kModeMaskedLogits;
  using E = Elem<T, 4>;
  constexpr int HALF = E::N;
  constexpr int EPL = 2 * HALF;    // elements per lane (HALF pairs)
  constexpr int LPK = D / EPL;     // lanes per key
  constexpr int KPW = 64 / LPK;    // keys per wave per sub-step
  constexpr int KPI = 4 * KPW;     // keys per workgroup per sub-step
  constexpr int D2 = D / 2;
  constexpr uint32_t ROW = D * sizeof(T);  // bytes per cache row
  static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "lane mapping");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int XS = p.chunk + kXsPad;  // row stride of xs
  const int region = (XS * G > 4 * G * D ? XS * G : 4 * G * D);
  float* xs = smem;                 // [G][XS] logits, then weights
  float* ored = smem;               // [4][G][D] the waves' outputs (after the V pass), then [G][D]
  float* red = smem + region;       // [4][U * G] / [4][G] cross-wave reductions (kTwopassRed floats)
  float* Mh = red + kTwopassRed;    // [G] the range's maxima
  float* Lh = Mh + G;               // [G] the range's sums

  // XCD-aware item order (see the one-pass kernel)
  const int per_xcd = (int)((gridDim.x + 7) / 8);
  const WorkItem wi = work_item(p, (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8));
  if (wi.split < 0) return;  // padding of the grid to a multiple of 8
  const int split = wi.split, g = wi.g, b = wi.b;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
  const int sub = lane % LPK, kg = lane / LPK;
  const int i0 = sub * HALF;  // first pair index owned by this lane
  const HeadView hv = head_view<T, D>(p, b, g);
  const int s_begin = split * p.chunk;
  if (s_begin >= hv.n) return;  // never taken: every listed item holds at least one slot
  const int n_splits = (hv.n + p.chunk - 1) / p.chunk;
  const int cnt = min(hv.n - s_begin, p.chunk);
  // the range's rows: uniform bases and 32-bit offsets (a range spans at most
  // chunk * ROW < 2^24 bytes)
  const char* kw = hv.k + (size_t)s_begin * ROW;
  const char* vw = hv.v + (size_t)s_begin * ROW;
  const uint32_t lo_off = (uint32_t)i0 * sizeof(T);
  const uint32_t hi_off = (uint32_t)(D2 + i0) * sizeof(T);
  // fused append: the workgroup whose range holds the new token's slot writes its K and
  // V rows into the cache first; after the barrier its loads read them like any other
  // row (the stores have completed and the waves share the CU's caches)
  const int nslot = new_slot_of(p, (size_t)b * p.Hkv + g);
  if (nslot >= s_begin && nslot < s_begin + cnt) {  // workgroup-uniform
    write_new_rows<T, D>(p, b, g, nslot, s_begin, cnt);
    __threadfence_block();
    __syncthreads();
  }
  // H2O blocks: a freed block reopened by this step holds only the new token
  const int new_key = nslot - s_begin;
  const int emp_lo = p.new_block ? new_key : INT_MAX, emp_hi = p.new_block ? new_key + p.bs : INT_MIN;
  // LDS staging area of the bf16 V pass (16 KiB: 4 waves x 32 rows x 128 bytes).  Until the
  // V pass it holds the H2O block cache's slot positions of the range (at most 4096 with
  // the chunk cap), so that the K pass reads them from LDS instead of issuing a global load
  // per key beside its K rows.
  constexpr bool MV = sizeof(T) == 2;
  constexpr int kStageBytes = 4 * 32 * 128;
  __shared__ __attribute__((aligned(16))) char vstage[MV || MASKED ? kStageBytes : 16];
  const int* msk = reinterpret_cast<const int*>(vstage);
  if constexpr (MASKED) {
    const int* mrow = p.mask_pos + ((size_t)b * p.Hkv + g) * p.C + s_begin;
    for (int i = threadIdx.x; i < cnt; i += kDecodeThreads) reinterpret_cast<int*>(vstage)[i] = mrow[i];
    __syncthreads();
  }

  // ---- queries of the group: load, rotate at the query's position, pre-scale.  Without
  // RoPE, bf16 queries stay packed: the K pass takes exact bf16 x bf16 pair products
  // with float32 sums (v_dot2_f32_bf16) and scales after the lane-group reduction.
  constexpr bool DOT2 = !ROPE && sizeof(T) == 2;
  float qf[G][EPL];
  Words<4> qlo[G], qhi[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const char* qrow = reinterpret_cast<const char*>(p.q) + ((size_t)b * p.Hq + g * G + j) * ROW;
    if constexpr (DOT2) {
      qlo[j] = load_words<4>(qrow + lo_off);
      qhi[j] = load_words<4>(qrow + hi_off);
      continue;
    }
    float lo[HALF], hi[HALF];
    E::cvt(load_words<4>(qrow + lo_off), lo);
    E::cvt(load_words<4>(qrow + hi_off), hi);
    if constexpr (ROPE) {
      float c[HALF], s[HALF];
      load_floats<HALF>(p.cos_t + (size_t)p.q_rank * D2 + i0, c);
      load_floats<HALF>(p.sin_t + (size_t)p.q_rank * D2 + i0, s);
#pragma unroll
      for (int e = 0; e < HALF; ++e) {
        const float a = lo[e], bb = hi[e];
        lo[e] = a * c[e] - bb * s[e];
        hi[e] = a * s[e] + bb * c[e];
      }
    }
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      qf[j][e] = lo[e] * p.qscale;
      qf[j][HALF + e] = hi[e] * p.qscale;
    }
  }

  // ---- in-cache positions.  A slot's position is its number, except in a wrapped ring:
  // there rank = slot + (slot >= S ? W - head : 0) - (slot >= S + head ? W : 0) with head
  // the ring index of the oldest window token, i.e. two breakpoints in the range's key
  // index, kb1 at the sink boundary and kb2 at the oldest token's slot (with head = 0
  // the two jumps cancel and there are none).
  int kb1 = INT_MAX, kb2 = INT_MAX;
  if (ROPE && p.full && p.ring_head > 0) {
    kb1 = p.S - s_begin;
    kb2 = p.S + p.ring_head - s_begin;
  }
  const int jump1 = p.W - p.ring_head;
  auto rank_of_key = [&](int key) { return s_begin + key + (key >= kb1 ? jump1 : 0) - (key >= kb2 ? p.W : 0); };
  // table rows by 32-bit byte offsets from the uniform table bases (the host keeps a
  // rotated cache's table below 4 GiB)
  const char* cos_b = reinterpret_cast<const char*>(p.cos_t);
  const char* sin_b = reinterpret_cast<const char*>(p.sin_t);
  auto load_cs = [&](int rank, float (&c)[HALF], float (&sn)[HALF]) {
    const uint32_t off = ((uint32_t)rank * D2 + (uint32_t)i0) * (uint32_t)sizeof(float);
    load_floats<HALF>(reinterpret_cast<const float*>(cos_b + off), c);
    load_floats<HALF>(reinterpret_cast<const float*>(sin_b + off), sn);
  };

  // ---- K pass: U keys per lane group per iteration, the next iteration's loads issued
  // before this iteration's arithmetic (two register sets alternate; G = 8 has room for
  // one).  RoPE: a lane group's keys of consecutive iterations are KPI slots apart, and
  // (except across a rank breakpoint) so are their ranks, so each key's table row is the
  // previous key's advanced by angle addition of (cos, sin)(KPI * theta_i).  A row is read
  // from the table only in every other iteration (an anchor, which bounds the rounding
  // carried along to 2U - 1 additions) and wherever the recurrence would cross a
  // breakpoint: table loads share the K rows' load path, and one row per iteration made the
  // GQA launch 3.5% slower (one per key, slower still; one per four iterations, no faster).
  constexpr int U = G <= 4 ? (ROPE ? 3 : 4) : 2;
  static_assert(U * G % 4 == 0 && U * G <= 16, "lane-group sums leave U * G / 4 values per lane");
  constexpr bool REC = ROPE;
  constexpr int STEP = KPI * U;
  float dc[HALF], ds[HALF];
  if constexpr (REC) {
    load_floats<HALF>(p.cos_t + (size_t)KPI * D2 + i0, dc);
    load_floats<HALF>(p.sin_t + (size_t)KPI * D2 + i0, ds);
  }
  constexpr int NC = REC ? 1 : (ROPE ? U : 1);  // table rows held per iteration
  struct KBuf {
    Words<4> lo[U], hi[U];
    float c[NC][HALF], sn[NC][HALF];  // RoPE: table rows (with angle additions: the first key's)
    int mp[U];                        // H2O blocks: the slots' positions (< 0: empty)
  };
  // TABLE: an anchor iteration, which also loads its first key's table row
  auto load_iter = [&](int base, KBuf& bf, auto table) {
    constexpr bool TABLE = decltype(table)::value;
    const int key0 = base + wave * KPW + kg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // keys past the range load the range's last row (masked in the last iteration), so
      // no branch separates the loads from their use
      const uint32_t off = (uint32_t)min(key0 + u * KPI, cnt - 1) * ROW;
      bf.lo[u] = load_words<4>(kw + (off + lo_off));
      bf.hi[u] = load_words<4>(kw + (off + hi_off));
    }
    if constexpr (MASKED) {  // an in-range index for every lane, then a select on the value
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = key0 + u * KPI;
        const int v = msk[min(key, cnt - 1)];
        // the new token's slot is filled; the rest of a reopened block is empty
        bf.mp[u] = key >= cnt ? -1 : key == new_key ? 0 : (key > emp_lo && key < emp_hi) ? -1 : v;
      }
    }
    if constexpr (ROPE && TABLE) {
#pragma unroll
      for (int u = 0; u < NC; ++u) load_cs(rank_of_key(min(key0 + u * KPI, cnt - 1)), bf.c[u], bf.sn[u]);
    }
  };
  // does this wave's set of keys at `base` straddle a rank breakpoint (wave-uniform)?
  auto straddles = [&](int base) {
    const int lo = base + wave * KPW, hi = lo + KPW - 1 + (U - 1) * KPI;
    return (kb1 > lo && kb1 <= hi) || (kb2 > lo && kb2 <= hi);
  };
  // does a breakpoint lie between the wave's keys of the previous iteration and this one's
  // first keys (wave-uniform)?
  auto jumps_before = [&](int base) {
    const int lo = base + wave * KPW - KPI, hi = base + wave * KPW + KPW - 1;
    return (kb1 > lo && kb1 <= hi) || (kb2 > lo && kb2 <= hi);
  };
  auto advance = [&](float (&c)[HALF], float (&sn)[HALF]) {  // by KPI ranks
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
      const float cc = c[e] * dc[e] - sn[e] * ds[e];
      sn[e] = sn[e] * dc[e] + c[e] * ds[e];
      c[e] = cc;
    }
  };
  float rc[HALF], rs[HALF];  // RoPE: the table row of the lane group's current key
  // after the lane-group sums a lane holds NF = U * G / 4 of the iteration's U * G logits:
  // value index vbase + i, i.e. key step slot_u[i] and query head slot_j[i]; the lanes that
  // hold totals and write them ("writers") are one per index class of each key group
  constexpr int NV = U * G, NF = NV / 4;
  const int vbase = (lane & 1) * (NV / 2) + ((lane >> 1) & 1) * (NV / 4);
  const bool writer = LPK == 8 ? (sub & 4) != 0 : sub < 4;
  int slot_u[NF], slot_j[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    slot_u[i] = (vbase + i) / G;
    slot_j[i] = (vbase + i) % G;
  }
  float mxs[NF];  // running maxima of this lane's value slots
#pragma unroll
  for (int i = 0; i < NF; ++i) mxs[i] = -INFINITY;
  auto compute_iter = [&](int base, KBuf& bf, auto tail, auto anchor) {
    constexpr bool TAIL = decltype(tail)::value;  // keys may lie past the range
    constexpr bool ANCHOR = decltype(anchor)::value;
    const int key0 = base + wave * KPW + kg;
    bool stepwise = false, gap = false;
    if constexpr (REC) {
      stepwise = straddles(base);
      if constexpr (!ANCHOR) gap = jumps_before(base);
    }
    float d[U * G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (DOT2) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qlo[j].w[w]),
                                                  __builtin_bit_cast(bf16x2, bf.lo[u].w[w]), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qhi[j].w[w]),
                                                  __builtin_bit_cast(bf16x2, bf.hi[u].w[w]), acc, false);
          }
          d[u * G + j] = acc;
        }
        continue;
      }
      float kf[EPL];
      {
        float lo[HALF], hi[HALF];
        E::cvt(bf.lo[u], lo);
        E::cvt(bf.hi[u], hi);
        if constexpr (ROPE) {
          if (u == 0) {
            if constexpr (ANCHOR) {
#pragma unroll
              for (int e = 0; e < HALF; ++e) {
                rc[e] = bf.c[0][e];
                rs[e] = bf.sn[0][e];
              }
            } else if (gap) {
              load_cs(rank_of_key(min(key0, cnt - 1)), rc, rs);
              wait_loads();  // complete here, so the common path keeps the next set's loads in flight
            }  // else rc / rs already hold this key's row (advanced after the previous iteration)
          } else if (stepwise) {
            load_cs(rank_of_key(min(key0 + u * KPI, cnt - 1)), rc, rs);
            wait_loads();
          } else {
            advance(rc, rs);
          }
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            kf[e] = lo[e] * rc[e] - hi[e] * rs[e];
            kf[HALF + e] = lo[e] * rs[e] + hi[e] * rc[e];
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
        float acc = qf[j][0] * kf[0];  // (starting from a product, not a zeroed register)
#pragma unroll
        for (int e = 1; e < EPL; ++e) acc = fmaf(qf[j][e], kf[e], acc);
        d[u * G + j] = acc;
      }
    }
    if constexpr (REC) advance(rc, rs);  // the row of the next iteration's first key
    // keys past the range (last iteration) and empty slots of a block cache: logit -inf in
    // every lane of the group, so their totals are -inf
    if constexpr (TAIL || MASKED) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bool dead = false;
        if constexpr (TAIL) dead = key0 + u * KPI >= cnt;
        if constexpr (MASKED) dead = dead || bf.mp[u] < 0;
#pragma unroll
        for (int j = 0; j < G; ++j) d[u * G + j] = dead ? -INFINITY : d[u * G + j];
      }
    }
    group_sum_transposed<LPK, NV>(d, lane);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if constexpr (DOT2) d[i] *= p.qscale;
      mxs[i] = fmaxf(mxs[i], d[i]);
    }
    if (writer) {
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int key = key0 + slot_u[i] * KPI;
        if (!TAIL || key < cnt) {
          xs[slot_j[i] * XS + key] = d[i];
        }
      }
    }
  };
  {
    constexpr bool KPF = G <= 6;
    if constexpr (KPF) {
      // A's iterations are the anchors
      const std::true_type yes{};
      const std::false_type no{};
      KBuf A, B;
      load_iter(0, A, yes);
      int base = 0;
      for (; base + 2 * STEP <= cnt; base += 2 * STEP) {  // both iterations wholly inside the range
        load_iter(base + STEP, B, no);
        compute_iter(base, A, no, yes);
        load_iter(base + 2 * STEP, A, yes);  // unconditional (past the range: clamped rows)
        compute_iter(base + STEP, B, no, no);
      }
      if (base < cnt) {  // one or two more iterations, the last partial
        load_iter(base + STEP, B, no);
        compute_iter(base, A, yes, yes);
        if (base + STEP < cnt) compute_iter(base + STEP, B, yes, no);
      }
    } else {  // every iteration an anchor
      int base = 0;
      for (; base + STEP <= cnt; base += STEP) {
        KBuf A;
        load_iter(base, A, std::true_type{});
        compute_iter(base, A, std::false_type{}, std::true_type{});
      }
      if (base < cnt) {
        KBuf A;
        load_iter(base, A, std::true_type{});
        compute_iter(base, A, std::true_type{}, std::true_type{});
      }
    }
  }

  // ---- V pass set-up.  bf16 values go through the matrix cores, float32 values through
  // the vector ALUs; either way the first rows are requested before the softmax barriers
  // (their latency overlaps them).
  // float32: UV rows per lane group per iteration, in registers
  constexpr int UV = G <= 6 ? 4 : 2;
  constexpr int VSTEP = KPI * UV;
  Words<4> vlo[UV], vhi[UV];
  auto load_v = [&](int base) {
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const uint32_t off = (uint32_t)min(base + u * KPI + wave * KPW + kg, cnt - 1) * ROW;  // unconditional loads
      vlo[u] = load_words<4>(vw + (off + lo_off));
      vhi[u] = load_words<4>(vw + (off + hi_off));
    }
  };
  // bf16: o^T = V^T P^T as 16 x 16 x 32 MFMAs (v_mfma_f32_16x16x32_bf16) over tiles of 32 keys.
  // A wave owns 64 dims (one 128-byte line of every row) of the tiles of its key group: the
  // D / 64 dim groups times 256 / D key groups make the 4 waves, key group k taking the
  // range's tiles k, k + KGN, ...  A tile's rows come into registers PFT tiles ahead, are
  // written to the wave's LDS staging area and read back transposed (ds_read_b64_tr_b16:
  // lane n of each 16-lane group gets column n of a 4 x 16 block), so each lane holds 8 keys
  // of one dim, the MFMA's B operand.  The A operand holds the weights of the 32 keys split
  // into two bf16 terms, hi = the weight with its low 16 bits cleared and lo =
  // bf16(weight - hi) (relative error < 2^-15): rows j < G of the 16 x 32 operand are
  // query head j's hi terms, rows G + j its lo terms, the rest zero, so one MFMA per 16
  // dims and 32 keys accumulates both; they are added together, and the key groups, at the end.
  constexpr int NDG = D / 64;          // dim groups
  constexpr int KGN = 4 / NDG;         // key groups
  constexpr int KSTR = KGN * 32;       // keys between a key group's consecutive tiles
  constexpr int IPT = 4;               // load instructions per tile (8 keys x 128 bytes each)
  constexpr int NT = 4;                // 16-dim column tiles per wave
  constexpr int PFT = 3;               // tiles in flight (2, 4, 6 and 8 measured slower)
  constexpr int SROW = 128;            // bytes of a staged row
  static_assert(!MV || 2 * G <= 16, "hi and lo weight rows of G query heads fill at most 16 rows");
  // staged piece c of key k sits at piece c ^ swz(k) of its row: the transposed reads of
  // 4 keys x 4 pieces per 16 lanes then cover all banks
  auto swz = [](int key) { return 2 * (key & 3); };
  static_assert(4 * 32 * SROW == kStageBytes, "staging area");
  char* stg = vstage + wave * (32 * SROW);
  const int vdg = wave % NDG, vkg = wave / NDG;  // the wave's dim group and key group
  const int lr = lane / 8, lc = lane % 8;        // load instruction: key, piece
  const uint32_t gl_off = (uint32_t)(vdg * SROW + lc * 16);
  Words<4> vb[MV ? PFT : 1][IPT];
  auto load_tile = [&](int kb, Words<4> (&r)[IPT]) {
#pragma unroll
    for (int i = 0; i < IPT; ++i)  // unconditional loads (keys past the range: the last row)
      r[i] = load_words<4>(vw + ((uint32_t)min(kb + i * 8 + lr, cnt - 1) * ROW + gl_off));
  };
  if constexpr (MV) {
#pragma unroll
    for (int t = 0; t < PFT; ++t) load_tile(vkg * 32 + t * KSTR, vb[t]);
  } else {
    load_v(0);
  }

  // ---- range maximum per query head: each value slot across the wave's key groups, the
  // slots of the writer lanes of key group 0 into LDS [4 waves][U * G], then across waves
  // and key steps
#pragma unroll
  for (int i = 0; i < NF; ++i) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) mxs[i] = fmaxf(mxs[i], __shfl_xor(mxs[i], off, 64));
  }
  if (writer && kg == 0) {
#pragma unroll
    for (int i = 0; i < NF; ++i) red[wave * NV + vbase + i] = mxs[i];
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int u = 0; u < U; ++u) m = fmaxf(m, red[w * NV + u * G + j]);
    M[j] = m;
  }
  if (threadIdx.x < G) Mh[threadIdx.x] = M[threadIdx.x];
  __syncthreads();  // red is reused below

  // ---- weights p = 2^(x - m) and their sums
  float ls[G];
#pragma unroll
  for (int j = 0; j < G; ++j) ls[j] = 0.f;
  for (int key = threadIdx.x; key < cnt; key += kDecodeThreads) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float e = exp2_weight(xs[j * XS + key] - M[j]);
      xs[j * XS + key] = e;
      ls[j] += e;
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float s = wave_sum(ls[j]);
    if (lane == 0) red[wave * G + j] = s;
  }
  __syncthreads();
  if (threadIdx.x < G)
    Lh[threadIdx.x] = red[threadIdx.x] + red[G + threadIdx.x] + red[2 * G + threadIdx.x] + red[3 * G + threadIdx.x];

  // ---- V pass, bf16: PFT tiles in flight; each tile is staged, its slot refilled with the
  // tile PFT ahead, then multiplied
  f32x4 acc[MV ? NT : 1];
  if constexpr (MV) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t st_off = (uint32_t)(lr * SROW + 16 * (lc ^ swz(lr)));  // (swz(8 i + lr) = swz(lr))
    // transposed reads: lane (g, e, q) = (lane / 16, lane / 4 % 4, lane % 4) addresses key
    // 8 g + e (+ 4 for the second read), dims 16 t + 4 q .. + 3 of column tile t
    const int tk = 8 * (lane >> 4) + ((lane >> 2) & 3), tq = lane & 3;
    uint32_t tr_off[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tr_off[t] = (uint32_t)(tk * SROW + 16 * ((2 * t + (tq >> 1)) ^ swz(tk)) + 8 * (tq & 1));
    // A operand: lane (g, m) = (lane / 16, lane % 16) holds row m for keys 8 g .. 8 g + 7
    const int am = lane & 15, ag = lane >> 4;
    const bool a_hi = am < G, a_lo = am >= G && am < 2 * G;
    const uint32_t m_hi = a_hi ? ~0u : 0u, m_lo = a_lo ? ~0u : 0u;  // masks: no branch per pair
    const float* wsrc = xs + (a_hi ? am : a_lo ? am - G : 0) * XS + 8 * ag;
    auto stage = [&](const Words<4> (&r)[IPT]) {
#pragma unroll
      for (int i = 0; i < IPT; ++i)
        *reinterpret_cast<u32x4*>(stg + st_off + i * 1024) = u32x4{r[i].w[0], r[i].w[1], r[i].w[2], r[i].w[3]};
    };
    auto multiply = [&](int kb, auto tail) {
      constexpr bool TAIL = decltype(tail)::value;  // keys may lie past the range
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(wsrc + kb);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(wsrc + kb + 4);
      float w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      if constexpr (TAIL) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = kb + 8 * ag + i < cnt ? w[i] : 0.f;
      }
      u32x4 a;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h0 = __float_as_uint(w[2 * k]) & 0xffff0000u, h1 = __float_as_uint(w[2 * k + 1]) & 0xffff0000u;
        const bf16x2 lo = {(__bf16)(w[2 * k] - __uint_as_float(h0)), (__bf16)(w[2 * k + 1] - __uint_as_float(h1))};
        a[k] = (((h0 >> 16) | h1) & m_hi) | (__builtin_bit_cast(uint32_t, lo) & m_lo);
      }
      const bf16x8 A = __builtin_bit_cast(bf16x8, a);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stg + tr_off[t]));
        const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stg + tr_off[t] + 4 * SROW));
        const bf16x8 B = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
      }
    };
    int kb = vkg * 32;
    for (; kb + (PFT - 1) * KSTR + 32 <= cnt; kb += PFT * KSTR) {  // PFT whole tiles
#pragma unroll
      for (int t = 0; t < PFT; ++t) {
        stage(vb[t]);
        load_tile(kb + (t + PFT) * KSTR, vb[t]);  // unconditional (past the range: clamped rows)
        multiply(kb + t * KSTR, std::false_type{});
      }
    }
#pragma unroll
    for (int t = 0; t < PFT; ++t) {  // the key group's last tiles, already in flight
      if (kb + t * KSTR < cnt) {
        stage(vb[t]);
        multiply(kb + t * KSTR, std::true_type{});
      }
    }
  }

  // ---- V pass, float32: UV rows per lane group per iteration; the next iteration's rows
  // are requested before this iteration's arithmetic (software pipelining)
  float o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
  auto v_iter = [&](int base, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    Words<4> clo[UV], chi[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      clo[u] = vlo[u];
      chi[u] = vhi[u];
    }
    load_v(base + VSTEP);  // unconditional (past the range: clamped rows)
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int key = base + u * KPI + wave * KPW + kg;
      if (!TAIL || key < cnt) {
        float lo[HALF], hi[HALF];
        E::cvt(clo[u], lo);
        E::cvt(chi[u], hi);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float w = xs[j * XS + key];
#pragma unroll
          for (int e = 0; e < HALF; ++e) {
            o[j][e] = fmaf(w, lo[e], o[j][e]);
            o[j][HALF + e] = fmaf(w, hi[e], o[j][HALF + e]);
          }
        }
      }
    }
  };
  if constexpr (!MV) {
    int base = 0;
    for (; base + VSTEP <= cnt; base += VSTEP) v_iter(base, std::false_type{});
    if (base < cnt) v_iter(base, std::true_type{});
  }
  if constexpr (LOGITS) {
    // the H2O epilogue's inputs: the range's weights 2^(x - m) per query head (m: the
    // range's maximum; a head with no live key in the range stores zeros), stored after the
    // V pass rather than key by key in the K pass: a wave's memory requests complete in
    // order, so device-coherent stores among the K loads would hold back every later load
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const bool live = Mh[j] > -INFINITY;
      float* dst = p.logits + ((size_t)b * p.Hq + g * G + j) * p.C + s_begin;
      for (int key = threadIdx.x; key < cnt; key += kDecodeThreads) store_dev(&dst[key], live ? xs[j * XS + key] : 0.f);
    }
  }
  __syncthreads();  // xs is reused as the output buffer below

  if constexpr (MV) {
    // lane (g, n) holds rows 4 g .. 4 g + 3 of column n of each tile: the hi rows first (key
    // group k into ored[k][G][D]), then the lo rows added to them, then the key groups summed
    const int ag = lane >> 4, n = lane & 15;
    float* mine = ored + vkg * G * D + vdg * 64 + n;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * ag + r < G) mine[(4 * ag + r) * D + 16 * t] = acc[t][r];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * ag + r >= G && 4 * ag + r < 2 * G) mine[(4 * ag + r - G) * D + 16 * t] += acc[t][r];
    __syncthreads();
    if constexpr (KGN > 1) {
      for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {  // each thread reads only its idx
        float x = ored[idx];
#pragma unroll
        for (int k = 1; k < KGN; ++k) x += ored[k * G * D + idx];
        ored[idx] = x;
      }
      __syncthreads();
    }
    split_finish<D, G, LOGITS, MASKED, true>(p, ored, Mh, Lh, split, n_splits, b, g);
    return;
  }

  // ---- merge the key groups of each wave, then the 4 waves
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
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads)  // each thread reads only its idx
    ored[idx] = ored[idx] + ored[G * D + idx] + ored[2 * G * D + idx] + ored[3 * G * D + idx];
  __syncthreads();
  split_finish<D, G, LOGITS, MASKED, true>(p, ored, Mh, Lh, split, n_splits, b, g);
}

// Victim choice for a seeded H2O layer (no decode step has run yet): the lowest score
// (token granule) or summed block score (blocks of bs slots) among candidates whose
// tokens have pos <= max_pos, ties evicting the newer token.
__global__ void __launch_bounds__(256) h2o_pick_victim_kernel(const float* score, const int* pos, int* victim, int C,
                                                              int n, int64_t max_pos, int bs) {
  __shared__ unsigned long long wkey[4];
  __shared__ int wat[4];
  const size_t bg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  Victim best;
  for (int base = threadIdx.x - lane; base < n; base += 256) {  // wave-uniform bound
    const int i = base + lane;
    const bool in = i < n;
    fold_victim(best, in ? score[bg * C + i] : 0.f, in ? pos[bg * C + i] : 0, i, in, max_pos, bs, lane);
  }
  const Victim v = reduce_victim(best, wkey, wat);
  if (threadIdx.x == 0 && v.key != ~0ull) victim[bg] = v.at;
}

hipError_t launch_h2o_pick_victim(const float* score, const int* pos, int* victim, int BHkv, int C, int n,
                                  int64_t max_pos, int bs, hipStream_t s) {
  hipLaunchKernelGGL(h2o_pick_victim_kernel, dim3(BHkv), dim3(256), 0, s, score, pos, victim, C, n, max_pos, bs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- dispatch
template <typename T, int D, int G>
static hipError_t launch_tdg(int mode, const DecodeParams& p, hipStream_t s) {
  const int items = p.duo ? p.ret_splits * p.B * p.Hret + p.str_splits * p.B * p.Hstr
                         : p.n_splits * p.B * p.Hkv;
  const dim3 grid(((items + 7) / 8) * 8), block(kDecodeThreads);
  if constexpr (G <= kOnepassMaxG) {
    const size_t lds = onepass_lds_bytes<D, G>();
    switch (mode) {
      case kModeRope: hipLaunchKernelGGL((decode_onepass_kernel<T, D, G, kModeRope>), grid, block, lds, s, p); break;
      case kModePlain: hipLaunchKernelGGL((decode_onepass_kernel<T, D, G, kModePlain>), grid, block, lds, s, p); break;
      case kModePlainLogits:
        hipLaunchKernelGGL((decode_onepass_kernel<T, D, G, kModePlainLogits>), grid, block, lds, s, p);
        break;
      case kModeMaskedLogits:
        hipLaunchKernelGGL((decode_onepass_kernel<T, D, G, kModeMaskedLogits>), grid, block, lds, s, p);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    // the block cache's slot positions of a range are staged in the kernel's 16 KiB area
    if (mode == kModeMaskedLogits && (size_t)p.chunk * sizeof(int) > 16384) return hipErrorInvalidValue;
    const size_t lds = twopass_lds_floats<D, G>(p.chunk) * sizeof(float);
    switch (mode) {
      case kModeRope: hipLaunchKernelGGL((decode_twopass_kernel<T, D, G, kModeRope>), grid, block, lds, s, p); break;
      case kModePlain: hipLaunchKernelGGL((decode_twopass_kernel<T, D, G, kModePlain>), grid, block, lds, s, p); break;
      case kModePlainLogits:
        hipLaunchKernelGGL((decode_twopass_kernel<T, D, G, kModePlainLogits>), grid, block, lds, s, p);
        break;
      case kModeMaskedLogits:
        hipLaunchKernelGGL((decode_twopass_kernel<T, D, G, kModeMaskedLogits>), grid, block, lds, s, p);
        break;
      default: return hipErrorInvalidValue;
    }
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

int decode_chunk_cap(int G) {
  if (G <= kOnepassMaxG) return 1 << 24;  // the one-pass kernel keeps no per-slot state in LDS
  // two-pass: (chunk + kXsPad) * G logits + the reduction and (max, sum) floats within 64 KiB,
  // 256 bytes kept for the small static shared variables (the bf16 V pass's 16 KiB staging
  // area brings a workgroup to at most 80 KiB, two per compute unit)
  return ((16384 - 64 - kTwopassRed - 2 * G) / G - kXsPad) / 64 * 64;
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
