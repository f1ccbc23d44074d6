// KV-cache maintenance kernels: appending rows, the in-cache position table and
// state fills.
//
// Keys are written exactly as given (un-rotated for a RoPE cache: [SINK] "como
// funciona" keeps keys before rotation and rotates them at every decode step).
#include <hip/hip_runtime.h>

#include "lcd_internal.h"

namespace lcd {

// Copy rows of the [BHkv][n_new][D] input into cache slots, 16 bytes per thread.
__global__ void append_rows_kernel(AppendParams p) {
  const int chunks = p.row_bytes / 16;
  const int64_t total = (int64_t)p.BHkv * p.n_rows * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % chunks);
    const int64_t rr = i / chunks;
    const int r = p.r0 + (int)(rr % p.n_rows);
    const int bh = (int)(rr / p.n_rows);
    int slot;
    if (r < p.r_split) {
      slot = p.slot_lin + (r - p.r0);
    } else {
      slot = p.S + (int)(((int64_t)p.ring_off + (r - p.r_split)) % p.W);
    }
    const size_t src = ((size_t)bh * p.n_new + r) * p.row_bytes + (size_t)c * 16;
    const size_t dst = ((size_t)bh * p.C + slot) * p.row_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(p.k_cache + dst) = *reinterpret_cast<const uint4*>(p.k_in + src);
    *reinterpret_cast<uint4*>(p.v_cache + dst) = *reinterpret_cast<const uint4*>(p.v_in + src);
  }
}

// H2O append: one row per (batch row, KV head), written into the next free slot or,
// once the budget is full, into the victim slot chosen by the previous decode step.
__global__ void append_h2o_kernel(AppendParams p) {
  const int bh = blockIdx.x;
  int slot;
  if (p.fill < p.C) {
    slot = p.fill;
  } else if (p.bs <= 1) {
    slot = p.victim[bh];
  } else if (p.new_block) {  // block-level: the freed block becomes the open block
    const int blk = p.victim[bh];
    slot = blk * p.bs;
    for (int e = 1 + threadIdx.x; e < p.bs; e += blockDim.x) {
      p.pos[(size_t)bh * p.C + slot + e] = -1;  // emptied: not attended until refilled
      p.score[(size_t)bh * p.C + slot + e] = 0.f;
    }
    if (threadIdx.x == 0) p.open[bh] = blk;
  } else {
    slot = p.open[bh] * p.bs + p.offset;
  }
  const int chunks = p.row_bytes / 16;
  const size_t src = (size_t)bh * p.row_bytes;
  const size_t dst = ((size_t)bh * p.C + slot) * p.row_bytes;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    *reinterpret_cast<uint4*>(p.k_cache + dst + (size_t)c * 16) =
        *reinterpret_cast<const uint4*>(p.k_in + src + (size_t)c * 16);
    *reinterpret_cast<uint4*>(p.v_cache + dst + (size_t)c * 16) =
        *reinterpret_cast<const uint4*>(p.v_in + src + (size_t)c * 16);
  }
  if (threadIdx.x == 0) {
    p.pos[(size_t)bh * p.C + slot] = (int)p.token;
    p.score[(size_t)bh * p.C + slot] = 0.f;
  }
}

// Mixed retrieval / streaming heads ([KVC] "Decomposição funcional com o
// DuoAttention"): input row r of (b, g) is token a = t0 + r.  A retrieval head keeps
// every token in slot a; a streaming head keeps its sinks (a < S, slot a) and the
// tokens of the final window (a >= a_first, slot S + (a - S) mod W), exactly the rows
// a sink + window cache holds after these tokens, each written once.
__global__ void append_duo_kernel(AppendParams p) {
  const int chunks = p.row_bytes / 16;
  const int64_t total = (int64_t)p.BHkv * p.n_new * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % chunks);
    const int64_t rr = i / chunks;
    const int r = (int)(rr % p.n_new);
    const int bh = (int)(rr / p.n_new);
    const int b = bh / p.Hkv, g = bh % p.Hkv;
    const int64_t a = p.t0 + r;
    const int m = p.duo_map[g];
    char* kc;
    char* vc;
    size_t dst;
    if (m >= 0) {
      dst = (((size_t)b * p.Hret + m) * p.C + (size_t)a) * p.row_bytes;
      kc = p.k_cache;
      vc = p.v_cache;
    } else {
      if (a >= p.S && a < p.a_first) continue;  // evicted by a later row of this call
      const int64_t slot = a < p.S ? a : p.S + (a - p.S) % p.W;
      dst = (((size_t)b * p.Hstr + (-1 - m)) * p.C2 + (size_t)slot) * p.row_bytes;
      kc = p.k2_cache;
      vc = p.v2_cache;
    }
    const size_t src = ((size_t)bh * p.n_new + r) * p.row_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(kc + dst + (size_t)c * 16) = *reinterpret_cast<const uint4*>(p.k_in + src);
    *reinterpret_cast<uint4*>(vc + dst + (size_t)c * 16) = *reinterpret_cast<const uint4*>(p.v_in + src);
  }
}

// cos/sin of (position * base^(-2i/D)) for every in-cache position and pair,
// evaluated in float64 and rounded to float32.
__global__ void rope_table_kernel(float* cos_t, float* sin_t, int C, int D, double base) {
  const int D2 = D / 2;
  const int64_t total = (int64_t)C * D2;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx / D2), i = (int)(idx % D2);
    const double inv = pow(base, -2.0 * (double)i / (double)D);
    const double a = (double)r * inv;
    cos_t[idx] = (float)cos(a);
    sin_t[idx] = (float)sin(a);
  }
}

__global__ void fill_i32_kernel(int* p, int value, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

__global__ void fill_f32_kernel(float* p, float value, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

static int grid_for(int64_t work, int threads) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  if (p.h2o) {
    hipLaunchKernelGGL(append_h2o_kernel, dim3(p.BHkv), dim3(64), 0, s, p);
  } else if (p.duo) {
    const int64_t work = (int64_t)p.BHkv * p.n_new * (p.row_bytes / 16);
    hipLaunchKernelGGL(append_duo_kernel, dim3(grid_for(work, 256)), dim3(256), 0, s, p);
  } else {
    const int64_t work = (int64_t)p.BHkv * p.n_rows * (p.row_bytes / 16);
    hipLaunchKernelGGL(append_rows_kernel, dim3(grid_for(work, 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_table(float* cos_t, float* sin_t, int C, int D, double base, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for((int64_t)C * (D / 2), 256)), dim3(256), 0, s, cos_t,
                     sin_t, C, D, base);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int value, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float value, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

}  // namespace lcd
