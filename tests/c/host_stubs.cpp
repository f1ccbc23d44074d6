// Stand-ins for the HIP runtime and the kernel launchers, so that the host side of the
// C ABI (lcd_host.cpp) can be built with the host compiler alone, under AddressSanitizer
// and UndefinedBehaviorSanitizer.  No device exists: launchers record the call and
// succeed, copies do nothing, device pointers are never dereferenced.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lcd_internal.h"

long g_launches = 0;  // kernel launches requested by the host code

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}

namespace lcd {
hipError_t launch_decode_split(int, int, int, int, const DecodeParams& p, hipStream_t) {
  // the plan the host hands over must be consistent
  if (p.n_splits < 1 || p.chunk < 64 || p.chunk % 64 != 0 || !p.out || !p.q) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_append(const AppendParams& p, hipStream_t) {
  if (p.n_rows < 0 || p.row_bytes <= 0) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_h2o_pick_victim(const float*, const int*, int*, int BHkv, int C, int, int64_t, int, hipStream_t) {
  if (BHkv < 1 || C < 1) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rope_table(float*, float*, int C, int D, double, hipStream_t) {
  if (C < 1 || D < 2) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fill_i32(int*, int, int64_t n, hipStream_t) {
  if (n < 0) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fill_f32(float*, float, int64_t n, hipStream_t) {
  if (n < 0) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
bool decode_supported(int dtype, int D, int G) {
  return (dtype == 0 || dtype == 1) && (D == 64 || D == 128 || D == 256) &&
         (G == 1 || G == 2 || G == 4 || G == 6 || G == 8);
}
int decode_chunk_cap(int G) { return G <= 2 ? 1 << 24 : (16384 - 128 - 2 * G) / G / 64 * 64; }
size_t snapkv_ws_bytes(int B, int H, int N, int Lobs) {
  return (size_t)B * H * ((size_t)N * 8 + (size_t)Lobs * 512) + 4096;
}
hipError_t launch_snapkv(const SnapkvParams& p, hipStream_t) {
  if (p.B < 1 || p.H < 1 || p.N < 1 || !p.k || !p.idx_out) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
size_t h2o_prompt_ws_bytes(int B, int Hq, int Hkv, int N) { return (size_t)B * (2 * Hq + Hkv) * N * 4 + 512; }
hipError_t launch_h2o_prompt(const H2oPromptParams& p, void*, float*, hipStream_t) {
  if (p.B < 1 || p.N < 1 || !p.pos_out) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t scratch_device_address(void** out) {
  *out = reinterpret_cast<void*>(uintptr_t(1) << 40);  // aligned stand-in, never dereferenced
  return hipSuccess;
}
}  // namespace lcd
