// Internal declarations shared by the libbsg translation units (device code
// for gfx950 and the host-side launchers).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsg.h"

namespace bsg {

constexpr int kRowBlock = 64;   // rows per layout tile = lanes per wavefront
constexpr int kGroupWords = 4;  // words per layout tile (one 16-byte load per lane)
constexpr int kMaxK = 8;
constexpr int kMaxB = 64;
// Every workspace starts with this many bytes of arrival counters (one per
// 64-row block), zero-filled once by the caller and left zero by every
// completed call; partial sums and other scratch follow.  The fixed size
// keeps the counter area in the same place for every shape, so one
// workspace serves calls of any size.
constexpr size_t kCounterBytes = 65536;
constexpr int kMaxRowBlocksSplit = (int)(kCounterBytes / 4);

// Words of one base in the device layout: M*ND rounded up to 64 words.
__host__ __device__ inline size_t plane_words(int M, int ND) {
  size_t w = (size_t)M * (size_t)ND;
  return (w + 63) / 64 * 64;
}

// Device-layout word offset of logical word w of row m of base k (the formula
// documented in bsg.h).
__host__ __device__ inline size_t layout_offset(int M, int ND, size_t plane, int k, int m, int w) {
  size_t rb = (size_t)m >> 6, r = (size_t)m & 63;
  size_t h = (size_t)M - rb * 64;
  if (h > 64) h = 64;
  size_t g = (size_t)w >> 2, j = (size_t)w & 3;
  size_t wg = (size_t)ND - g * 4;
  if (wg > 4) wg = 4;
  return (size_t)k * plane + rb * 64 * (size_t)ND + g * 4 * h + r * wg + j;
}

// bf16 / fp16 bit patterns -> fp32 (exact).
__device__ inline float bf16_bits_to_float(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ inline float f16_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ inline float load_x(const void* x, int dt, size_t i) {
  if (dt == BSG_F32) return ((const float*)x)[i];
  if (dt == BSG_BF16) return bf16_bits_to_float(((const uint16_t*)x)[i]);
  return f16_bits_to_float(((const uint16_t*)x)[i]);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch plan of the sign products: 64-row blocks (one wavefront each) times
// S column splits of wb words; each split builds its own activation tables.
struct GemvPlan {
  int BB;    // batch columns per launch (1, 2, 4, 8 or 16)
  int S;     // column splits
  int wb;    // words per split (multiple of 4, except that the last split may be short)
  int nrb;   // 64-row blocks
  int nchunk;// launches over batch chunks of BB
  size_t part_bytes;  // partial sums (S > 1)
  size_t ws_bytes;    // kCounterBytes + part_bytes when S > 1, else 0
};

GemvPlan plan_gemv(int K, int M, int N, int B, bool int8_mode);

struct GemvArgs {
  const uint32_t* bits;
  const float* alpha;        // fp32 [K][M] or NULL
  const uint16_t* alpha_h;   // fp16 [K][M] or NULL (alpha == NULL && alpha_h == NULL -> 1)
  const uint16_t* colscale;  // fp16 [K][N] or NULL
  const void* x;             // [N][B]
  float* y;                  // [M][B]
  float* part;               // [S][M][BB] partials
  unsigned* cnt;             // [nrb] arrival counters
  size_t plane;
  int K, M, N, ND, B, b0, xdt, accumulate, S, wb;
};

struct GemvI8Args {
  const uint32_t* bits;
  const float* alpha;
  const int8_t* xq;          // [N][B]
  const float* sx;           // [B]
  int32_t* acc;              // [K][M][B] or NULL
  float* y;                  // [M][B] or NULL
  int32_t* part;             // [S][K][M][BB]
  unsigned* cnt;
  size_t plane;
  int K, M, N, ND, B, b0, accumulate, S, wb;
};

hipError_t launch_gemv_f(const GemvArgs& a, const GemvPlan& p, hipStream_t s);
hipError_t launch_gemv_i8(const GemvI8Args& a, const GemvPlan& p, hipStream_t s);

}  // namespace bsg
