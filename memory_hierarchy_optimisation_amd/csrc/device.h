// device.h -- gfx950 device helpers shared by the kernels: vector types, the
// workgroup -> C-tile mapping, output conversion and the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace mhg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

#define MHG_LDS __attribute__((address_space(3)))

struct HalfF16 {};
struct HalfBF16 {};

// One 16x16x32 matrix multiply-accumulate on a wave: acc += A(16x32) * B(32x16).
// Lane l holds A row (l % 16), k = 8*(l/16) .. +7 and B column (l % 16) over the same
// k; the accumulator holds rows 4*(l/16) .. +3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16(HalfBF16, u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(HalfF16, u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS transpose read of four 16-bit elements.  Within each group of 16 lanes, lane t
// receives element (t & 3) of the 8-byte rows addressed by lanes 4q + (t >> 2),
// q = 0..3: a 4 x 16 block of a row-major tile comes back column by column.
__device__ __forceinline__ u32x2 lds_read_tr16(const char *lds_byte_ptr) {
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MHG_LDS bf16x4 *)(lds_byte_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// Workgroup id -> (tile row, tile column).  Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs, each with its own L2, so ids are first regrouped so
// that every XCD receives a contiguous run of logical tiles; logical tiles are then
// walked group_m rows of tiles at a time, so that the tiles in flight on one XCD
// share A row-panels and B column-panels ("Tiling 策略与内存层次优化", L2 cache: hit
// rate is raised only through the access pattern).
__device__ __forceinline__ void tile_of(int bid, int gm, int gn, int group_m, int &tm, int &tn) {
  const int nwg = gm * gn;
  const int q = nwg >> 3, r = nwg & 7;
  const int x = bid & 7, loc = bid >> 3;
  const int logical = x * q + min(x, r) + loc;
  const int per_group = group_m * gn;
  const int g = logical / per_group;
  const int first = g * group_m;
  const int gsz = min(gm - first, group_m);
  const int in = logical - g * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Store four consecutive elements C[idx .. idx+3] from fp32 values, converting to the
// output type (round to nearest even).  `vec`: the four are inside the matrix and the
// address is aligned for one 8-byte (16-bit types) or 16-byte (fp32) store; otherwise
// element `e` is stored only when e < n_in.  (Ordinary stores: streaming ones here
// measured slower, 1024^3 f16 9.0 -> 10.8 us.)
__device__ __forceinline__ void store_out4(void *C, int64_t idx, f32x4 v, int out_code, bool vec, int n_in) {
  if (out_code == E_F32) {
    float *c = reinterpret_cast<float *>(C) + idx;
    if (vec) {
      *reinterpret_cast<f32x4 *>(c) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < n_in) c[e] = v[e];
    }
    return;
  }
  uint16_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    h[e] = out_code == E_F16 ? __builtin_bit_cast(uint16_t, (_Float16)v[e])
                             : __builtin_bit_cast(uint16_t, (__bf16)v[e]);
  uint16_t *c = reinterpret_cast<uint16_t *>(C) + idx;
  if (vec) {
    *reinterpret_cast<u32x2 *>(c) = u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                          uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < n_in) c[e] = h[e];
  }
}

// fp32 -> output element, round to nearest even for the 16-bit types.
__device__ __forceinline__ void store_out(void *C, int64_t idx, float v, int out_code) {
  if (out_code == E_F32) {
    reinterpret_cast<float *>(C)[idx] = v;
  } else if (out_code == E_F16) {
    reinterpret_cast<_Float16 *>(C)[idx] = (_Float16)v;
  } else {
    reinterpret_cast<__bf16 *>(C)[idx] = (__bf16)v;
  }
}

// Output element -> fp32 (exact: every fp16 / bf16 value is an fp32 value).
__device__ __forceinline__ float load_out(const void *C, int64_t idx, int out_code) {
  if (out_code == E_F32) return reinterpret_cast<const float *>(C)[idx];
  if (out_code == E_F16) return float(reinterpret_cast<const _Float16 *>(C)[idx]);
  return float(reinterpret_cast<const __bf16 *>(C)[idx]);
}

// The fused epilogue on one accumulated element of C[row][col], in fp32, before the
// single rounding to the output type: element-wise work done on the tile's output on
// its way to HBM ("Tiling 策略与内存层次优化", fusion stage: bias and ReLU fused into
// the GEMM tile's output end).  beta == 0 reads nothing from C, so C's prior contents
// (even NaN) do not matter then.  ReLU maps everything that is not above zero (NaN
// included) to +0.
__device__ __forceinline__ float epilogue1(const LaunchArgs &p, float v, int64_t row, int64_t col) {
  float t = p.alpha * v;
  if (p.beta != 0.0f) t += p.beta * load_out(p.C, row * p.ldc + col, p.out_code);
  if (p.bias) t += p.bias[col];
  if (p.act == 1) t = t > 0.0f ? t : 0.0f;
  return t;
}

// Prior C[row][col .. col + 3] as fp32 (elements past N read as 0): one 16- or 8-byte
// load when all four lie inside the matrix and C allows vector access (col is a
// multiple of 4 at every call site), else element by element.
__device__ __forceinline__ f32x4 prior4(const LaunchArgs &p, int64_t row, int64_t col, int64_t n_in) {
  const int64_t idx = row * p.ldc + col;
  if (n_in >= 4 && p.c_vec) {
    if (p.out_code == E_F32) return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.C) + idx);
    const u32x2 h = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p.C) + idx);
    f32x4 c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t b = uint16_t(h[e >> 1] >> (16 * (e & 1)));
      c[e] = p.out_code == E_F16 ? float(__builtin_bit_cast(_Float16, b)) : float(__builtin_bit_cast(__bf16, b));
    }
    return c;
  }
  f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (e < n_in) c[e] = load_out(p.C, idx + e, p.out_code);
  return c;
}

// bias[col .. col + 3] (0 past N or without a bias).
__device__ __forceinline__ f32x4 bias4(const LaunchArgs &p, int64_t col, int64_t n_in) {
  f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
  if (p.bias) {
    if (n_in >= 4 && p.bias_vec) {
      b = *reinterpret_cast<const f32x4 *>(p.bias + col);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < n_in) b[e] = p.bias[col + e];
    }
  }
  return b;
}

// The epilogue on C[row][col .. col + 3] given its prior values (ignored when beta is
// 0) and its bias values; elements e >= n_in (past N) are left as they are.
__device__ __forceinline__ f32x4 epilogue4pb(const LaunchArgs &p, f32x4 v, f32x4 prior, f32x4 b, int64_t n_in) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (e >= n_in) break;
    float t = p.alpha * v[e];
    if (p.beta != 0.0f) t += p.beta * prior[e];
    t += b[e];
    if (p.act == 1) t = t > 0.0f ? t : 0.0f;
    v[e] = t;
  }
  return v;
}

// The same, reading the prior and bias values itself.
__device__ __forceinline__ f32x4 epilogue4(const LaunchArgs &p, f32x4 v, int64_t row, int64_t col, int64_t n_in) {
  const f32x4 prior = p.beta != 0.0f ? prior4(p, row, col, n_in) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  return epilogue4pb(p, v, prior, bias4(p, col, n_in), n_in);
}

}  // namespace mhg
