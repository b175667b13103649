// Device-side helpers shared by the gfx950 kernels of libpa.
//
// Element types are fp16 and bf16; every product and sum is carried in fp32.
// Exponentials use the hardware base-2 exponential (v_exp_f32) on logits that
// were pre-multiplied by log2(e): exp(x) = 2^(x * log2 e).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max seed: finite, so 2^(seed - m) is 0 or 1

// Per-type operations on pairs of 16-bit values packed in one 32-bit word.
template <typename T> struct Pair;

template <> struct Pair<f16> {
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
  __device__ static inline float lo(uint32_t a) { return (float)__builtin_bit_cast(f16x2, a)[0]; }
  __device__ static inline float hi(uint32_t a) { return (float)__builtin_bit_cast(f16x2, a)[1]; }
  __device__ static inline uint32_t pack(float a, float b) {
    f16x2 v = {(f16)a, (f16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
};

template <> struct Pair<bf16> {
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
  __device__ static inline float lo(uint32_t a) { return __uint_as_float(a << 16); }
  __device__ static inline float hi(uint32_t a) { return __uint_as_float(a & 0xffff0000u); }
  __device__ static inline uint32_t pack(float a, float b) {
    bf16x2 v = {(bf16)a, (bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Softmax weights for a matrix-core P.V product, whose operands are 16-bit.
// Each fp32 weight p becomes hi = p rounded to the input type plus lo = the
// rest (p - hi) rounded the same way, and the product is run on both, so the
// weights reach P.V with about 16 (bf16) or 22 (fp16) significant bits rather
// than 8 or 11.  Two weights per packed word, as the operands hold them:
// returns {hi, lo}.
template <typename T>
__device__ inline u32x2 split_weights(float p0, float p1) {
  const uint32_t hi = Pair<T>::pack(p0, p1);
  return u32x2{hi, Pair<T>::pack(p0 - Pair<T>::lo(hi), p1 - Pair<T>::hi(hi))};
}

// 32x32x16 matrix-core product, fp32 accumulate: D = A (32x16) * B (16x32) + C.
template <typename T> struct Mfma;
template <> struct Mfma<f16> {
  __device__ static inline f32x16 mm32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<bf16> {
  __device__ static inline f32x16 mm32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// 16x16x32 matrix-core product, fp32 accumulate: D = A (16x32) * B (32x16) + C.
// Lane l holds A row l%16 and B column l%16, k = 8*(l/16) .. +7, and D column
// l%16, rows 4*(l/16) .. +3 (checked on the GPU with an in-bounds probe).
template <typename T> struct Mfma16;
template <> struct Mfma16<f16> {
  __device__ static inline f32x4 mm(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16<bf16> {
  __device__ static inline f32x4 mm(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): in each 16-lane group,
// lane i receives element i%4 of the 8-byte reads of lanes i/4, i/4+4,
// i/4+8, i/4+12.  When lane j reads V[k0 + j/4][d0 + 4(j%4) .. +3], lane i
// gets V[k0 + e][d0 + i], e = 0..3 (checked on the GPU with an in-bounds probe).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ inline u32x2 ds_read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// DPP controls (gfx9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;   // lane i <-> 7-i within each 8-lane half-row
constexpr int kDppRowMirror = 0x140;       // lane i <-> 15-i within each 16-lane row

template <int kCtrl>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the sum.
__device__ inline float row16_sum(float v) {
  v += dpp<kDppQuadSwap1>(v);
  v += dpp<kDppQuadSwap2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Agent-scope relaxed atomic store / load of one float: coherent across the
// XCDs (their L2s are not coherent with each other for plain accesses).
__device__ inline void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Accesses `lane_bytes` past a wave-uniform address, through a buffer
// resource built in scalar registers: the per-lane address arithmetic is one
// 32-bit offset, and accesses past `range_bytes` read 0 / are dropped.  Word 3
// of a gfx9 buffer descriptor: 32-bit data format.  kAux is the cache policy;
// kSc1 makes the access coherent at agent scope (across the XCDs' separate
// L2s), as the relaxed agent-scope atomics above are.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kSc1 = 16;
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* uniform_base, int32_t range_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_base), (short)0, range_bytes,
                                           kBufferWord3);
}
template <int kAux = 0>
__device__ inline u32x4 load16_at(const void* uniform_base, uint32_t lane_bytes,
                                  int32_t range_bytes) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       buffer_rsrc(uniform_base, range_bytes), lane_bytes, 0, kAux));
}
template <int kAux = 0>
__device__ inline u32x2 load8_at(const void* uniform_base, uint32_t lane_bytes,
                                 int32_t range_bytes) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                       buffer_rsrc(uniform_base, range_bytes), lane_bytes, 0, kAux));
}
template <int kAux = 0>
__device__ inline void store16_at(void* uniform_base, uint32_t lane_bytes, int32_t range_bytes,
                                  u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, buffer_rsrc(uniform_base, range_bytes), lane_bytes, 0,
                                         kAux);
}
template <int kAux = 0>
__device__ inline void store8_at(void* uniform_base, uint32_t lane_bytes, int32_t range_bytes,
                                 u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, buffer_rsrc(uniform_base, range_bytes), lane_bytes, 0,
                                        kAux);
}

__device__ inline u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Nontemporal 16-byte load, for data read exactly once (K/V tiles in decode).
__device__ inline u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ inline void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// The prefill's ranking key of a sequence of n new rows (n * G query rows per
// KV head) and context C: its time in 64-key tile steps, weighted by what a
// step costs, or 0 for a sequence the decode kernel takes (at most
// kDecodeRows rows) or one without keys.  A run of at most 128 rows is one
// item of at most one 32-row wave per SIMD, whose steps stream at the tile
// loads' pace (weight 4); longer runs are items of 256 rows, where a SIMD
// holds two waves and a step costs about a third more (weight 5 per item;
// measured on the multi-turn prefill, 1-2% shorter than counting 128-row
// tiles, which priced such items at twice the short ones).  The prefill
// takes sequences by decreasing key, ties by index.
__device__ inline uint32_t prefill_work_key(int32_t C, int32_t n, int32_t G) {
  const int64_t rows = (int64_t)n * G;
  const int64_t kv_tiles = ((int64_t)C + 63) / 64;
  if (rows <= kDecodeRows || kv_tiles <= 0) return 0u;
  const int64_t items = (rows + kWideWgRows - 1) / kWideWgRows;
  const int64_t w = (rows <= kWgRows ? 4 : 5 * items) * kv_tiles;
  return (uint32_t)(w < (int64_t)UINT32_MAX ? w : (int64_t)UINT32_MAX);
}

}  // namespace pa
