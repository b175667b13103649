// pa_quantize_pages: 128-token pages of K and V at 2 bits per value, the 16
// key channels of largest mean magnitude at 4 (KV-cache textbook ch.22, the
// Kitty passage: a quantization group of 128 tokens is one page, kept
// compatible with paged attention; promoted channels store their high 2 bits
// in a small sparse plane beside the dense plane of every channel's low 2
// bits).  Keys are quantized per channel along the page's tokens, values per
// token along its channels.  For a group of values x: mn = min x, scale =
// (max x - mn) / levels and code = min(levels, rint((x - mn) / scale)),
// every step in float32 with round-to-nearest-even (code 0 when scale is 0);
// the value a code stands for is mn + code * scale.
//
// One workgroup per (page, KV head).  The page's 8 source blocks are staged
// in LDS (K and V, 16-bit); thread c then takes key channel c and thread t
// value token t for the statistics, and the codes are written in the
// decode's lane order (qpage.h).
#include "pa_device.h"
#include "pa_launch.h"
#include "qpage.h"

namespace pa {

namespace {

template <typename T>
__device__ inline float to_f32(uint16_t bits);
template <>
__device__ inline float to_f32<f16>(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}
template <>
__device__ inline float to_f32<bf16>(uint16_t bits) {
  return __uint_as_float((uint32_t)bits << 16);
}

// Code of x in a group (mn, scale, levels), as the header defines it.
__device__ inline uint32_t code_of(float x, float mn, float scale, float levels) {
  if (scale == 0.f) return 0u;
  const float c = __builtin_rintf(__fdiv_rn(x - mn, scale));
  return (uint32_t)fminf(c, levels);
}

template <typename T>
__global__ __launch_bounds__(128) void quantize_pages_kernel(
    uint8_t* __restrict__ qpool, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ page_ids,
    const int32_t* __restrict__ src_blocks, int32_t num_pages, int32_t num_blocks,
    int32_t num_kv_heads) {
  constexpr int kT = kQPageTokens, kD = kHeadDim;
  __shared__ uint16_t k_lds[kT * kD];
  __shared__ uint16_t v_lds[kT * kD];
  __shared__ float k_mn[kD], k_sc[kD], v_mn[kT], v_sc[kT], k_sum[kD];
  __shared__ uint8_t boosted[kD];
  __shared__ uint8_t boost_list[kQBoost];
  const int tid = threadIdx.x;
  const int item = blockIdx.x, g = blockIdx.y;
  const int32_t page = page_ids[item];
  if ((uint32_t)page >= (uint32_t)num_pages) return;
  for (int b = 0; b < kQPageBlocks; ++b) {
    const int32_t blk = src_blocks[item * kQPageBlocks + b];
    if ((uint32_t)blk >= (uint32_t)num_blocks) return;  // uniform: nothing is written
  }
  // Stage the page: 8 blocks x 16 tokens x 128 dims of K and of V.
  for (int b = 0; b < kQPageBlocks; ++b) {
    const size_t base = ((size_t)src_blocks[item * kQPageBlocks + b] * num_kv_heads + g) *
                        kBlockSize * kD;
    const u32x4* ks = reinterpret_cast<const u32x4*>(k_pool + base);
    const u32x4* vs = reinterpret_cast<const u32x4*>(v_pool + base);
    u32x4* kd = reinterpret_cast<u32x4*>(k_lds + b * kBlockSize * kD);
    u32x4* vd = reinterpret_cast<u32x4*>(v_lds + b * kBlockSize * kD);
    for (int i = tid; i < kBlockSize * kD / 8; i += blockDim.x) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
  __syncthreads();
  // Statistics: key channel tid along the tokens (|k| summed in token
  // order), value token tid along the channels.
  {
    const int c = tid;
    float mn = to_f32<T>(k_lds[c]), mx = mn, sum = 0.f;
    for (int t = 0; t < kT; ++t) {
      const float x = to_f32<T>(k_lds[t * kD + c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
      sum += fabsf(x);
    }
    k_mn[c] = mn;
    k_sc[c] = mx;  // the span is finished below, once the channel's levels are known
    k_sum[c] = sum;
    const int t = tid;
    float vmn = to_f32<T>(v_lds[t * kD]), vmx = vmn;
    for (int dd = 0; dd < kD; ++dd) {
      // each thread starts at its own channel: the threads' rows are 256 B
      // apart, so reading the same channel at once would hit one bank
      const int d = (dd + t) & (kD - 1);
      const float x = to_f32<T>(v_lds[t * kD + d]);
      vmn = fminf(vmn, x);
      vmx = fmaxf(vmx, x);
    }
    v_mn[t] = vmn;
    v_sc[t] = __fdiv_rn(vmx - vmn, 3.f);
  }
  __syncthreads();
  // Promotion: channel c is among the 16 of largest sum (ties to the lower
  // index) when fewer than 16 channels rank above it.
  {
    const int c = tid;
    const float mine = k_sum[c];
    int above = 0;
    for (int o = 0; o < kD; ++o) {
      const float s = k_sum[o];
      above += (s > mine) | ((s == mine) & (o < c));
    }
    const bool b = above < kQBoost;
    boosted[c] = b;
    k_sc[c] = __fdiv_rn(k_sc[c] - k_mn[c], b ? 15.f : 3.f);
  }
  __syncthreads();
  uint8_t* qp = qpool + ((size_t)page * num_kv_heads + g) * kQPageBytes;
  if (tid < kD && boosted[tid]) {
    int pos = 0;
    for (int o = 0; o < tid; ++o) pos += boosted[o];
    boost_list[pos] = (uint8_t)tid;
  }
  {  // parameters
    float* ksc = reinterpret_cast<float*>(qp + kQKScale);
    float* kmn = reinterpret_cast<float*>(qp + kQKMin);
    ksc[tid] = k_sc[tid];
    kmn[tid] = k_mn[tid];
    // value parameters in the decode's order: block b, lane-row r, token i
    // of the block's 16 (token 4i + r) -> entry b*16 + r*4 + i
    const int t = tid, b = t >> 4, w = t & 15, r = w & 3, i = w >> 2;
    float* vsc = reinterpret_cast<float*>(qp + kQVScale);
    float* vmn = reinterpret_cast<float*>(qp + kQVMin);
    vsc[b * 16 + r * 4 + i] = v_sc[t];
    vmn[b * 16 + r * 4 + i] = v_mn[t];
  }
  __syncthreads();
  if (tid < kQBoost) qp[kQBoostList + tid] = boost_list[tid];
  // Codes.  Field (block b, channel group j, lane-row r): 4 tokens (4i + r,
  // i = 0..3) x 8 channels (8j + e) x 2 bits, token i in bits 16i..16i+15,
  // channel e at bits 2e; fields in the order (b, j, r), 8 bytes each.
  for (int f = tid; f < kQPageBlocks * 16 * 4; f += blockDim.x) {
    const int b = f >> 6, j = (f >> 2) & 15, r = f & 3;
    uint32_t kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = b * kBlockSize + 4 * i + r;
      uint32_t kf = 0u, vf = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * j + e;
        const uint32_t kc = code_of(to_f32<T>(k_lds[t * kD + c]), k_mn[c], k_sc[c],
                                    boosted[c] ? 15.f : 3.f);
        const uint32_t vc = code_of(to_f32<T>(v_lds[t * kD + c]), v_mn[t], v_sc[t], 3.f);
        kf |= (kc & 3u) << (2 * e);
        vf |= vc << (2 * e);
      }
      kw[i >> 1] |= kf << (16 * (i & 1));
      vw[i >> 1] |= vf << (16 * (i & 1));
    }
    *reinterpret_cast<u32x2*>(qp + kQKLo + f * 8) = u32x2{kw[0], kw[1]};
    *reinterpret_cast<u32x2*>(qp + kQVLo + f * 8) = u32x2{vw[0], vw[1]};
  }
  // High bits of the promoted channels.  Byte (slot j, lane-row r, block b):
  // token 4i + r of block b in bits 2i..2i+1; bytes in the order (j, r, b).
  for (int f = tid; f < kQBoost * 4 * kQPageBlocks; f += blockDim.x) {
    const int j = f >> 5, r = (f >> 3) & 3, b = f & 7;
    const int c = boost_list[j];
    uint32_t byte = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = b * kBlockSize + 4 * i + r;
      const uint32_t kc = code_of(to_f32<T>(k_lds[t * kD + c]), k_mn[c], k_sc[c], 15.f);
      byte |= (kc >> 2) << (2 * i);
    }
    qp[kQKHi + f] = (uint8_t)byte;
  }
}

}  // namespace

hipError_t launch_quantize_pages(bool is_bf16, void* qpool, const void* k_pool,
                                 const void* v_pool, const int32_t* page_ids,
                                 const int32_t* src_blocks, int32_t num_encode,
                                 int32_t num_pages, int32_t num_blocks, int32_t num_kv_heads,
                                 hipStream_t stream) {
  if (num_encode == 0) return hipSuccess;
  const dim3 grid((unsigned)num_encode, (unsigned)num_kv_heads);
  if (is_bf16)
    hipLaunchKernelGGL(quantize_pages_kernel<bf16>, grid, dim3(128), 0, stream,
                       static_cast<uint8_t*>(qpool), static_cast<const uint16_t*>(k_pool),
                       static_cast<const uint16_t*>(v_pool), page_ids, src_blocks, num_pages,
                       num_blocks, num_kv_heads);
  else
    hipLaunchKernelGGL(quantize_pages_kernel<f16>, grid, dim3(128), 0, stream,
                       static_cast<uint8_t*>(qpool), static_cast<const uint16_t*>(k_pool),
                       static_cast<const uint16_t*>(v_pool), page_ids, src_blocks, num_pages,
                       num_blocks, num_kv_heads);
  return hipGetLastError();
}

}  // namespace pa
