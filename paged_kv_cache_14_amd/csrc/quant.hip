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
// decode's operand order (qpage.h).
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
  {  // parameters: keys per channel, values per token, in plain order
    float* ksc = reinterpret_cast<float*>(qp + kQKScale);
    float* kmn = reinterpret_cast<float*>(qp + kQKMin);
    float* vsc = reinterpret_cast<float*>(qp + kQVScale);
    float* vmn = reinterpret_cast<float*>(qp + kQVMin);
    ksc[tid] = k_sc[tid];
    kmn[tid] = k_mn[tid];
    vsc[tid] = v_sc[tid];
    vmn[tid] = v_mn[tid];
  }
  __syncthreads();
  if (tid < kQBoost) qp[kQBoostList + tid] = boost_list[tid];
  auto kcode = [&](int t, int c) {
    return code_of(to_f32<T>(k_lds[t * kD + c]), k_mn[c], k_sc[c], boosted[c] ? 15.f : 3.f);
  };
  auto vcode = [&](int t, int d) {
    return code_of(to_f32<T>(v_lds[t * kD + d]), v_mn[t], v_sc[t], 3.f);
  };
  // Word f = 256 s + 4 l + w of each code plane: step s, decode lane
  // l = 16q + j, word w (qpage.h).
  for (int f = tid; f < 4 * 64 * 4; f += blockDim.x) {
    const int st = f >> 8, l = (f >> 2) & 63, w = f & 3;
    const int q = l >> 4, j = l & 15;
    uint32_t kw = 0u, vw = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = i & 3;
      {  // keys: half H, channel block m
        const int H = w >> 1, m = 2 * (w & 1) + (i >> 2);
        const int t = 32 * st + 8 * (j >> 2) + 4 * H + (j & 3);
        const int c = 32 * m + 8 * q + 2 * p;
        kw |= ((kcode(t, c) & 3u) << (2 * i)) | ((kcode(t, c + 1) & 3u) << (16 + 2 * i));
      }
      {  // values: dim tile tt
        const int tt = 2 * w + (i >> 2);
        const int d = 16 * tt + j;
        const int t = 32 * st + 8 * q + 2 * p;
        vw |= (vcode(t, d) << (2 * i)) | (vcode(t + 1, d) << (16 + 2 * i));
      }
    }
    *reinterpret_cast<uint32_t*>(qp + kQKLo + 4 * f) = kw;
    *reinterpret_cast<uint32_t*>(qp + kQVLo + 4 * f) = vw;
  }
  // High bits of the promoted channels: word f = 32 s + l for lanes l < 32.
  for (int f = tid; f < 4 * 32; f += blockDim.x) {
    const int st = f >> 5, l = f & 31;
    const int q = l >> 4, j = l & 15;
    uint32_t hw = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int H = i >> 2, p = i & 3;
      const int t = 32 * st + 8 * (j >> 2) + 4 * H + (j & 3);
      const int slot = 8 * q + 2 * p;
      hw |= ((kcode(t, boost_list[slot]) >> 2) << (2 * i)) |
            ((kcode(t, boost_list[slot + 1]) >> 2) << (16 + 2 * i));
    }
    *reinterpret_cast<uint32_t*>(qp + kQKHi + 4 * f) = hw;
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
