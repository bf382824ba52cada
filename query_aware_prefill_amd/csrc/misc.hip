// Memory-bound kernels of the prefill path on gfx950: embedding gather,
// RMSNorm, last-row gather, the 8-column head with its argmax/boolean, and the
// E4M3 codec used by the fp8 KV store. All are one wave per row with 16-byte
// vector accesses; rows are independent.
#include "device_common.h"
#include "quail_internal.h"

namespace quail {

// h[r] = embed[tokens[tok_map ? tok_map[r] : r]], widened to the fp32
// residual stream. A token id outside [0, vocab) is counted in *bad (when
// given) and embeds row 0 instead, so a bad id never becomes an out-of-range
// read.
__global__ void __launch_bounds__(256) embed_kernel(const int32_t* tokens, const int32_t* tok_map,
                                                    const uint16_t* embed, float* h,
                                                    int32_t rows, int32_t H, int32_t vocab,
                                                    uint32_t* bad) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = tok_map ? tok_map[r] : r;
  int64_t tok = tokens[src];
  if (tok < 0 || tok >= vocab) {
    if (lane == 0 && bad) atomicAdd(bad, 1u);
    tok = 0;
  }
  const uint4* s = reinterpret_cast<const uint4*>(embed + tok * H);
  float4* d = reinterpret_cast<float4*>(h + (int64_t)r * H);
  for (int c = lane; c < H / 8; c += 64) {
    const uint4 v = s[c];
    d[2 * c] = make_float4(bf16_bits_to_f32(v.x & 0xFFFF), bf16_bits_to_f32(v.x >> 16),
                           bf16_bits_to_f32(v.y & 0xFFFF), bf16_bits_to_f32(v.y >> 16));
    d[2 * c + 1] = make_float4(bf16_bits_to_f32(v.z & 0xFFFF), bf16_bits_to_f32(v.z >> 16),
                               bf16_bits_to_f32(v.w & 0xFFFF), bf16_bits_to_f32(v.w >> 16));
  }
}

hipError_t launch_embed(const int32_t* tokens, const int32_t* tok_map, const uint16_t* embed,
                        float* h, int32_t rows, int32_t H, int32_t vocab, uint32_t* bad,
                        hipStream_t s) {
  if (rows == 0) return hipSuccess;
  embed_kernel<<<dim3((rows + 3) / 4), dim3(256), 0, s>>>(tokens, tok_map, embed, h, rows, H, vocab, bad);
  return hipGetLastError();
}

// Guard regions of the KV pool: 256 bytes after every slab (and at the
// pool's end) hold a fixed pattern. mode 1 writes the pattern into regions
// base + offs[i]; mode 0 checks it and counts every region that differs in
// *bad. One wave per region, 4 bytes per lane.
constexpr uint32_t kGuardWord = 0xA5C3965Au;

__global__ void __launch_bounds__(256) guard_kernel(uint8_t* base, const int64_t* offs, int32_t n,
                                                    int32_t mode, uint32_t* bad) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  uint32_t* g = reinterpret_cast<uint32_t*>(base + offs[i]) + lane;
  if (mode == 1) {
    *g = kGuardWord ^ (uint32_t)lane;
  } else {
    const bool ok = *g == (kGuardWord ^ (uint32_t)lane);
    if (__ballot(!ok) != 0 && lane == 0) atomicAdd(bad, 1u);
  }
}

hipError_t launch_guard(uint8_t* base, const int64_t* offs, int32_t n, int32_t mode, uint32_t* bad,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  guard_kernel<<<dim3((n + 3) / 4), dim3(256), 0, s>>>(base, offs, n, mode, bad);
  return hipGetLastError();
}

// n 32-bit words = 0 (a kernel rather than a memset node, so that it also
// behaves under graph capture)
__global__ void __launch_bounds__(64) zero_words_kernel(uint32_t* p, int32_t n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_words_kernel<<<dim3(1), dim3(64), 0, s>>>(p, n);
  return hipGetLastError();
}

// fp32 residual rows -> bf16 rows (round to nearest even)
__global__ void __launch_bounds__(256) copy_rows_kernel(const float* src, int64_t lds,
                                                        const int32_t* src_idx, uint16_t* dst,
                                                        int64_t ldd, const int32_t* dst_idx,
                                                        int32_t rows, int32_t H) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int64_t sr = src_idx ? src_idx[r] : r;
  const int64_t dr = dst_idx ? dst_idx[r] : r;
  const float4* s = reinterpret_cast<const float4*>(src + sr * lds);
  uint4* d = reinterpret_cast<uint4*>(dst + dr * ldd);
  for (int c = lane; c < H / 8; c += 64) {
    const float4 a = s[2 * c], b = s[2 * c + 1];
    d[c] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                      pack_bf16x2(b.z, b.w));
  }
}

hipError_t launch_copy_rows(const float* src, int64_t lds, const int32_t* src_idx,
                            uint16_t* dst, int64_t ldd, const int32_t* dst_idx, int32_t rows,
                            int32_t H, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  copy_rows_kernel<<<dim3((rows + 3) / 4), dim3(256), 0, s>>>(src, lds, src_idx, dst, ldd,
                                                              dst_idx, rows, H);
  return hipGetLastError();
}

// The first `rows` rows of every (layer, K|V, kv head) block of one slab into
// the same rows of another slab whose blocks are longer: each block is
// [padded length][head_dim], so those rows are one contiguous run of
// rows x row_chunks 16-byte chunks at the start of the block.
__global__ void __launch_bounds__(256) copy_slab_rows_kernel(const uint8_t* src, int64_t src_block,
                                                             uint8_t* dst, int64_t dst_block,
                                                             int64_t per_block, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t b = i / per_block, c = i - b * per_block;
  reinterpret_cast<uint4*>(dst + b * dst_block)[c] = reinterpret_cast<const uint4*>(src + b * src_block)[c];
}

hipError_t launch_copy_slab_rows(const uint8_t* src, int64_t src_block, uint8_t* dst, int64_t dst_block,
                                 int32_t rows, int32_t row_bytes, int32_t n_blocks, hipStream_t s) {
  if (rows <= 0 || n_blocks <= 0) return hipSuccess;
  if (row_bytes % 16 != 0 || (int64_t)rows * row_bytes > src_block || (int64_t)rows * row_bytes > dst_block)
    return hipErrorInvalidValue;
  const int64_t per_block = (int64_t)rows * (row_bytes / 16);
  const int64_t total = per_block * n_blocks;
  copy_slab_rows_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(src, src_block, dst, dst_block,
                                                                                     per_block, total);
  return hipGetLastError();
}

// Per-token E4M3 quantisation of bf16 rows (the W8A8 projections' inputs):
// amax = the row's largest magnitude, code = E4M3(x * (448 / amax)) with the
// division and the product single fp32 operations, scale = amax / 448; a row
// of zeros gets codes 0 and scale 0. Helpers shared by the quantiser and the
// RMSNorm that emits codes directly.
__device__ __forceinline__ float absmax_bf16x8(const uint4& v, float m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    m = fmaxf(m, fmaxf(__uint_as_float((w[e] & 0x7FFFu) << 16), __uint_as_float(w[e] & 0x7FFF0000u)));
  return m;
}

// 8 bf16 -> 8 E4M3 codes of x * inv (byte i = element i); inv == 0 (a row of
// zeros) gives codes 0, also for -0 elements
__device__ __forceinline__ uint2 quant_bf16x8(const uint4& v, float inv) {
  if (inv == 0.0f) return make_uint2(0, 0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c[e] = f32_to_e4m3(__uint_as_float(w[e] << 16) * inv) |
           (f32_to_e4m3(__uint_as_float(w[e] & 0xFFFF0000u) * inv) << 8);
  return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

__device__ __forceinline__ float quant_inv(float amax) { return amax > 0.0f ? 448.0f / amax : 0.0f; }
__device__ __forceinline__ float quant_scale(float amax) { return amax > 0.0f ? amax / 448.0f : 0.0f; }

// One wave per row of K bf16 values; rows of up to 64 * 8 * CH values stay
// in registers between the max pass and the encode pass (longer rows are read
// twice, the second read from the cache).
template <int CH>
__global__ void __launch_bounds__(256)
act_quant_e4m3_kernel(int32_t M, int32_t K, const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                      float* __restrict__ scale) {
  constexpr int kQuantChunks = CH;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * K);
  uint2* cr = reinterpret_cast<uint2*>(codes + (int64_t)row * K);
  const int n8 = K / 8;
  if (n8 <= 64 * kQuantChunks) {
    uint4 v[kQuantChunks];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < kQuantChunks; ++c) {
      const int i = c * 64 + lane;
      v[c] = i < n8 ? xr[i] : make_uint4(0, 0, 0, 0);
      m = absmax_bf16x8(v[c], m);
    }
    const float amax = wave_max(m);
    const float inv = quant_inv(amax);
#pragma unroll
    for (int c = 0; c < kQuantChunks; ++c) {
      const int i = c * 64 + lane;
      if (i < n8) cr[i] = quant_bf16x8(v[c], inv);
    }
    if (lane == 0) scale[row] = quant_scale(amax);
    return;
  }
  float m = 0.0f;
  for (int i = lane; i < n8; i += 64) m = absmax_bf16x8(xr[i], m);
  const float amax = wave_max(m);
  const float inv = quant_inv(amax);
  for (int i = lane; i < n8; i += 64) cr[i] = quant_bf16x8(xr[i], inv);
  if (lane == 0) scale[row] = quant_scale(amax);
}

// Long rows (up to 256 * 8 * CH values, e.g. the 9728-wide MLP product):
// one workgroup of 4 waves per row, each thread holding CH 8-value chunks, the
// row maximum combined across the waves through LDS (a maximum is exact, so
// the result is the same as the one-wave kernel's).
template <int CH>
__global__ void __launch_bounds__(256)
act_quant_e4m3_row_kernel(int32_t K, const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                          float* __restrict__ scale) {
  __shared__ float wmax[4];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * K);
  uint2* cr = reinterpret_cast<uint2*>(codes + (int64_t)row * K);
  const int n8 = K / 8;
  uint4 v[CH];
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = c * 256 + t;
    v[c] = i < n8 ? xr[i] : make_uint4(0, 0, 0, 0);
    m = absmax_bf16x8(v[c], m);
  }
  m = wave_max(m);
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = quant_inv(amax);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = c * 256 + t;
    if (i < n8) cr[i] = quant_bf16x8(v[c], inv);
  }
  if (t == 0) scale[row] = quant_scale(amax);
}

hipError_t launch_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes, float* scale,
                                 hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (K > 64 * 8 * 8 && K <= 256 * 8 * 8)
    act_quant_e4m3_row_kernel<8><<<dim3((unsigned)M), dim3(256), 0, s>>>(K, x, codes, scale);
  else
    act_quant_e4m3_kernel<8><<<dim3((M + 3) / 4), dim3(256), 0, s>>>(M, K, x, codes, scale);
  return hipGetLastError();
}

// y = bf16(x / sqrt(mean(x^2) + eps) * gamma), x an fp32 residual row, one
// wave per row; 8 columns per lane and chunk (two 16-B loads, one 16-B
// store). Up to kNormChunks chunks per lane stay in registers: rows of up to
// 64 * 8 * 8 = 4096 columns are read once, with all their loads in flight
// together; longer rows are read a second time for the output pass.
// Q: instead of the bf16 row, its per-token E4M3 codes (yq, row stride H)
// and scale (ys), quantised from the bf16 values exactly as the standalone
// quantiser would (long rows recompute the bf16 values for each pass).
constexpr int kNormChunks = 8;

// bf16(x * inv * gamma) of one 8-column chunk
__device__ __forceinline__ uint4 norm_chunk(const float4& a, const float4& b, float inv, const uint4* gm, int c) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const uint4 gg = gm ? gm[c] : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf16x2(v[2 * i] * inv * bf16_bits_to_f32(gw[i] & 0xFFFF),
                       v[2 * i + 1] * inv * bf16_bits_to_f32(gw[i] >> 16));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <bool Q>
__device__ __forceinline__ void rmsnorm_row(const NormParams& p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= p.rows) return;
  const int src = p.row_map ? p.row_map[r] : r;
  const float4* x = reinterpret_cast<const float4*>(p.x + (int64_t)src * p.ldx);
  const int nc = p.H / 8;
  uint4* y = Q ? nullptr : reinterpret_cast<uint4*>(p.y + (int64_t)r * p.ldy);
  uint2* yq = Q ? reinterpret_cast<uint2*>(p.yq + (int64_t)r * p.H) : nullptr;
  const uint4* gm = reinterpret_cast<const uint4*>(p.gamma);
  // per lane, chunks lane, lane + 64, ... in order (the same summation order
  // in both branches)
  if (nc <= 64 * kNormChunks) {
    float4 a[kNormChunks], b[kNormChunks];
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) {
        a[i] = x[2 * c];
        b[i] = x[2 * c + 1];
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i)
      if (lane + 64 * i < nc)
        ss += a[i].x * a[i].x + a[i].y * a[i].y + a[i].z * a[i].z + a[i].w * a[i].w + b[i].x * b[i].x +
              b[i].y * b[i].y + b[i].z * b[i].z + b[i].w * b[i].w;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
    if (!Q) {
#pragma unroll
      for (int i = 0; i < kNormChunks; ++i) {
        const int c = lane + 64 * i;
        if (c < nc) y[c] = norm_chunk(a[i], b[i], inv, gm, c);
      }
      return;
    }
    uint4 yv[kNormChunks];
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = lane + 64 * i;
      yv[i] = c < nc ? norm_chunk(a[i], b[i], inv, gm, c) : make_uint4(0, 0, 0, 0);
      mx = absmax_bf16x8(yv[i], mx);
    }
    const float amax = wave_max(mx);
    const float qi = quant_inv(amax);
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) yq[c] = quant_bf16x8(yv[i], qi);
    }
    if (lane == 0) p.ys[r] = quant_scale(amax);
    return;
  }
  float ss = 0.0f;
  for (int c = lane; c < nc; c += 64) {
    const float4 a = x[2 * c], b = x[2 * c + 1];
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
  if (!Q) {
    for (int c = lane; c < nc; c += 64) y[c] = norm_chunk(x[2 * c], x[2 * c + 1], inv, gm, c);
    return;
  }
  float mx = 0.0f;
  for (int c = lane; c < nc; c += 64) mx = absmax_bf16x8(norm_chunk(x[2 * c], x[2 * c + 1], inv, gm, c), mx);
  const float amax = wave_max(mx);
  const float qi = quant_inv(amax);
  for (int c = lane; c < nc; c += 64) yq[c] = quant_bf16x8(norm_chunk(x[2 * c], x[2 * c + 1], inv, gm, c), qi);
  if (lane == 0) p.ys[r] = quant_scale(amax);
}

__global__ void __launch_bounds__(256) rmsnorm_kernel(NormParams p) { rmsnorm_row<false>(p); }
__global__ void __launch_bounds__(256) rmsnorm_quant_kernel(NormParams p) { rmsnorm_row<true>(p); }

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  if (p.yq) rmsnorm_quant_kernel<<<dim3((p.rows + 3) / 4), dim3(256), 0, s>>>(p);
  else rmsnorm_kernel<<<dim3((p.rows + 3) / 4), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

// Argmax (first maximum), boolean and store for one row's 8 logits (lane 0).
__device__ __forceinline__ void head8_finish(const float (&lg)[8], uint32_t true_mask, int out,
                                             float* logits, uint8_t* token, uint8_t* decision) {
  int best = 0;
#pragma unroll
  for (int j = 1; j < 8; ++j)
    if (lg[j] > lg[best]) best = j;
  if (logits) {
    float4* lp = reinterpret_cast<float4*>(logits + (int64_t)out * 8);
    lp[0] = make_float4(lg[0], lg[1], lg[2], lg[3]);
    lp[1] = make_float4(lg[4], lg[5], lg[6], lg[7]);
  }
  if (token) token[out] = (uint8_t)best;
  decision[out] = (uint8_t)((true_mask >> best) & 1u);
}

// z = bf16(RMSNorm(h_row; gamma)); logits = z . w8 (fp32); argmax; boolean.
__global__ void __launch_bounds__(256) head8_kernel(Head8Params p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= p.rows) return;
  const int src = p.row_map ? p.row_map[r] : r;
  const uint16_t* x = p.h + (int64_t)src * p.ldh;
  float inv = 1.0f;
  if (p.gamma) {
    float ss = 0.0f;
    for (int i = lane; i < p.H; i += 64) {
      const float a = bf16_bits_to_f32(x[i]);
      ss += a * a;
    }
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
  }
  float lg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = lane; i < p.H; i += 64) {
    float z = bf16_bits_to_f32(x[i]);
    if (p.gamma) z = bf16_bits_to_f32(f32_to_bf16_bits(z * inv * bf16_bits_to_f32(p.gamma[i])));
    const uint4 w = *reinterpret_cast<const uint4*>(p.w8 + (int64_t)i * 8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lg[2 * j] += z * bf16_bits_to_f32(ww[j] & 0xFFFF);
      lg[2 * j + 1] += z * bf16_bits_to_f32(ww[j] >> 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = wave_sum(lg[j]);
  if (lane == 0)
    head8_finish(lg, p.true_mask, p.out_map ? p.out_map[r] : r, p.logits, p.token, p.decision);
}

hipError_t launch_head8(const Head8Params& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  head8_kernel<<<dim3((p.rows + 3) / 4), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) head8_f32_kernel(int32_t n, int32_t H, const float* x,
                                                        const float* w8, uint32_t true_mask,
                                                        float* logits, uint8_t* token,
                                                        uint8_t* decision) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  float lg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = lane; i < H; i += 64) {
    const float z = x[(int64_t)r * H + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) lg[j] += z * w8[(int64_t)i * 8 + j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = wave_sum(lg[j]);
  if (lane == 0) head8_finish(lg, true_mask, r, logits, token, decision);
}

hipError_t launch_head8_f32(int32_t n, int32_t H, const float* x, const float* w8,
                            uint32_t true_mask, float* logits, uint8_t* token,
                            uint8_t* decision, hipStream_t s) {
  if (n == 0) return hipSuccess;
  head8_f32_kernel<<<dim3((n + 3) / 4), dim3(256), 0, s>>>(n, H, x, w8, true_mask, logits, token,
                                                          decision);
  return hipGetLastError();
}

__global__ void fp8_encode_kernel(int64_t n, const float* x, float inv_scale, uint8_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)f32_to_e4m3(x[i] * inv_scale);
}

__global__ void fp8_decode_kernel(int64_t n, const uint8_t* codes, float scale, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = fp8x2_to_f32<false>((uint32_t)codes[i])[0] * scale;
}

hipError_t launch_fp8_encode(int64_t n, const float* x, float inv_scale, uint8_t* out,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  fp8_encode_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(n, x, inv_scale, out);
  return hipGetLastError();
}

hipError_t launch_fp8_decode(int64_t n, const uint8_t* codes, float scale, float* out,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  fp8_decode_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(n, codes, scale, out);
  return hipGetLastError();
}

}  // namespace quail
