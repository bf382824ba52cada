// W8A8 projection on gfx950: E4M3 activations with one scale per token times
// E4M3 weights with one bf16 scale per output row, on the fp8 MFMA.
//
// The pages run the projections as FP8 GEMMs ([pt] "Como funciona": the
// engine's FP8 GEMM kernels; [fa] key points: qwen3-4b-fp8). With the
// activations quantised too, both operands of the product are E4M3 codes and
// the product runs on v_mfma_scale_f32_32x32x64_f8f6f4 (twice the bf16 rate):
//   codes[m][k] = E4M3(x[m][k] * (448 / amax_m)),  s_x[m] = amax_m / 448
//   y[m][n]     = bf16( s_w[n] * s_x[m] * sum_k decode(cx[m][k]) * decode(cw[n][k]) )
// amax_m is the largest magnitude of token m's row; a row of zeros has scale
// 0 and codes 0. The division and the product that decide each code are
// single fp32 operations (IEEE, round to nearest even).
//
// Tiling (gemm_w8a8_kernel): 256 tokens x 256 output columns per workgroup,
// 8 waves of 64 tokens x 128 columns, k-steps of KS bytes staged in LDS by
// global_load_lds (no register round trip). The MFMA computes the transposed
// product D = W_tile . X_tile^T, so a lane owns one token row and, in each
// 32-column block, 16 output columns; the epilogue stages each 32-token block
// through LDS so that global stores move whole 16-byte pieces of rows.
// Workgroups follow the grouped, XCD-contiguous order of the W8A16 kernel.
#include "device_common.h"
#include "w8a8.h"

namespace quail {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Per-token activation quantisation: one wave per row of K bf16 values.
// Rows up to 64 * 8 * kQuantChunks values stay in registers between the
// max pass and the encode pass; longer rows are read twice (the second read
// hits the cache).
// ---------------------------------------------------------------------------
constexpr int kQuantChunks = 8;

__device__ __forceinline__ float absmax_bf16x8(const uint4& v, float m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    m = fmaxf(m, fmaxf(__uint_as_float((w[e] & 0x7FFFu) << 16), __uint_as_float(w[e] & 0x7FFF0000u)));
  return m;
}

// 8 bf16 -> 8 E4M3 codes of x * inv (byte i = element i)
__device__ __forceinline__ uint2 quant_bf16x8(const uint4& v, float inv) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c[e] = f32_to_e4m3(__uint_as_float(w[e] << 16) * inv) |
           (f32_to_e4m3(__uint_as_float(w[e] & 0xFFFF0000u) * inv) << 8);
  return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

__global__ void __launch_bounds__(256)
act_quant_e4m3_kernel(int32_t M, int32_t K, const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                      float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * K);
  uint2* cr = reinterpret_cast<uint2*>(codes + (int64_t)row * K);
  const int n8 = K / 8;
  const bool in_regs = n8 <= 64 * kQuantChunks;
  uint4 v[kQuantChunks];
  float m = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kQuantChunks; ++c) {
      const int i = c * 64 + lane;
      v[c] = i < n8 ? xr[i] : make_uint4(0, 0, 0, 0);
      m = absmax_bf16x8(v[c], m);
    }
  } else {
    for (int i = lane; i < n8; i += 64) m = absmax_bf16x8(xr[i], m);
  }
  const float amax = wave_max(m);
  if (!(amax > 0.0f)) {
    // a row of zeros: codes 0 (also for -0 elements), scale 0
    for (int i = lane; i < n8; i += 64) cr[i] = make_uint2(0, 0);
    if (lane == 0) scale[row] = 0.0f;
    return;
  }
  const float inv = 448.0f / amax;
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kQuantChunks; ++c) {
      const int i = c * 64 + lane;
      if (i < n8) cr[i] = quant_bf16x8(v[c], inv);
    }
  } else {
    for (int i = lane; i < n8; i += 64) cr[i] = quant_bf16x8(xr[i], inv);
  }
  if (lane == 0) scale[row] = amax / 448.0f;
}

hipError_t launch_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes, float* scale,
                                 hipStream_t s) {
  if (M <= 0) return hipSuccess;
  act_quant_e4m3_kernel<<<dim3((M + 3) / 4), dim3(256), 0, s>>>(M, K, x, codes, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The GEMM.
//
// Operand layout of the 32x32x64 fp8 MFMA: a lane holds 32 codes (8 dwords)
// of row lane % 32 of its operand, lanes 0-31 one half of the 64 k values and
// lanes 32-63 the other. The sum over k does not depend on how a lane's k
// values are ordered as long as both operands order them alike: here lane
// half h of MFMA sub-step j holds the bytes [64 j + 32 h, 64 j + 32 h + 32) of
// the staged k-step, for weights and activations both. The scale operands
// are 127 (E8M0 2^0): a plain product; format selectors 0: E4M3 for both.
//
// LDS rows are KS bytes (16-byte chunks, XOR-swizzled by row so that the 16
// rows one read cycle of a 16-byte LDS read touches hit 16 distinct bank
// groups: KS = 128: chunk ^= (row / 2) % 8; KS = 64: chunk ^= (row / 4) % 4).
// Each k-step is one stage; the copies of the next STAGES - 1 steps are in
// flight while a step computes; every step starts with an explicit wait for
// its own copies and a raw s_barrier (a fenced __syncthreads would wait for
// every copy in flight).
// ---------------------------------------------------------------------------
constexpr int kW8GroupM = 4;   // token tiles per workgroup group

template <int KS>
__device__ __forceinline__ int swz8(int row, int chunk) {
  return KS == 128 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

__device__ __forceinline__ f32x16_t mfma_f8_32x32x64(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// two 16-byte LDS chunks -> the 8 dwords of one MFMA operand
__device__ __forceinline__ i32x8_t lds_operand(const uint8_t* row_base, int c0, int c1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row_base + c0 * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(row_base + c1 * 16);
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int KS, int STAGES>
__global__ void __launch_bounds__(512)
gemm_w8a8_kernel(W8A8Params p) {
  constexpr int BM = 256, BN = 256, WM = 4, NW = 8;
  constexpr int MB = 2;                                  // 32-token blocks per wave
  constexpr int TILE = BM * KS;                          // bytes of one operand per stage
  constexpr int PW = TILE / 1024 / NW;                   // 1-KB copies per wave per operand
  constexpr int CPW = 2 * PW;
  constexpr int RPC = 1024 / KS;                         // rows per 1-KB copy
  constexpr int LPR = KS / 16;                           // lanes per row in a copy
  static_assert(STAGES * 2 * TILE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES][2 * TILE];

  const int n_tn = p.N / BN;
  const int n_tm = (p.M + BM - 1) / BM;
  const int64_t total = (int64_t)n_tn * n_tm;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  const int64_t per_group = (int64_t)kW8GroupM * n_tn;
  const int64_t grp = wid / per_group;
  const int64_t rem = wid % per_group;
  const int gm_rows = (int)min<int64_t>(kW8GroupM, n_tm - grp * kW8GroupM);
  const int tm = (int)(grp * kW8GroupM + rem % gm_rows);
  const int tn = (int)(rem / gm_rows);
  const int m0 = tm * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int wm = wave % WM;
  const int wn = wave / WM;

  // per-lane copy sources (rows past M read row M - 1; their results are
  // not stored)
  const uint8_t* a_src[PW];
  const uint8_t* b_src[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int row = (wave * PW + i) * RPC + lane / LPR;
    const int m = min(m0 + row, p.M - 1);
    a_src[i] = p.A + (int64_t)m * p.K + swz8<KS>(row, lane % LPR) * 16;
    b_src[i] = p.B + (int64_t)(tn * BN + row) * p.K + swz8<KS>(row, lane % LPR) * 16;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem[kt % STAGES];
#pragma unroll
    for (int i = 0; i < PW; ++i) copy16_to_lds(a_src[i] + kt * KS, st + (wave * PW + i) * 1024);
#pragma unroll
    for (int i = 0; i < PW; ++i) copy16_to_lds(b_src[i] + kt * KS, st + TILE + (wave * PW + i) * 1024);
  };

  f32x16_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  const int nk = p.K / KS;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // steps issued beyond kt: min(STAGES - 2, nk - 1 - kt); their copies may stay in flight
    const int ahead = min(STAGES - 2, nk - 1 - kt);
    if (STAGES >= 4 && ahead >= 2) wait_vmcnt<(STAGES >= 4 ? 2 : 0) * CPW>();
    else if (STAGES >= 3 && ahead >= 1) wait_vmcnt<(STAGES >= 3 ? 1 : 0) * CPW>();
    else wait_vmcnt<0>();
    raw_barrier();                  // step kt landed everywhere; stage (kt - 1) % STAGES is free
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const uint8_t* st = smem[kt % STAGES];
#pragma unroll
    for (int j = 0; j < KS / 64; ++j) {
      const int c0 = 4 * j + 2 * hi;
      i32x8_t af[MB], bw[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = wn * 128 + nb * 32 + l32;
        bw[nb] = lds_operand(st + TILE + row * KS, swz8<KS>(row, c0), swz8<KS>(row, c0 + 1));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = wm * 64 + mb * 32 + l32;
        af[mb] = lds_operand(st + row * KS, swz8<KS>(row, c0), swz8<KS>(row, c0 + 1));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_f8_32x32x64(bw[nb], af[mb], acc[mb][nb]);
    }
  }

  // Epilogue: lane owns token m_row0 + mb*32 + l32 and, in column block nb,
  // columns nb*32 + rg*8 + hi*4 + e of the wave's 128. Each 32-token block is
  // written to the wave's 8-KB LDS region as bf16 rows of 256 B (16-byte
  // chunks XOR-swizzled by row & 15) and read back 16 lanes per row.
  __syncthreads();                  // every wave is done with the stages
  uint8_t* lds = &smem[0][0] + wave * 8192;
  const int m_row0 = m0 + wm * 64;
  const int n_base = tn * BN + wn * 128;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float sx = p.a_scale[min(m_row0 + mb * 32 + l32, p.M - 1)];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int i0 = nb * 32 + rg * 8 + hi * 4;
        const uint2 sw = *reinterpret_cast<const uint2*>(p.b_scale + n_base + i0);
        const float y0 = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sw.x & 0xFFFF) * sx;
        const float y1 = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sw.x >> 16) * sx;
        const float y2 = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sw.y & 0xFFFF) * sx;
        const float y3 = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sw.y >> 16) * sx;
        const int c = i0 >> 3;      // 16-byte chunk of 8 bf16; this lane writes half hi of it
        *reinterpret_cast<uint2*>(lds + l32 * 256 + ((c ^ (l32 & 15)) << 4) + hi * 8) =
            make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
      }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + (lane >> 4);
      const int c = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(lds + r * 256 + ((c ^ (r & 15)) << 4));
      const int mr = m_row0 + mb * 32 + r;
      if (mr < p.M) *reinterpret_cast<uint4*>(p.Y + (int64_t)mr * p.N + n_base + c * 8) = v;
    }
  }
}

hipError_t launch_gemm_w8a8(const W8A8Params& p, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  const int64_t total = (int64_t)(p.N / 256) * ((p.M + 255) / 256);
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  gemm_w8a8_kernel<128, 2><<<dim3((unsigned)grid), dim3(512), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace quail
