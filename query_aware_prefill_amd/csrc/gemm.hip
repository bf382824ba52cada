// W8A16 GEMM for the decoder projections on gfx950.
//
// The model runs with FP8 weights and bf16 activations ([it] "Quail, il
// motore di inferenza ...", second paragraph: Qwen3 4B FP8; [fa] key points:
// qwen3-4b-fp8). Weights are OCP E4M3 codes [out][in] with one bf16 scale per
// output row. Every E4M3 value is a bf16 value, so the codes are decoded
// exactly into bf16 while they are staged in LDS and the product runs on the
// bf16 MFMA with fp32 accumulation; the row scale is applied in the epilogue:
//   y[m][n] = scale[n] * sum_k x[m][k] * decode(w[n][k]).
//
// Tiling (see gemm_direct_kernel): 256 tokens x 256 output columns x 64 k per
// workgroup step, each wave owning 64 tokens x 128 columns. The MFMA computes
// the transposed product
// D = W_tile . X_tile^T (v_mfma_f32_32x32x16_bf16), so each lane owns one
// token row and 16 output columns per 32-column block: a whole 128-column
// head lives in one wave, the RoPE pair (i, i + 64) sits in one lane, and the
// per-row epilogue work (RoPE position, residual row, KV destination) is a
// per-lane scalar. The copies for step k+1 are in flight while step k
// computes (double-buffered LDS). Workgroups are remapped so each
// XCD sweeps all column tiles of a contiguous range of token tiles, keeping
// that token tile resident in the XCD's L2.
//
// Epilogues (fused so no extra pass touches HBM):
//   STORE : y = bf16(acc * scale)
//   RESID : h = bf16(h + acc * scale)                   (O and down projections)
//   SWIGLU: m = bf16(silu(acc_gate * s_g) * acc_up * s_u)  (gate/up projection;
//           a column tile holds 64 gate rows and the 64 matching up rows)
//   QKV   : RoPE (rotate-half, table of cos/sin per position) on q and k heads,
//           then q -> q buffer; k, v -> suffix buffers or the anchor's pool slab
//           (bf16, or E4M3 codes of k/k_scale and v/v_scale).
#include "device_common.h"
#include "quail_internal.h"

namespace quail {

// token tiles per workgroup group (see the grouped order in gemm_direct_kernel)
constexpr int kGemmGroupM = 4;

// silu(g) = g / (1 + e^-g): v_exp_f32 (2^x) and v_rcp_f32, each about 1 ulp,
// far below the bf16 rounding of the product that follows
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Epilogue of one 32-row block of a wave: lane owns row m and, in column block
// nb, columns nb*32 + rg*8 + hi*4 + e (e = 0..3) of the wave's 128 columns,
// which start at n_base (SWIGLU: output column o_base, gate rows o_base + j,
// up rows inter + o_base + j for j < 64).
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, const f32x16_t (&acc)[4], int m,
                                         int n_base, int o_base, int hi) {
  if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n_base + nb * 32 + rg * 8 + hi * 4;
        const uint2 sc = *reinterpret_cast<const uint2*>(p.scale + n);
        float v0 = acc[nb][rg * 4 + 0] * bf16_bits_to_f32(sc.x & 0xFFFF);
        float v1 = acc[nb][rg * 4 + 1] * bf16_bits_to_f32(sc.x >> 16);
        float v2 = acc[nb][rg * 4 + 2] * bf16_bits_to_f32(sc.y & 0xFFFF);
        float v3 = acc[nb][rg * 4 + 3] * bf16_bits_to_f32(sc.y >> 16);
        uint2* yp = reinterpret_cast<uint2*>(p.Y + (int64_t)m * p.ldy + n);
        if (EPI == EPI_RESID) {
          const uint2 h = *yp;
          v0 += bf16_bits_to_f32(h.x & 0xFFFF);
          v1 += bf16_bits_to_f32(h.x >> 16);
          v2 += bf16_bits_to_f32(h.y & 0xFFFF);
          v3 += bf16_bits_to_f32(h.y >> 16);
        }
        *yp = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      }
    }
  } else if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = nb * 32 + rg * 8 + hi * 4;
        const uint2 sg = *reinterpret_cast<const uint2*>(p.scale + o_base + j);
        const uint2 su = *reinterpret_cast<const uint2*>(p.scale + p.inter + o_base + j);
        float g[4], u[4];
        g[0] = acc[nb][rg * 4 + 0] * bf16_bits_to_f32(sg.x & 0xFFFF);
        g[1] = acc[nb][rg * 4 + 1] * bf16_bits_to_f32(sg.x >> 16);
        g[2] = acc[nb][rg * 4 + 2] * bf16_bits_to_f32(sg.y & 0xFFFF);
        g[3] = acc[nb][rg * 4 + 3] * bf16_bits_to_f32(sg.y >> 16);
        u[0] = acc[nb + 2][rg * 4 + 0] * bf16_bits_to_f32(su.x & 0xFFFF);
        u[1] = acc[nb + 2][rg * 4 + 1] * bf16_bits_to_f32(su.x >> 16);
        u[2] = acc[nb + 2][rg * 4 + 2] * bf16_bits_to_f32(su.y & 0xFFFF);
        u[3] = acc[nb + 2][rg * 4 + 3] * bf16_bits_to_f32(su.y >> 16);
        uint2 w;
        w.x = pack_bf16x2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
        w.y = pack_bf16x2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
        *reinterpret_cast<uint2*>(p.Y + (int64_t)m * p.ldy + o_base + j) = w;
      }
    }
  } else {  // EPI_QKV: the wave's 128 columns are one head
    const int head = n_base / kHeadDim;
    const int kind = head < p.hq ? 0 : (head < p.hq + p.hkv ? 1 : 2);   // q, k, v
    float y[4][16];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n_base + nb * 32 + rg * 8 + hi * 4;
        const uint2 sc = *reinterpret_cast<const uint2*>(p.scale + n);
        y[nb][rg * 4 + 0] = acc[nb][rg * 4 + 0] * bf16_bits_to_f32(sc.x & 0xFFFF);
        y[nb][rg * 4 + 1] = acc[nb][rg * 4 + 1] * bf16_bits_to_f32(sc.x >> 16);
        y[nb][rg * 4 + 2] = acc[nb][rg * 4 + 2] * bf16_bits_to_f32(sc.y & 0xFFFF);
        y[nb][rg * 4 + 3] = acc[nb][rg * 4 + 3] * bf16_bits_to_f32(sc.y >> 16);
      }
    if (kind != 2) {
      const float2* rp = p.rope + (int64_t)p.pos[m] * 64;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = nb * 32 + rg * 8 + hi * 4 + e;
            const float2 cs = rp[i];
            const float x1 = y[nb][rg * 4 + e];
            const float x2 = y[nb + 2][rg * 4 + e];
            y[nb][rg * 4 + e] = x1 * cs.x - x2 * cs.y;
            y[nb + 2][rg * 4 + e] = x2 * cs.x + x1 * cs.y;
          }
    }
    if (kind == 0 || p.kv_mode == 0 || !p.kv_fp8) {
      uint16_t* dst;
      if (kind == 0) {
        dst = p.q_out + (int64_t)m * p.hq * kHeadDim + head * kHeadDim;
      } else if (p.kv_mode == 0) {
        const int g = head - p.hq - (kind == 2 ? p.hkv : 0);
        dst = (kind == 1 ? p.k_out : p.v_out) + ((int64_t)m * p.hkv + g) * kHeadDim;
      } else {
        const int g = head - p.hq - (kind == 2 ? p.hkv : 0);
        const int64_t off = p.kv_row[m] +
            ((int64_t)(p.layer * 2 + (kind == 2)) * p.hkv + g) * (int64_t)p.kv_lapad[m] * kHeadDim;
        dst = reinterpret_cast<uint16_t*>(p.pool) + off;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          uint2 w;
          w.x = pack_bf16x2(y[nb][rg * 4 + 0], y[nb][rg * 4 + 1]);
          w.y = pack_bf16x2(y[nb][rg * 4 + 2], y[nb][rg * 4 + 3]);
          *reinterpret_cast<uint2*>(dst + nb * 32 + rg * 8 + hi * 4) = w;
        }
    } else {
      // anchor K/V into an fp8 slab: E4M3 code of (value / scale), after the
      // bf16 rounding the value has in the bf16 pipeline
      const int g = head - p.hq - (kind == 2 ? p.hkv : 0);
      const float inv = kind == 1 ? p.k_inv_scale : p.v_inv_scale;
      const int64_t off = p.kv_row[m] +
          ((int64_t)(p.layer * 2 + (kind == 2)) * p.hkv + g) * (int64_t)p.kv_lapad[m] * kHeadDim;
      uint8_t* dst = reinterpret_cast<uint8_t*>(p.pool) + off;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          uint32_t w = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float b = bf16_bits_to_f32(f32_to_bf16_bits(y[nb][rg * 4 + e]));
            w |= f32_to_e4m3(b * inv) << (8 * e);
          }
          *reinterpret_cast<uint32_t*>(dst + nb * 32 + rg * 8 + hi * 4) = w;
        }
    }
  }
}

// ----------------------------------------------------------------------------
// The GEMM kernel: both operands copied HBM->LDS by global_load_lds (issued
// as inline asm so the compiler does not make the operand reads wait for
// copies in flight), fp8 weight codes kept as codes in LDS (half the bytes)
// and decoded after each read with v_cvt_scalef32_pk_bf16_fp8 (exact, scale
// 1). k-steps of 64 over 3 LDS stages; the copies of step k+2 are in flight
// while step k computes. Each step starts with an explicit wait for this
// step's copies and a raw s_barrier (a fenced __syncthreads would wait for all
// copies in flight).
//
// k order inside a step: the MFMA k-slots may take any permutation of k as
// long as both operands use the same one. Here MFMA t of pair j (k-substep
// 2j+t), lane group h (= lane / 32), element e holds k = 32j + 16h + 8t + e,
// so that one 16-B read of a weight row gives a lane the codes of two
// MFMAs.
//
// LDS (64 banks x 4 B per cycle; a 16-B read serves 16 lanes per cycle): A
// rows are 128 B, chunk ^= (row/2) % 8; B rows are 64 B, chunk ^= (row/4) % 4;
// the 16 rows one read cycle touches then hit 16 distinct chunks.
// ----------------------------------------------------------------------------
__device__ __forceinline__ int swz_a(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int swz_b(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// 8 E4M3 codes -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bitcast<bf16x8_t>(make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)));
}

template <int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_direct_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int MW = BM / WM;
  constexpr int MB = MW / 32;
  constexpr int STAGES = 3;
  constexpr int A_ROW = 128, B_ROW = 64;           // bytes per LDS row (k = 64)
  constexpr int A_BYTES = BM * A_ROW, B_BYTES = BN * B_ROW;
  constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;   // 1-KB copies per wave
  constexpr int CPW = A_PW + B_PW;
  static_assert(BN / WN == 128, "each wave owns 128 columns");
  static_assert((A_BYTES / 1024) % NW == 0 && (B_BYTES / 1024) % NW == 0, "copy split");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES][A_BYTES + B_BYTES];

  const int n_tn = (EPI == EPI_SWIGLU) ? p.N / (BN / 2) : p.N / BN;
  const int n_tm = (p.M + BM - 1) / BM;
  const int64_t total = (int64_t)n_tn * n_tm;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  // Grouped order: logical ids sweep kGemmGroupM token tiles x all column
  // tiles, column-major inside the group, so the workgroups that run at the
  // same time on one XCD share both their activation rows and their weight
  // rows through that XCD's L2.
  const int64_t per_group = (int64_t)kGemmGroupM * n_tn;
  const int64_t grp = wid / per_group;
  const int64_t rem = wid % per_group;
  const int gm_rows = (int)min<int64_t>(kGemmGroupM, n_tm - grp * kGemmGroupM);
  const int tm = (int)(grp * kGemmGroupM + rem % gm_rows);
  const int tn = (int)(rem / gm_rows);
  const int m0 = tm * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int wm = wave % WM;
  const int wn = wave / WM;

  auto wrow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) {
      const int pr = r >> 7, j = r & 63;
      const int base = tn * (BN / 2) + pr * 64 + j;
      return (r & 64) ? p.inter + base : base;
    }
    return tn * BN + r;
  };
  // per-lane copy sources: A copies are 8 rows x 128 B, B copies 16 rows x 64 B
  const uint8_t* a_src[A_PW];
  const uint8_t* b_src[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 8 + (lane >> 3);
    const int m = min(m0 + row, p.M - 1);
    a_src[i] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)m * p.lda) + swz_a(row, lane & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_PW; ++i) {
    const int row = (wave * B_PW + i) * 16 + (lane >> 2);
    b_src[i] = p.B + (int64_t)wrow(row) * p.K + swz_b(row, lane & 3) * 16;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem[kt % STAGES];
#pragma unroll
    for (int i = 0; i < A_PW; ++i) copy16_to_lds(a_src[i] + kt * 128, st + (wave * A_PW + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_PW; ++i) copy16_to_lds(b_src[i] + kt * 64, st + A_BYTES + (wave * B_PW + i) * 1024);
  };

  f32x16_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  const int nk = p.K / 64;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmcnt<CPW>();      // the copies of step kt+1 may stay in flight
    else wait_vmcnt<0>();
    raw_barrier();                           // step kt landed everywhere; stage (kt-1)%3 is free
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const uint8_t* st = smem[kt % STAGES];
#pragma unroll
    for (int j = 0; j < 2; ++j) {            // pairs of MFMA k-substeps
      uint4 bw[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = wn * 128 + nb * 32 + l32;
        bw[nb] = *reinterpret_cast<const uint4*>(st + A_BYTES + row * B_ROW + swz_b(row, 2 * j + hi) * 16);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8_t af[MB], bfr[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = wm * MW + mb * 32 + l32;
          af[mb] = bitcast<bf16x8_t>(
              *reinterpret_cast<const uint4*>(st + row * A_ROW + swz_a(row, 4 * j + 2 * hi + t) * 16));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          bfr[nb] = t == 0 ? fp8x8_to_bf16x8(bw[nb].x, bw[nb].y) : fp8x8_to_bf16x8(bw[nb].z, bw[nb].w);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_32x32x16(bfr[nb], af[mb], acc[mb][nb]);
      }
    }
  }

  const int n_base = tn * BN + wn * 128;
  const int o_base = tn * (BN / 2) + wn * 64;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + wm * MW + mb * 32 + l32;
    if (m >= p.M) continue;
    epilogue<EPI>(p, acc[mb], m, n_base, o_base, hi);
  }
}

hipError_t launch_gemm(const GemmParams& p, GemmEpi epi, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  // 256x256 tiles (8 waves of 64 rows x 128 columns) when the columns allow
  // (SWIGLU: 128 output columns per tile), else 256x128 (4 waves)
  const bool wide = (epi == EPI_SWIGLU) ? (p.N % 128 == 0) : (p.N % 256 == 0);
  const int bn = wide ? 256 : 128;
  const int n_tn = (epi == EPI_SWIGLU) ? p.N / (bn / 2) : p.N / bn;
  const int64_t total = (int64_t)n_tn * ((p.M + 255) / 256);
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid);
#define QUAIL_GEMM_LAUNCH(E)                                                              \
  if (wide) gemm_direct_kernel<E, 256, 256, 4, 2><<<g, dim3(512), 0, s>>>(p);             \
  else gemm_direct_kernel<E, 256, 128, 4, 1><<<g, dim3(256), 0, s>>>(p);
  switch (epi) {
    case EPI_STORE: QUAIL_GEMM_LAUNCH(EPI_STORE); break;
    case EPI_RESID: QUAIL_GEMM_LAUNCH(EPI_RESID); break;
    case EPI_SWIGLU: QUAIL_GEMM_LAUNCH(EPI_SWIGLU); break;
    case EPI_QKV: QUAIL_GEMM_LAUNCH(EPI_QKV); break;
    default: return hipErrorInvalidValue;
  }
#undef QUAIL_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace quail
