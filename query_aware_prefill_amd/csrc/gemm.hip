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
// Tiling: a 256 (tokens) x 128 (output columns) x 64 (k) workgroup tile, four
// waves of 64 tokens x 128 columns. The MFMA computes the transposed product
// D = W_tile . X_tile^T (v_mfma_f32_32x32x16_bf16), so each lane owns one
// token row and 16 output columns per 32-column block: a whole 128-column
// head lives in one wave, the RoPE pair (i, i + 64) sits in one lane, and the
// per-row epilogue work (RoPE position, residual row, KV destination) is a
// per-lane scalar. Global loads for step k+1 are issued before the MFMAs of
// step k (register prefetch, one LDS buffer). Workgroups are remapped so each
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

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int ASTR = BK + 8;   // LDS row stride (u16): 144 B
constexpr int BSTR = BK + 8;

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int EPI>
__global__ void __launch_bounds__(256) gemm_w8a16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * ASTR];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * BSTR];

  const int n_tn = (EPI == EPI_SWIGLU) ? p.N / 64 : p.N / BN;
  const int n_tm = (p.M + BM - 1) / BM;
  const int64_t total = (int64_t)n_tn * n_tm;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  const int tm = (int)(wid / n_tn);
  const int tn = (int)(wid % n_tn);
  const int m0 = tm * BM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // weight row of LDS B-tile row r
  auto wrow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) return r < 64 ? tn * 64 + r : p.inter + tn * 64 + (r - 64);
    return tn * BN + r;
  };

  uint4 ra[8];
  uint4 rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int chunk = tid + 256 * j;
      const int row = chunk >> 3;
      const int kc = chunk & 7;
      const int m = m0 + row;
      ra[j] = m < p.M ? *reinterpret_cast<const uint4*>(p.A + (int64_t)m * p.lda + k0 + kc * 8)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = tid + 256 * j;
      const int row = chunk >> 2;
      const int kc = chunk & 3;
      rb[j] = *reinterpret_cast<const uint4*>(p.B + (int64_t)wrow(row) * p.K + k0 + kc * 16);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int chunk = tid + 256 * j;
      *reinterpret_cast<uint4*>(As + (chunk >> 3) * ASTR + (chunk & 7) * 8) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = tid + 256 * j;
      uint32_t w[8];
      fp8x4_to_bf16x4(rb[j].x, w[0], w[1]);
      fp8x4_to_bf16x4(rb[j].y, w[2], w[3]);
      fp8x4_to_bf16x4(rb[j].z, w[4], w[5]);
      fp8x4_to_bf16x4(rb[j].w, w[6], w[7]);
      uint16_t* dst = Bs + (chunk >> 2) * BSTR + (chunk & 3) * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
    }
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  const int nk = p.K / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[2], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4*>(
            As + (wave * 64 + mb * 32 + l32) * ASTR + kk * 16 + hi * 8));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bfr[nb] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4*>(
            Bs + (nb * 32 + l32) * BSTR + kk * 16 + hi * 8));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_32x32x16(bfr[nb], af[mb], acc[mb][nb]);
    }
  }

  // ---- epilogue: lane owns row m, columns nb*32 + rg*8 + hi*4 + e ----
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wave * 64 + mb * 32 + l32;
    if (m >= p.M) continue;
    if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = tn * BN + nb * 32 + rg * 8 + hi * 4;
          const uint2 sc = *reinterpret_cast<const uint2*>(p.scale + n);
          float v0 = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sc.x & 0xFFFF);
          float v1 = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sc.x >> 16);
          float v2 = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sc.y & 0xFFFF);
          float v3 = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sc.y >> 16);
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
          const uint2 sg = *reinterpret_cast<const uint2*>(p.scale + tn * 64 + j);
          const uint2 su = *reinterpret_cast<const uint2*>(p.scale + p.inter + tn * 64 + j);
          float g[4], u[4];
          g[0] = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sg.x & 0xFFFF);
          g[1] = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sg.x >> 16);
          g[2] = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sg.y & 0xFFFF);
          g[3] = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sg.y >> 16);
          u[0] = acc[mb][nb + 2][rg * 4 + 0] * bf16_bits_to_f32(su.x & 0xFFFF);
          u[1] = acc[mb][nb + 2][rg * 4 + 1] * bf16_bits_to_f32(su.x >> 16);
          u[2] = acc[mb][nb + 2][rg * 4 + 2] * bf16_bits_to_f32(su.y & 0xFFFF);
          u[3] = acc[mb][nb + 2][rg * 4 + 3] * bf16_bits_to_f32(su.y >> 16);
          uint2 w;
          w.x = pack_bf16x2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
          w.y = pack_bf16x2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
          *reinterpret_cast<uint2*>(p.Y + (int64_t)m * p.ldy + tn * 64 + j) = w;
        }
      }
    } else {  // EPI_QKV: column tile tn is one head
      const int head = tn;
      const int kind = head < p.hq ? 0 : (head < p.hq + p.hkv ? 1 : 2);   // q, k, v
      float y[4][16];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = head * BN + nb * 32 + rg * 8 + hi * 4;
          const uint2 sc = *reinterpret_cast<const uint2*>(p.scale + n);
          y[nb][rg * 4 + 0] = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sc.x & 0xFFFF);
          y[nb][rg * 4 + 1] = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sc.x >> 16);
          y[nb][rg * 4 + 2] = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sc.y & 0xFFFF);
          y[nb][rg * 4 + 3] = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sc.y >> 16);
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
}

hipError_t launch_gemm(const GemmParams& p, GemmEpi epi, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  const int n_tn = (epi == EPI_SWIGLU) ? p.N / 64 : p.N / BN;
  const int64_t total = (int64_t)n_tn * ((p.M + BM - 1) / BM);
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(256);
  switch (epi) {
    case EPI_STORE: gemm_w8a16_kernel<EPI_STORE><<<g, b, 0, s>>>(p); break;
    case EPI_RESID: gemm_w8a16_kernel<EPI_RESID><<<g, b, 0, s>>>(p); break;
    case EPI_SWIGLU: gemm_w8a16_kernel<EPI_SWIGLU><<<g, b, 0, s>>>(p); break;
    case EPI_QKV: gemm_w8a16_kernel<EPI_QKV><<<g, b, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace quail
