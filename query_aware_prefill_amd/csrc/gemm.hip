// W8A16 GEMM for the decoder projections on gfx950 (and its W8A8 variant,
// gemm_a8_kernel, for per-token E4M3 activations).
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
//   RESID : h = h + acc * scale, h the fp32 residual     (O and down projections)
//           (optionally gathered: A rows and residual rows through row maps,
//           for the rows whose output is still needed)
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

// ----------------------------------------------------------------------------
// Staged epilogue of one wave tile (MB blocks of 32 tokens x 128 columns).
// In the MFMA output layout a lane owns one token and, in column block nb,
// columns nb*32 + rg*8 + hi*4 + e (e = 0..3) of the wave's 128 columns, which
// start at n_base (SWIGLU: output column o_base, gate rows o_base + j, up rows
// inter + o_base + j for j < 64). Stored directly, one instruction would write
// 8-byte pieces of 32 different rows; instead each 32-token block is written
// to an 8-KB LDS region of the wave (rows XOR-swizzled by 16-byte chunk) and
// read back so that 8 or 16 lanes cover one row: every global store and
// residual load then moves whole 16-byte pieces of contiguous rows. The
// caller hands each wave its own region after a workgroup barrier that ends
// the use of the pipeline stages; LDS operations of one wave complete in
// order, so no further barrier is needed.
//   lds: wave-uniform LDS byte address of the region; m_row0: first token of
//   the wave tile.
// ----------------------------------------------------------------------------
typedef uint32_t lds_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t lds_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_write_b64(uint32_t addr, uint2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) lds_u32x2*>(addr) = __builtin_bit_cast(lds_u32x2, v);
}
__device__ __forceinline__ void lds_write_b128(uint32_t addr, uint4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) lds_u32x4*>(addr) = __builtin_bit_cast(lds_u32x4, v);
}
__device__ __forceinline__ void lds_write_b32(uint32_t addr, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(addr) = v;
}
__device__ __forceinline__ uint4 lds_read_b128(uint32_t addr) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) lds_u32x4*>(addr));
}

// bf16 (or E4M3 when FP8) rows of 128 columns: STORE and QKV
template <int EPI, bool FP8, int MB>
__device__ __forceinline__ void epilogue_rows(const GemmParams& p, const f32x16_t (&acc)[MB][4],
                                              uint32_t lds, int m_row0, int n_base, int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  int kind = 0, g = 0;
  float inv = 1.0f;
  if (EPI == EPI_QKV) {
    const int head = n_base / kHeadDim;
    kind = head < p.hq ? 0 : (head < p.hq + p.hkv ? 1 : 2);
    g = head - p.hq - (kind == 2 ? p.hkv : 0);
    inv = kind == 1 ? p.k_inv_scale : p.v_inv_scale;
  }
  // bf16 rows: 256 B = 16 chunks, swizzle row & 15; E4M3 rows: 128 B = 8
  // chunks, swizzle row & 7
  constexpr int ROW = FP8 ? 128 : 256;
  constexpr int SWM = FP8 ? 7 : 15;
  constexpr int LPR = FP8 ? 8 : 16;          // lanes per row on the way out
  constexpr int PASSES = 32 * LPR / 64;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m_row0 + mb * 32 + l32;
    const float2* rp = nullptr;
    if (EPI == EPI_QKV && kind != 2) rp = p.rope + (int64_t)p.pos[min(m, p.M - 1)] * 64;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int i0 = nb * 32 + rg * 8 + hi * 4;
        const uint2 s1 = *reinterpret_cast<const uint2*>(p.scale + n_base + i0);
        const uint2 s2 = *reinterpret_cast<const uint2*>(p.scale + n_base + 64 + i0);
        float x1[4], x2[4];
        x1[0] = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(s1.x & 0xFFFF);
        x1[1] = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(s1.x >> 16);
        x1[2] = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(s1.y & 0xFFFF);
        x1[3] = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(s1.y >> 16);
        x2[0] = acc[mb][nb + 2][rg * 4 + 0] * bf16_bits_to_f32(s2.x & 0xFFFF);
        x2[1] = acc[mb][nb + 2][rg * 4 + 1] * bf16_bits_to_f32(s2.x >> 16);
        x2[2] = acc[mb][nb + 2][rg * 4 + 2] * bf16_bits_to_f32(s2.y & 0xFFFF);
        x2[3] = acc[mb][nb + 2][rg * 4 + 3] * bf16_bits_to_f32(s2.y >> 16);
        if (EPI == EPI_QKV && kind != 2) {
          // RoPE (rotate-half): pairs (i, i + 64) sit in blocks nb, nb + 2
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 cs = rp[i0 + e];
            const float a = x1[e], b = x2[e];
            x1[e] = a * cs.x - b * cs.y;
            x2[e] = b * cs.x + a * cs.y;
          }
        }
        if (!FP8) {
          // column i0 is chunk i0/8 = nb*4 + rg, 8-byte half hi
          const int c1 = nb * 4 + rg, c2 = c1 + 8;
          lds_write_b64(lds + l32 * ROW + ((c1 ^ (l32 & SWM)) << 4) + hi * 8,
                        make_uint2(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])));
          lds_write_b64(lds + l32 * ROW + ((c2 ^ (l32 & SWM)) << 4) + hi * 8,
                        make_uint2(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3])));
        } else {
          // E4M3 code of (value / scale), after the bf16 rounding the value
          // has in the bf16 pipeline; column i0 is chunk i0/16
          uint32_t w1 = 0, w2 = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w1 |= f32_to_e4m3(bf16_bits_to_f32(f32_to_bf16_bits(x1[e])) * inv) << (8 * e);
            w2 |= f32_to_e4m3(bf16_bits_to_f32(f32_to_bf16_bits(x2[e])) * inv) << (8 * e);
          }
          const int c1 = i0 >> 4, c2 = c1 + 4;
          lds_write_b32(lds + l32 * ROW + ((c1 ^ (l32 & SWM)) << 4) + (i0 & 15), w1);
          lds_write_b32(lds + l32 * ROW + ((c2 ^ (l32 & SWM)) << 4) + (i0 & 15), w2);
        }
      }
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int r = it * (64 / LPR) + lane / LPR;
      const int c = lane % LPR;
      const uint4 v = lds_read_b128(lds + r * ROW + ((c ^ (r & SWM)) << 4));
      const int mr = m_row0 + mb * 32 + r;
      if (mr >= p.M) continue;
      uint4* dst;
      if (EPI == EPI_STORE) {
        dst = reinterpret_cast<uint4*>(p.Y + (int64_t)mr * p.ldy + n_base + c * 8);
      } else if (kind == 0) {
        dst = reinterpret_cast<uint4*>(p.q_out + (int64_t)mr * p.hq * kHeadDim + n_base + c * 8);
      } else if (p.kv_mode == 0) {
        dst = reinterpret_cast<uint4*>((kind == 1 ? p.k_out : p.v_out) + ((int64_t)mr * p.hkv + g) * kHeadDim + c * 8);
      } else {
        const int64_t off = p.kv_row[mr] +
            ((int64_t)(p.layer * 2 + (kind == 2)) * p.hkv + g) * (int64_t)p.kv_lapad[mr] * kHeadDim;
        dst = FP8 ? reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.pool) + off + c * 16)
                  : reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.pool) + off + c * 8);
      }
      *dst = v;
    }
  }
}

template <int EPI, int MB>
__device__ __forceinline__ void epilogue_staged(const GemmParams& p, const f32x16_t (&acc)[MB][4],
                                                uint32_t lds, int m_row0, int n_base, int o_base,
                                                int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int sw16 = l32 & 15;                 // row swizzle of the writing lane (row = l32)
  if (EPI == EPI_STORE) {
    epilogue_rows<EPI_STORE, false, MB>(p, acc, lds, m_row0, n_base, lane);
  } else if (EPI == EPI_QKV) {
    const int head = n_base / kHeadDim;
    const bool to_fp8 = head >= p.hq && p.kv_mode == 1 && p.kv_fp8;
    if (to_fp8) epilogue_rows<EPI_QKV, true, MB>(p, acc, lds, m_row0, n_base, lane);
    else epilogue_rows<EPI_QKV, false, MB>(p, acc, lds, m_row0, n_base, lane);
  } else if (EPI == EPI_RESID) {
    // fp32 staging (the residual add happens after the read-back): per 32
    // tokens and 64 columns, 256-B rows
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int nbl = 0; nbl < 2; ++nbl)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int nb = half * 2 + nbl;
            const int n = n_base + nb * 32 + rg * 8 + hi * 4;
            const uint2 sc = *reinterpret_cast<const uint2*>(p.scale + n);
            uint4 v;
            v.x = __float_as_uint(acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sc.x & 0xFFFF));
            v.y = __float_as_uint(acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sc.x >> 16));
            v.z = __float_as_uint(acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sc.y & 0xFFFF));
            v.w = __float_as_uint(acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sc.y >> 16));
            const int c = nbl * 8 + rg * 2 + hi;             // 16-B chunk of 4 fp32
            lds_write_b128(lds + l32 * 256 + ((c ^ sw16) << 4), v);
          }
        // 8 lanes per row (8 columns each): 8 rows per pass
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 8 + (lane >> 3);
          const int c8 = lane & 7;                           // 8 columns = chunks 2c8, 2c8+1
          const uint4 a = lds_read_b128(lds + r * 256 + (((2 * c8) ^ (r & 15)) << 4));
          const uint4 b = lds_read_b128(lds + r * 256 + (((2 * c8 + 1) ^ (r & 15)) << 4));
          const int mr = m_row0 + mb * 32 + r;
          if (mr >= p.M) continue;
          const int yr = p.y_map ? p.y_map[mr] : mr;
          float4* yp = reinterpret_cast<float4*>(p.Yf + (int64_t)yr * p.ldy + n_base + half * 64 + c8 * 8);
          const float4 h0 = yp[0], h1 = yp[1];
          yp[0] = make_float4(__uint_as_float(a.x) + h0.x, __uint_as_float(a.y) + h0.y,
                              __uint_as_float(a.z) + h0.z, __uint_as_float(a.w) + h0.w);
          yp[1] = make_float4(__uint_as_float(b.x) + h1.x, __uint_as_float(b.y) + h1.y,
                              __uint_as_float(b.z) + h1.z, __uint_as_float(b.w) + h1.w);
        }
      }
    }
  } else {  // EPI_SWIGLU: 64 output columns, bf16 rows of 128 B (8 chunks)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int j = nb * 32 + rg * 8 + hi * 4;
          const uint2 sg = *reinterpret_cast<const uint2*>(p.scale + o_base + j);
          const uint2 su = *reinterpret_cast<const uint2*>(p.scale + p.inter + o_base + j);
          float gt[4], u[4];
          gt[0] = acc[mb][nb][rg * 4 + 0] * bf16_bits_to_f32(sg.x & 0xFFFF);
          gt[1] = acc[mb][nb][rg * 4 + 1] * bf16_bits_to_f32(sg.x >> 16);
          gt[2] = acc[mb][nb][rg * 4 + 2] * bf16_bits_to_f32(sg.y & 0xFFFF);
          gt[3] = acc[mb][nb][rg * 4 + 3] * bf16_bits_to_f32(sg.y >> 16);
          u[0] = acc[mb][nb + 2][rg * 4 + 0] * bf16_bits_to_f32(su.x & 0xFFFF);
          u[1] = acc[mb][nb + 2][rg * 4 + 1] * bf16_bits_to_f32(su.x >> 16);
          u[2] = acc[mb][nb + 2][rg * 4 + 2] * bf16_bits_to_f32(su.y & 0xFFFF);
          u[3] = acc[mb][nb + 2][rg * 4 + 3] * bf16_bits_to_f32(su.y >> 16);
          const int c = nb * 4 + rg;
          lds_write_b64(lds + l32 * 128 + ((c ^ (l32 & 7)) << 4) + hi * 8,
                        make_uint2(pack_bf16x2(silu_f(gt[0]) * u[0], silu_f(gt[1]) * u[1]),
                                   pack_bf16x2(silu_f(gt[2]) * u[2], silu_f(gt[3]) * u[3])));
        }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int c = lane & 7;
        const uint4 v = lds_read_b128(lds + r * 128 + ((c ^ (r & 7)) << 4));
        const int mr = m_row0 + mb * 32 + r;
        if (mr < p.M) *reinterpret_cast<uint4*>(p.Y + (int64_t)mr * p.ldy + o_base + c * 8) = v;
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
    const int ma = p.a_map ? p.a_map[m] : m;
    a_src[i] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)ma * p.lda) + swz_a(row, lane & 7) * 16;
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
  __syncthreads();   // every wave is done with the stages: they become staging space
  epilogue_staged<EPI, MB>(p, acc, lds_addr_of(&smem[0][0]) + wave * 8192, m0 + wm * MW, n_base, o_base, lane);
}

// ----------------------------------------------------------------------------
// W8A8 kernel: E4M3 activation codes (one fp32 scale per row) times E4M3
// weights on the fp8 MFMA, v_mfma_scale_f32_32x32x64_f8f6f4 (twice the bf16
// rate; scale operands 127 = E8M0 2^0, so a plain product; format selectors
// 0 = E4M3 for both operands). Same workgroup tile, wave split, tile order
// and epilogues as gemm_direct_kernel; the k-step is 128 bytes of both
// operands (the same MFMA time per step as the bf16 kernel's 64), staged over
// 2 LDS stages of 64 KB. The MFMA operand layout: a lane holds 32 codes of
// row lane % 32, lanes 0-31 one half of the MFMA's 64 k values and lanes
// 32-63 the other; the sum over k does not depend on how a lane's values are
// ordered as long as both operands order them alike: lane half h of MFMA
// sub-step j holds bytes [64 j + 32 h, 64 j + 32 h + 32) of the k-step for
// weights and activations both. LDS rows are 128 B with chunk ^= (row/2) % 8.
// Before the epilogue each lane multiplies its token's accumulators by the
// token's activation scale; the epilogue then applies the weight scales.
// ----------------------------------------------------------------------------
constexpr int kGemmA8GroupM = 2;   // token tiles per group (measured best for this kernel)

// D = W . X^T on one 32x32x64 block: (w0, w1) the 32 weight codes of this
// lane, (x0, x1) its 32 activation codes
__device__ __forceinline__ f32x16_t mfma_f8_32x32x64(const uint4& w0, const uint4& w1, const uint4& x0,
                                                     const uint4& x1, f32x16_t c) {
  typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t a = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
  const i32x8_t b = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int EPI>
__global__ void __launch_bounds__(512)
gemm_a8_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 4, NW = 8, MB = 2;
  constexpr int KS = 128;                           // bytes (= k values) per step
  constexpr int TILE = BM * KS;                     // 32 KB per operand and stage
  constexpr int PW = TILE / 1024 / NW;              // 1-KB copies per wave per operand
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2 * TILE];

  const int n_tn = (EPI == EPI_SWIGLU) ? p.N / (BN / 2) : p.N / BN;
  const int n_tm = (p.M + BM - 1) / BM;
  const int64_t total = (int64_t)n_tn * n_tm;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  const int64_t per_group = (int64_t)kGemmA8GroupM * n_tn;
  const int64_t grp = wid / per_group;
  const int64_t rem = wid % per_group;
  const int gm_rows = (int)min<int64_t>(kGemmA8GroupM, n_tm - grp * kGemmA8GroupM);
  const int tm = (int)(grp * kGemmA8GroupM + rem % gm_rows);
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
  // per-lane copy sources, 8 rows x 128 B per copy (rows past M read row
  // M - 1; their results are not stored)
  const uint8_t* a_src[PW];
  const uint8_t* b_src[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int row = (wave * PW + i) * 8 + (lane >> 3);
    const int m = min(m0 + row, p.M - 1);
    const int ma = p.a_map ? p.a_map[m] : m;
    a_src[i] = p.A8 + (int64_t)ma * p.lda + swz_a(row, lane & 7) * 16;
    b_src[i] = p.B + (int64_t)wrow(row) * p.K + swz_a(row, lane & 7) * 16;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem[kt & 1];
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
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    raw_barrier();                 // step kt landed everywhere; the other stage is free
    if (kt + 1 < nk) issue(kt + 1);
    const uint8_t* st = smem[kt & 1];
#pragma unroll
    for (int j = 0; j < KS / 64; ++j) {
      const int c0 = 4 * j + 2 * hi;
      uint4 b0[4], b1[4], a0[MB], a1[MB];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const uint8_t* rb = st + TILE + (wn * 128 + nb * 32 + l32) * KS;
        const int row = wn * 128 + nb * 32 + l32;
        b0[nb] = *reinterpret_cast<const uint4*>(rb + swz_a(row, c0) * 16);
        b1[nb] = *reinterpret_cast<const uint4*>(rb + swz_a(row, c0 + 1) * 16);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = wm * 64 + mb * 32 + l32;
        const uint8_t* rb = st + row * KS;
        a0[mb] = *reinterpret_cast<const uint4*>(rb + swz_a(row, c0) * 16);
        a1[mb] = *reinterpret_cast<const uint4*>(rb + swz_a(row, c0 + 1) * 16);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = mfma_f8_32x32x64(b0[nb], b1[nb], a0[mb], a1[mb], acc[mb][nb]);
    }
  }

  // the token's activation scale (lane = token within each 32-token block)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = min(m0 + wm * 64 + mb * 32 + l32, p.M - 1);
    const float sx = p.a_scale[p.a_map ? p.a_map[m] : m];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] *= sx;
  }
  const int n_base = tn * BN + wn * 128;
  const int o_base = tn * (BN / 2) + wn * 64;
  __syncthreads();   // every wave is done with the stages: they become staging space
  epilogue_staged<EPI, MB>(p, acc, lds_addr_of(&smem[0][0]) + wave * 8192, m0 + wm * 64, n_base, o_base, lane);
}

hipError_t launch_gemm(const GemmParams& p, GemmEpi epi, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  if (p.A8) {
    // 256x256 tiles only (SWIGLU: 128 output columns per tile); K in steps of 128
    if ((epi == EPI_SWIGLU ? p.N % 128 : p.N % 256) || p.K % 128 || !p.a_scale) return hipErrorInvalidValue;
    const int n_tn = (epi == EPI_SWIGLU) ? p.N / 128 : p.N / 256;
    const int64_t total = (int64_t)n_tn * ((p.M + 255) / 256);
    const int64_t grid = (total + 7) / 8 * 8;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    switch (epi) {
      case EPI_STORE: gemm_a8_kernel<EPI_STORE><<<g, dim3(512), 0, s>>>(p); break;
      case EPI_RESID: gemm_a8_kernel<EPI_RESID><<<g, dim3(512), 0, s>>>(p); break;
      case EPI_SWIGLU: gemm_a8_kernel<EPI_SWIGLU><<<g, dim3(512), 0, s>>>(p); break;
      case EPI_QKV: gemm_a8_kernel<EPI_QKV><<<g, dim3(512), 0, s>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
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
