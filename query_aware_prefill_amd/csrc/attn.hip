// Cascade attention for AI.IF join prefill on gfx950.
//
// [pt] "Como funciona", simplified cascade attention: each suffix token
// attends to every key of its anchor (cross-attention), then causally to the
// keys of its own suffix, and the two softmax partials are combined by LSE
// rescaling. The same kernel runs the anchor's own causal attention (no
// cross part; the "self" keys are the anchor's stored slab).
//
// bf16 kernel (head_dim 128)
// --------------------------
// One workgroup = one tile of query tokens x one KV head g. Its NW waves cover
// the G query heads of g (GQA group) x NW/G groups of 32 tokens; every wave
// reads the same K/V tiles from LDS. Per 64-key tile each wave computes
//   S^T = K . Q^T      (v_mfma_f32_32x32x16_bf16, A = K rows, B = Q rows)
// so that each lane owns ONE query row (lane % 32) and 32 of the tile's keys:
// the row max and row sum are per-lane scalars, combined with the partner
// lane (lane ^ 32) by one exchange. Then
//   O^T += V^T . P^T   (A = V^T rows from a transposed LDS tile, B = P)
// where P comes straight from the S^T accumulator registers in the k-slot
// order the MFMA expects; V^T is read with the same key permutation.
// The cross keys and the self keys form one sequence of tiles with one online
// softmax: rescaling the running cross accumulator by exp(m_cross - m) when
// the self keys arrive is exactly the LSE merge of the two partials
// (O = e^(L_c - L) O_c + e^(L_s - L) O_s with L = logaddexp(L_c, L_s)).
//
// fp32 kernel (head_dim 64 or 128)
// --------------------------------
// One wave per (query token, query head); computes the cross partial (O_c,
// L_c) and the self partial (O_s, L_s) separately and merges them with the
// LSE formula. Used for the fp32 configuration, where accuracy, not speed,
// is the point.
#include "device_common.h"
#include "quail_internal.h"

namespace quail {

// A wave-uniform value as an opaque register operand: a choice among
// members of one object, made on such values, cannot be folded into a load
// through a chosen member address (which would keep the object in scratch
// memory instead of registers).
template <typename T>
__device__ __forceinline__ T in_sreg(T x) {
  asm volatile("" : "+s"(x));
  return x;
}

constexpr int KSTR = kHeadDim + 8;   // K tile row stride in LDS (u16): 272 B
constexpr int VSTR = kKeyTile + 4;   // V^T tile row stride in LDS (u16): 136 B

struct TileView {
  const uint8_t* k;       // byte pointer to (row 0, head g)
  const uint8_t* v;
  int64_t tok_bytes;      // bytes between tokens
  int32_t kbase;          // first key index of the tile
  int32_t len;            // valid rows of the source
  int32_t fp8;
};

// Register prefetch of one K/V tile. K: KC chunks of 8 elements per thread.
// V: one 4-key x 8-dim block per thread (threads < 256).
template <int NT>
struct TileRegs {
  static constexpr int KC = (kKeyTile * kHeadDim / 8) / NT;
  uint4 k[KC];
  uint4 v[4];
};

// Rows at or beyond the source length are clamped to its last row: their
// scores are masked to -inf and their P is 0, so only finiteness matters, and
// the loads stay unconditional (no wait per load).
template <int NT>
__device__ __forceinline__ void load_tile(TileRegs<NT>& r, const TileView& t, int tid) {
  if (t.fp8) {
#pragma unroll
    for (int i = 0; i < TileRegs<NT>::KC; ++i) {
      const int chunk = tid + i * NT;
      const int key = min(t.kbase + (chunk >> 4), t.len - 1);
      const uint2 w = *reinterpret_cast<const uint2*>(t.k + (int64_t)key * t.tok_bytes + (chunk & 15) * 8);
      r.k[i] = make_uint4(w.x, w.y, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TileRegs<NT>::KC; ++i) {
      const int chunk = tid + i * NT;
      const int key = min(t.kbase + (chunk >> 4), t.len - 1);
      r.k[i] = *reinterpret_cast<const uint4*>(t.k + (int64_t)key * t.tok_bytes + (chunk & 15) * 16);
    }
  }
  if (NT <= 256 || tid < 256) {
    // V block: 4 keys x 8 dims; key groups run fastest across lanes so that
    // the transposed LDS writes of 16 lanes form one contiguous 128-B row
    const int blk = tid & 255;
    const int kg = blk & 15;
    const int c8 = blk >> 4;
    if (t.fp8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(t.kbase + kg * 4 + j, t.len - 1);
        const uint2 w = *reinterpret_cast<const uint2*>(t.v + (int64_t)key * t.tok_bytes + c8 * 8);
        r.v[j] = make_uint4(w.x, w.y, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(t.kbase + kg * 4 + j, t.len - 1);
        r.v[j] = *reinterpret_cast<const uint4*>(t.v + (int64_t)key * t.tok_bytes + c8 * 16);
      }
    }
  }
}

template <int NT>
__device__ __forceinline__ void store_tile(const TileRegs<NT>& r, int fp8, float ks, float vs,
                                           uint16_t* Ks, uint16_t* Vt, int tid) {
#pragma unroll
  for (int i = 0; i < TileRegs<NT>::KC; ++i) {
    const int chunk = tid + i * NT;
    const int row = chunk >> 4;
    const int c8 = chunk & 15;
    uint4 val = r.k[i];
    if (fp8) {
      uint32_t a, b, c, d;
      fp8x4_to_bf16x4_scaled(val.x, ks, a, b);
      fp8x4_to_bf16x4_scaled(val.y, ks, c, d);
      val = make_uint4(a, b, c, d);
    }
    *reinterpret_cast<uint4*>(Ks + row * KSTR + c8 * 8) = val;
  }
  if (NT <= 256 || tid < 256) {
    const int blk = tid & 255;
    const int kg = blk & 15;
    const int c8 = blk >> 4;
    uint32_t w[4][4];   // w[j] = 8 bf16 of key kg*4+j, packed in 4 words
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 val = r.v[j];
      if (fp8) {
        uint32_t a, b, c, d;
        fp8x4_to_bf16x4_scaled(val.x, vs, a, b);
        fp8x4_to_bf16x4_scaled(val.y, vs, c, d);
        val = make_uint4(a, b, c, d);
      }
      w[j][0] = val.x; w[j][1] = val.y; w[j][2] = val.z; w[j][3] = val.w;
    }
    // transpose: dim c8*8 + e, keys kg*4 .. kg*4+3
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // bytes of the low (e even) or high (e odd) halves of two words
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int word = e >> 1;
      uint2 out;
      out.x = __builtin_amdgcn_perm(w[1][word], w[0][word], sel);
      out.y = __builtin_amdgcn_perm(w[3][word], w[2][word], sel);
      *reinterpret_cast<uint2*>(Vt + (c8 * 8 + e) * VSTR + kg * 4) = out;
    }
  }
}

template <int G>
__global__ void __launch_bounds__(64 * (G >= 4 ? G : 4))
attn_bf16_kernel(AttnParams p) {
  constexpr int NW = G >= 4 ? G : 4;     // waves per workgroup
  constexpr int NT = 64 * NW;
  constexpr int TOKG = NW / G;           // token groups of 32
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKeyTile * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VSTR];

  const int64_t total = (int64_t)p.n_tiles * p.hkv;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  const int g = (int)(wid / p.n_tiles);            // kv head (slow index)
  const AttnTile tile = p.tiles[wid % p.n_tiles];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int head = g * G + (wave % G);
  const int tg = wave / G;
  const int qrow = tg * kQRows + l32;              // offset from tile.q0
  const bool row_ok = qrow < tile.nq;
  const int64_t tok = (int64_t)tile.q0 + qrow;

  // Q fragments: B operand, lane holds query row l32, dims ks*16 + hi*8 .. +7
  bf16x8_t qf[8];
  {
    const uint16_t* qp = p.q + tok * p.q_stride + head * kHeadDim + hi * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = bitcast<bf16x8_t>(u);
    }
  }
  const int seg_lo = row_ok ? p.seg_lo[tok] : 0x7FFFFFFF;
  const int self_q = tile.self_qbase + qrow;       // self-key index of this query

  KVSrc cs{}, cs2{}, ss{};
  int n_c1 = 0, n_ct = 0, n_st = 0;
  if (tile.cross >= 0) { cs = p.srcs[tile.cross]; n_c1 = (cs.len + kKeyTile - 1) / kKeyTile; }
  n_ct = n_c1;
  if (tile.cross2 >= 0) { cs2 = p.srcs[tile.cross2]; n_ct += (cs2.len + kKeyTile - 1) / kKeyTile; }
  if (tile.self >= 0) {
    ss = p.srcs[tile.self];
    const int self_end = tile.self_qbase + tile.nq;
    n_st = (self_end - tile.self_k0 + kKeyTile - 1) / kKeyTile;
    if (n_st < 0) n_st = 0;
  }
  const int n_tiles = n_ct + n_st;

  auto view = [&](int it) {
    TileView t;
    // the source's fields, chosen among register values (in_sreg)
    const bool a = it < n_c1, b = it < n_ct;
    const int fp8 = a ? in_sreg(cs.fp8) : (b ? in_sreg(cs2.fp8) : in_sreg(ss.fp8));
    const int64_t hs = a ? in_sreg(cs.head_stride) : (b ? in_sreg(cs2.head_stride) : in_sreg(ss.head_stride));
    const int64_t ts = a ? in_sreg(cs.tok_stride) : (b ? in_sreg(cs2.tok_stride) : in_sreg(ss.tok_stride));
    const void* kp = a ? in_sreg(cs.k) : (b ? in_sreg(cs2.k) : in_sreg(ss.k));
    const void* vp = a ? in_sreg(cs.v) : (b ? in_sreg(cs2.v) : in_sreg(ss.v));
    const int esz = fp8 ? 1 : 2;
    t.k = reinterpret_cast<const uint8_t*>(kp) + (int64_t)g * hs * esz;
    t.v = reinterpret_cast<const uint8_t*>(vp) + (int64_t)g * hs * esz;
    t.tok_bytes = ts * esz;
    t.kbase = a ? it * kKeyTile : (b ? (it - n_c1) * kKeyTile : tile.self_k0 + (it - n_ct) * kKeyTile);
    t.len = a ? in_sreg(cs.len) : (b ? in_sreg(cs2.len) : in_sreg(ss.len));
    t.fp8 = fp8;
    return t;
  };

  f32x16_t o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;

  TileRegs<NT> regs;
  if (n_tiles > 0) load_tile<NT>(regs, view(0), tid);

  for (int it = 0; it < n_tiles; ++it) {
    const bool is_cross = it < n_ct;
    const int fp8 = is_cross ? in_sreg(cs.fp8) : in_sreg(ss.fp8);   // both cross levels: slabs of one format
    const int kbase = it < n_c1 ? it * kKeyTile
                                : (is_cross ? (it - n_c1) * kKeyTile : tile.self_k0 + (it - n_ct) * kKeyTile);
    const int clen = it < n_c1 ? in_sreg(cs.len) : in_sreg(cs2.len);
    __syncthreads();
    store_tile<NT>(regs, fp8, p.k_scale, p.v_scale, Ks, Vt, tid);
    __syncthreads();
    if (it + 1 < n_tiles) load_tile<NT>(regs, view(it + 1), tid);

    // S^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      const uint16_t* kp = Ks + (kb * 32 + l32) * KSTR + hi * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8_t a = bitcast<bf16x8_t>(*reinterpret_cast<const uint4*>(kp + ks * 16));
        s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
      }
    }
    // Mask (key of (kb, r) = kbase + kb*32 + (r/4)*8 + hi*4 + r%4), then the
    // row max of this tile over both lanes of the row (scores are raw here;
    // the softmax scale is folded into the exponent below).
    const bool need_mask = is_cross ? (kbase + kKeyTile > clen) : true;
    if (need_mask) {
      const int lo = is_cross ? 0 : seg_lo;
      const int hi_k = is_cross ? clen - 1 : self_q;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          s[kb][r] = (key >= lo && key <= hi_k) ? s[kb][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * p.scale_log2;
    // Lazy rescale: the running reference m_run moves only when a row's max
    // exceeds it by more than 8 (log2 units), so P stays below 2^8 and the
    // O accumulator is rescaled only on those (rare, wave-uniform) tiles.
    // The final O / l and the LSE are exact for any reference.
    if (__ballot(mt > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first visible tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;

    // P (bf16) as the B operand: k-step (kb, sp) takes regs 8*sp .. 8*sp+7
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][sp * 8 + 2 * e], p.scale_log2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][sp * 8 + 2 * e + 1], p.scale_log2, -m_use));
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[kb][sp] = bitcast<bf16x8_t>(make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    // O^T += V^T . P^T ; A lane: dim row cb*32 + l32, keys kb*32 + sp*16 + hi*4 + {0..3, 8..11}
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint16_t* vp = Vt + (cb * 32 + l32) * VSTR + hi * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vp + kb * 32 + sp * 16);
          const uint2 hi2 = *reinterpret_cast<const uint2*>(vp + kb * 32 + sp * 16 + 8);
          bf16x8_t a = bitcast<bf16x8_t>(make_uint4(lo.x, lo.y, hi2.x, hi2.y));
          o[cb] = mfma_32x32x16(a, pb[kb][sp], o[cb]);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* op = p.out + tok * p.o_stride + head * kHeadDim + hi * 4;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      uint2 w;
      w.x = pack_bf16x2(o[cb][rg * 4 + 0] * inv, o[cb][rg * 4 + 1] * inv);
      w.y = pack_bf16x2(o[cb][rg * 4 + 2] * inv, o[cb][rg * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + cb * 32 + rg * 8) = w;
    }
  }
  if (p.lse != nullptr && hi == 0) {
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    const float L = l_tot > 0.0f ? (m_use + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    p.lse[tok * p.hq + head] = L;
  }
}

// ----------------------------------------------------------------------------
// Kernel with direct HBM->LDS copies; K/V tiles in bf16 or as E4M3 codes.
//
// K and V tiles are copied from HBM straight into LDS by global_load_lds
// (16 B per lane, no staging registers; issued as inline asm so the compiler
// does not make the operand reads wait for copies in flight). bf16 rows are
// 256 B, E4M3 rows 128 B (decoded to bf16 after each LDS read, exactly:
// every E4M3 value is a bf16 value); each row's 16-B chunks are XOR-swizzled
// so that the MFMA operand reads are free of bank conflicts on gfx950's
// 64-bank LDS. V stays in its natural [key][dim] layout and the transposed A
// operand of O^T += V^T P^T comes from the LDS transpose reads:
//   ds_read_tr16_b64: within a 16-lane block, pointing lane s at
//     V[K0 + s/4][D0 + 4(s%4)] hands lane j the keys K0..K0+3 of dim D0 + j;
//   ds_read_tr8_b64: pointing lane s at V[K0 + s/2][D0 + 8(s%2)] hands lane j
//     the keys K0..K0+7 of dim D0 + j.
// Key order inside a 32-key half: S^T row r holds key pi(r), pi swapping bits
// 2 and 3, so that the P values a lane holds for one MFMA k-step are 8
// consecutive keys (what one tr8 read, or two tr16 reads, deliver for V^T).
// Dim order of the S^T k-steps: k-step 2t+u, lane half hi, slot e holds dim
// 32t + 16hi + 8u + e, so one 16-B read of an E4M3 K row serves two k-steps.
// ----------------------------------------------------------------------------
constexpr int kRowElems = kHeadDim;                 // 128 bf16 = 256 B per key row
constexpr int kTileElems = kKeyTile * kRowElems;    // 8192 bf16 = 16 KB

// LDS serves 64 banks x 4 B per cycle: 16 lanes of a 16-B read, 32 lanes of
// an 8-B read.
// bf16 K (16 chunks per row): the 16 rows one ds_read_b128 cycle touches
// (same chunk) land on 16 distinct chunks. bf16 V: one tr16 cycle reads 4
// consecutive rows x 64 B; shifting each row's chunks by 4*(row % 4) puts the
// four rows on disjoint 64-B bank groups.
__device__ __forceinline__ int swz_k(int key, int chunk) { return chunk ^ (key & 15); }
__device__ __forceinline__ int swz_v(int key, int chunk) { return chunk ^ ((key & 3) << 2); }
// E4M3 K (8 chunks per 128-B row, two rows per 256-B bank cycle): the 16
// rows of a cycle pair up by parity and (row / 2) % 8 spreads each parity
// over the 8 chunk positions. E4M3 V: one tr8 cycle reads 8 consecutive rows
// x two 16-B chunks; (row / 2) % 4 moves the same-parity rows onto disjoint
// chunk pairs.
__device__ __forceinline__ int swz8_k(int key, int chunk) { return chunk ^ ((key >> 1) & 7); }
__device__ __forceinline__ int swz8_v(int key, int chunk) { return chunk ^ (((key >> 1) & 3) << 1); }

// S^T row -> key offset inside a 32-key half (and back: pi is an involution)
__device__ __forceinline__ int key_pi(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i16_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16_t __attribute__((address_space(3)))*)(__attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ v2i32_t lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (v2i32_t __attribute__((address_space(3)))*)(__attribute__((address_space(3))) char*)p);
}

// 8 E4M3 codes (two words) -> 8 bf16, exact
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bitcast<bf16x8_t>(make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)));
}

// The direct copies of one 64-key K (IS_V = false) or V tile of kv head g into
// the LDS slot at byte address `dst`, by wave `wave` of NW: 1-KB slices of 4
// bf16 rows or 8 E4M3 rows; lane L writes 16-B slot L % (16 or 8) of its row
// and reads the chunk the swizzle puts there. Rows at or past the source
// length are clamped to its last row (their scores are masked); full tiles
// skip the clamp. Per-lane offsets are 24-bit products (token strides are
// bounded on the host).
template <int NW, bool IS_V, int ROWS = kKeyTile, bool NT = false>
struct TileCopy {
  const uint8_t* b8;
  uint32_t tb, last, dst;
  bool full, fp8;
  __device__ __forceinline__ TileCopy(const KVSrc& src, int g, int kbase, uint32_t dst_) {
    fp8 = uniform(src.fp8) != 0;
    const int sh = fp8 ? 0 : 1;                  // log2 of the element size
    tb = (uint32_t)src.tok_stride << sh;
    const int64_t base = ((int64_t)g * src.head_stride + (int64_t)kbase * src.tok_stride) << sh;
    b8 = reinterpret_cast<const uint8_t*>(IS_V ? src.v : src.k) + base;
    full = kbase + ROWS <= src.len;
    last = (uint32_t)max(src.len - 1 - kbase, 0);
    dst = dst_;
  }
  __device__ __forceinline__ void issue_all(int wave, int lane) const {
    // every wave copies at least one 1-KB slice (E4M3 tiles have 32 or 64
    // keys; the 16-key quarter tiles are bf16 only)
    static_assert(ROWS / 4 / NW >= 1 && (ROWS < 32 || ROWS / 8 / NW >= 1), "copy split");
    if (!fp8) {
      constexpr int PER = ROWS / 4 / NW;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int slice = wave * PER + i;
        const uint32_t row = slice * 4 + (lane >> 4);
        const uint32_t off = (IS_V ? swz_v(row, lane & 15) : swz_k(row, lane & 15)) * 16;
        const uint32_t r = full ? row : min(row, last);
        if (NT) copy16_to_lds_off_nt(b8, __umul24(r, tb) + off, dst + slice * 1024);
        else copy16_to_lds_off(b8, __umul24(r, tb) + off, dst + slice * 1024);
      }
    } else {
      constexpr int PER = ROWS / 8 / NW;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int slice = wave * PER + i;
        const uint32_t row = slice * 8 + (lane >> 3);
        const uint32_t off = (IS_V ? swz8_v(row, lane & 7) : swz8_k(row, lane & 7)) * 16;
        const uint32_t r = full ? row : min(row, last);
        if (NT) copy16_to_lds_off_nt(b8, __umul24(r, tb) + off, dst + slice * 1024);
        else copy16_to_lds_off(b8, __umul24(r, tb) + off, dst + slice * 1024);
      }
    }
  }
};

// The same copies for the full tiles of one source whose element format is
// known at compile time: a lane's source offsets depend only on its slice,
// the token stride and the swizzle, so they are formed once per workgroup
// and each tile adds only its (wave-uniform) base.
template <int NW, bool IS_V, int ROWS, bool NT, bool FP8>
struct FullTileCopy {
  static constexpr int PER = FP8 ? ROWS / 8 / NW : ROWS / 4 / NW;
  uint32_t voff[PER];
  __device__ __forceinline__ FullTileCopy(const KVSrc& src, int wave, int lane) {
    static_assert(PER >= 1, "copy split");
    const uint32_t tb = (uint32_t)src.tok_stride << (FP8 ? 0 : 1);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slice = wave * PER + i;
      const uint32_t row = FP8 ? slice * 8 + (lane >> 3) : slice * 4 + (lane >> 4);
      const uint32_t off = FP8 ? (IS_V ? swz8_v(row, lane & 7) : swz8_k(row, lane & 7)) * 16
                               : (IS_V ? swz_v(row, lane & 15) : swz_k(row, lane & 15)) * 16;
      voff[i] = __umul24(row, tb) + off;
    }
  }
  // the tile of kv head g starting at key kbase into the slot at dst
  __device__ __forceinline__ void issue(const KVSrc& src, int g, int kbase, uint32_t dst, int wave) const {
    const int64_t base = ((int64_t)g * src.head_stride + (int64_t)kbase * src.tok_stride) << (FP8 ? 0 : 1);
    const uint8_t* b8 = reinterpret_cast<const uint8_t*>(IS_V ? src.v : src.k) + base;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (NT) copy16_to_lds_off_nt(b8, voff[i], dst + (wave * PER + i) * 1024);
      else copy16_to_lds_off(b8, voff[i], dst + (wave * PER + i) * 1024);
    }
  }
};

template <bool B>
struct MaskTag { static constexpr bool value = B; };

// The key tiles one workgroup visits: first the cross tiles of its anchor
// source (the last one ragged), then those of the second cross source (a
// shared suffix prefix; its last tile ragged), then the self tiles from
// self_k0 up to its last query. Tiles j >= n_full need masking. kbase is the
// tile's first key within its own source.
// TKC / TKS: keys per cross / self tile (64, or 32 for the half tiles of
// packed launches). L2: launches with a second cross level; without it the
// tile -> source selects stay two-way (they sit in the copy and mask paths of
// every step).
template <int TKC = kKeyTile, int TKS = kKeyTile, bool L2 = false>
struct TileSeq {
  KVSrc cs{}, cs2{}, ss{};
  int n_c1 = 0, n_ct = 0, n_st = 0, n_full = 0, n_tiles = 0, self_k0 = 0;
  __device__ __forceinline__ TileSeq(const AttnParams& p, const AttnTile& tile) {
    if (tile.cross >= 0) {
      cs = p.srcs[tile.cross];
      n_c1 = (cs.len + TKC - 1) / TKC;
      n_full = cs.len / TKC;
    }
    n_ct = n_c1;
    if (L2 && tile.cross2 >= 0) {
      cs2 = p.srcs[tile.cross2];
      n_ct += (cs2.len + TKC - 1) / TKC;
      if (n_full == n_c1) n_full += cs2.len / TKC;   // the first level ends on a tile boundary
    }
    if (tile.self >= 0) {
      ss = p.srcs[tile.self];
      n_st = max(0, (tile.self_qbase + tile.nq - tile.self_k0 + TKS - 1) / TKS);
    }
    n_tiles = n_ct + n_st;
    self_k0 = tile.self_k0;
  }
  // by value, field by field, choosing among register values (in_sreg)
  __device__ __forceinline__ KVSrc src(int j) const {
    if constexpr (!L2) {
      return j < n_ct ? cs : ss;
    } else {
      const bool a = j < n_c1, b = j < n_ct;
      KVSrc r;
      r.k = a ? in_sreg(cs.k) : (b ? in_sreg(cs2.k) : in_sreg(ss.k));
      r.v = a ? in_sreg(cs.v) : (b ? in_sreg(cs2.v) : in_sreg(ss.v));
      r.tok_stride = a ? in_sreg(cs.tok_stride) : (b ? in_sreg(cs2.tok_stride) : in_sreg(ss.tok_stride));
      r.head_stride = a ? in_sreg(cs.head_stride) : (b ? in_sreg(cs2.head_stride) : in_sreg(ss.head_stride));
      r.len = a ? in_sreg(cs.len) : (b ? in_sreg(cs2.len) : in_sreg(ss.len));
      r.fp8 = a ? in_sreg(cs.fp8) : (b ? in_sreg(cs2.fp8) : in_sreg(ss.fp8));
      return r;
    }
  }
  __device__ __forceinline__ int kbase(int j) const {
    if constexpr (!L2) return j < n_ct ? j * TKC : self_k0 + (j - n_ct) * TKS;
    else return j < n_c1 ? j * TKC : (j < n_ct ? (j - n_c1) * TKC : self_k0 + (j - n_ct) * TKS);
  }
  // valid keys of a cross tile's source
  __device__ __forceinline__ int clen(int j) const {
    if constexpr (!L2) return cs.len;
    else return j < n_c1 ? in_sreg(cs.len) : in_sreg(cs2.len);
  }
};

// One wave's share of the bf16 MFMA attention: 32 query rows of one head
// (lane % 32 owns row l32; the two lanes of a row split its keys), the O^T
// accumulator and the online-softmax state. Operand offsets into the LDS
// tiles are formed where used (a few VALU ops next to the MFMAs) rather than
// kept in registers across the loop.
struct WaveAttn {
  bf16x8_t qf[8];       // Q as the B operand of k-step 2t+u: dims 32t + 16hi + 8u .. +7
  f32x16_t o[4];
  float m_run, l_run, scale_log2;
  int lane, hi, lo_self, hi_self;

  __device__ __forceinline__ void init(const AttnParams& p, const AttnTile& tile, int64_t tok,
                                       bool row_ok, int qrow, int head, int lane_) {
    lane = lane_;
    hi = lane >> 5;
    const uint16_t* qp = p.q + tok * p.q_stride + head * kHeadDim + hi * 16;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int d = 32 * (ks >> 1) + 8 * (ks & 1);
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + d) : make_uint4(0, 0, 0, 0);
      qf[ks] = bitcast<bf16x8_t>(u);
    }
    // self keys visible to this row: [first key of its segment, its own key]
    lo_self = row_ok ? p.seg_lo[tok] : 0;
    hi_self = row_ok ? tile.self_qbase + qrow : -1;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
    // running reference of the online softmax (log2 units); finite start:
    // the first visible score always triggers a rescale (alpha = 0), and
    // rows with no visible key keep P = 0
    m_run = -1e30f;
    l_run = 0.0f;
    scale_log2 = p.scale_log2;
    // Make the Q and segment loads complete here, visibly to the compiler:
    // otherwise its wait-count pass, which does not see the inline-asm tile
    // copies, keeps these loads pending into the tile loop and waits for
    // vmcnt(0) before the first MFMA of every step -- which also waits for
    // the tile copies just issued and undoes the prefetch.
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
    asm volatile("" ::"v"(lo_self));
  }

  // S^T = K . Q^T of the tile at Kt (two 32-key halves); lane l32 reads key
  // row pi(l32) of each half
  // NK: keys in the tile's slot (64, 32 or 16). Below 64 only the first
  // 32-key half is computed and the second half's scores are -inf (no key);
  // with 16, rows 16..31 of that half read past the slot (inside this
  // workgroup's LDS) and are masked by the caller (mask with the same NK).
  template <bool FP8, int NK = kKeyTile>
  __device__ __forceinline__ void scores(const uint16_t* Kt, f32x16_t (&s)[2]) const {
    constexpr bool HALF = NK < kKeyTile;
    const int krow = key_pi(lane & 31);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = (HALF && kb == 1) ? -INFINITY : 0.0f;
    if constexpr (!FP8) {
#pragma unroll
      for (int kb = 0; kb < (HALF ? 1 : 2); ++kb) {
        const int row = kb * 32 + krow;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int chunk = 4 * (ks >> 1) + 2 * hi + (ks & 1);
          const bf16x8_t a = bitcast<bf16x8_t>(
              *reinterpret_cast<const uint4*>(Kt + row * kRowElems + swz_k(row, chunk) * 8));
          s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
        }
      }
    } else {
      const uint8_t* K8 = reinterpret_cast<const uint8_t*>(Kt);
#pragma unroll
      for (int kb = 0; kb < (HALF ? 1 : 2); ++kb) {
        const int row = kb * 32 + krow;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 c = *reinterpret_cast<const uint4*>(K8 + row * 128 + swz8_k(row, 2 * t + hi) * 16);
          s[kb] = mfma_32x32x16(e4m3x8_to_bf16x8(c.x, c.y), qf[2 * t], s[kb]);
          s[kb] = mfma_32x32x16(e4m3x8_to_bf16x8(c.z, c.w), qf[2 * t + 1], s[kb]);
        }
      }
    }
  }

  // mask a tile starting at key kbase: visible keys are [0, cross_len) for a
  // cross tile, [lo_self, hi_self] for a self tile -- never past the tile's
  // NK keys when a self tile has NK = 16; register i of half kb holds key
  // kbase + kb*32 + 16*(i/8) + 8*hi + i%8 (unsigned range test)
  // A row's range is empty (hk < lo) when a 16-key self tile lies wholly
  // before the row's segment (packed tiles of several waves span more than
  // one such tile); the unsigned test alone would wrap there.
  template <int NKS = kKeyTile>
  __device__ __forceinline__ void mask(f32x16_t (&s)[2], int kbase, bool cross, int cross_len) const {
    const int lo = cross ? 0 : lo_self;
    const int hk = cross ? cross_len - 1 : (NKS < 32 ? min(hi_self, kbase + NKS - 1) : hi_self);
    const bool any = hk >= lo;
    const uint32_t range = (uint32_t)(hk - lo);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t x = (uint32_t)(kbase + kb * 32 + hi * 8 - lo);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t c = (uint32_t)(16 * (r >> 3) + (r & 7));
        s[kb][r] = (any && x + c <= range) ? s[kb][r] : -INFINITY;
      }
    }
  }

  // row max of a tile over both lanes of the row, log2 units
  __device__ __forceinline__ float row_max(const f32x16_t (&s)[2]) const {
    // max(m, a, b) per register pair: one v_max3_f32 each
    float m0 = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) m0 = fmaxf(fmaxf(m0, s[0][r]), s[1][r]);
    return xor32_max(m0) * scale_log2;
  }

  // Lazy rescale: the running reference moves only when a row's max exceeds
  // it by more than 8 (log2 units), so P stays below 2^8 and O is rescaled
  // only on those (rare, wave-uniform) occasions. O / l and the LSE are exact
  // for any reference.
  __device__ __forceinline__ void rescale(float mt) {
    if (__ballot(mt > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
    }
  }

  // P = 2^(s*scale - m_run) in bf16 as the B operand: k-step (kb, sp) takes
  // regs 8*sp .. 8*sp+7 of half kb, i.e. keys kb*32 + 16sp + 8hi + 0..7; the
  // row sum adds the fp32 values
  // NK < 64: the second half's scores are -inf and its P is never read (pv
  // with the same NK skips it), so it is not computed
  template <int NK = kKeyTile>
  __device__ __forceinline__ void probs(const f32x16_t (&s)[2], bf16x8_t (&pb)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < (NK < kKeyTile ? 1 : 2); ++kb)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][sp * 8 + 2 * e], scale_log2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][sp * 8 + 2 * e + 1], scale_log2, -m_run));
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[kb][sp] = bitcast<bf16x8_t>(make_uint4(w[0], w[1], w[2], w[3]));
      }
  }

  // O^T += V^T . P^T with the tile at Vt; A lane: dim row cb*32 + l32, keys
  // kb*32 + 16sp + 8hi + 0..7. The 16-lane block (lane / 16) covers dims
  // cb*32 + 16*(block % 2) .. +15 and keys +8 for blocks 2, 3.
  // NK: keys in the slot (64, 32 or 16); only their P is used
  template <bool FP8, int NK = kKeyTile>
  __device__ __forceinline__ void pv(const uint16_t* Vt, const bf16x8_t (&pb)[2][2]) {
    constexpr bool HALF = NK < kKeyTile;
    constexpr int NSP = NK < 32 ? 1 : 2;       // 16-key k-steps per 32-key half
    const int s16 = lane & 15;
    const int dhalf = (lane >> 4) & 1;
    if constexpr (!FP8) {
      // two tr16 reads: keys +0..3 and +4..7; lane s16 points at key
      // s16 / 4 of the group and dims 4*(s16 % 4) .. +3 of the 16-dim half
      const int key0 = hi * 8 + (s16 >> 2);
#pragma unroll
      for (int kb = 0; kb < (HALF ? 1 : 2); ++kb)
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int key = kb * 32 + sp * 16 + key0;
            const int d0 = cb * 32 + 16 * dhalf + 4 * (s16 & 3);
            const uint16_t* vp = Vt + key * kRowElems + swz_v(key, d0 >> 3) * 8 + (d0 & 7);
            const uint2 a_lo = __builtin_bit_cast(uint2, lds_read_tr16(vp));
            const uint2 a_hi = __builtin_bit_cast(uint2, lds_read_tr16(vp + 4 * kRowElems));
            o[cb] = mfma_32x32x16(bitcast<bf16x8_t>(make_uint4(a_lo.x, a_lo.y, a_hi.x, a_hi.y)),
                                  pb[kb][sp], o[cb]);
          }
    } else {
      // one tr8 read: lane s16 points at key s16 / 2 of the 8-key group and
      // dims 8*(s16 % 2) .. +7 of the 16-dim half
      const uint8_t* V8 = reinterpret_cast<const uint8_t*>(Vt);
      const int key0 = hi * 8 + (s16 >> 1);
#pragma unroll
      for (int kb = 0; kb < (HALF ? 1 : 2); ++kb)
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int key = kb * 32 + sp * 16 + key0;
            const uint8_t* vp = V8 + key * 128 + swz8_v(key, 2 * cb + dhalf) * 16 + 8 * (s16 & 1);
            const v2i32_t c = lds_read_tr8(vp);
            o[cb] = mfma_32x32x16(e4m3x8_to_bf16x8((uint32_t)c.x, (uint32_t)c.y), pb[kb][sp], o[cb]);
          }
    }
  }

  // O / l as bf16 and the natural-log LSE (-inf without a visible key)
  __device__ __forceinline__ void store(const AttnParams& p, int64_t tok, bool row_ok, int head) const {
    const float l_tot = xor32_sum(l_run);
    if (!row_ok) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* op = p.out + tok * p.o_stride + head * kHeadDim + hi * 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        uint2 w;
        w.x = pack_bf16x2(o[cb][rg * 4 + 0] * inv, o[cb][rg * 4 + 1] * inv);
        w.y = pack_bf16x2(o[cb][rg * 4 + 2] * inv, o[cb][rg * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + cb * 32 + rg * 8) = w;
      }
    if (p.lse != nullptr && hi == 0) {
      const float L = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      p.lse[tok * p.hq + head] = L;
    }
  }
};

// rows of a tile with no visible key at all: zero output, LSE -inf
__device__ __forceinline__ void store_empty(const AttnParams& p, int64_t tok, bool row_ok, int head, int hi) {
  if (!row_ok) return;
  uint16_t* op = p.out + tok * p.o_stride + head * kHeadDim + hi * 4;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) *reinterpret_cast<uint2*>(op + cb * 32 + rg * 8) = make_uint2(0, 0);
  if (p.lse != nullptr && hi == 0) p.lse[tok * p.hq + head] = -INFINITY;
}

// Every barrier that publishes copied tiles: the copies are inline asm,
// invisible to the compiler's wait-count tracking, and a workgroup barrier's
// fence does not wait for them, so the issuing wave waits for all of its
// copies in flight first.
__device__ __forceinline__ void publish() {
  wait_vmcnt<0>();
  __syncthreads();
}
// Same, leaving this wave's N most recent copies in flight (copies complete
// in issue order for the wait count).
template <int N>
__device__ __forceinline__ void publish_keep() {
  wait_vmcnt<N>();
  __syncthreads();
}

// Software pipeline over the key tiles: while the softmax of tile j (exp,
// bf16 packing, row sums) runs on the VALU, the S MFMAs of tile j+1 are in
// flight, and the PV MFMAs of tile j overlap the masking and row max of tile
// j+1. K has two LDS slots and V three; at step j the copies of K(j+2) and
// V(j+2) are issued into the slots that step j-1 finished reading, so one
// barrier per tile suffices, and both K and V copies have two steps to land
// (with two workgroups per CU, 2 x 80 KB fill the 160-KB LDS). The step is instantiated per tile format (FC:
// cross tiles are E4M3 codes, FS: self tiles are) and per masking need, so
// that no MFMA accumulator crosses a runtime branch: full cross tiles, the
// remaining (ragged) cross tiles, the cross -> self transition, self tiles.
// One workgroup: the G query heads of one kv head x (waves / G) groups of 32
// query tokens, all sharing every K/V tile copied into LDS. PACK > 0
// (launches whose anchors have few query tokens, where K/V streaming is the
// work): PACK waves, each of whose 32 rows are the G heads x 32/G tokens of
// its share of the tile (wave w holds tokens w*32/G .. (w+1)*32/G - 1), so
// that every K/V tile feeds rows that exist instead of 32 per head.
template <int G, bool FC, bool FS, int PACK, bool L2>
__global__ void __launch_bounds__(PACK ? 64 * PACK : 64 * (G >= 4 ? G : 4), 2)
attn_direct_kernel(AttnParams p) {
  constexpr int NW = PACK ? PACK : (G >= 4 ? G : 4);
  // Packed launches use 8-KB slots, 40 KB per workgroup, four workgroups per
  // CU: an E4M3 tile of 64 keys is 8 KB, and bf16 tiles are half tiles of 32
  // keys, whose second 32-key half of the scores is -inf. With E4M3 cross
  // and bf16 self tiles and G >= 2 (SMALL: a packed tile's queries, hence
  // its self keys, number at most 32/G <= 16), slots are 4 KB -- E4M3 half
  // tiles of 32 keys, bf16 quarter tiles of 16 keys -- 20 KB per workgroup,
  // eight workgroups (two waves per SIMD) per CU.
  constexpr bool SMALL = PACK && FC && !FS && G >= 2;
  constexpr int NKC = PACK && (SMALL || !FC) ? kKeyTile / 2 : kKeyTile;          // keys per cross tile
  constexpr int NKS = PACK && !FS ? (SMALL ? kKeyTile / 4 : kKeyTile / 2) : kKeyTile;   // per self tile
  constexpr uint32_t kSlotBytes = PACK ? (SMALL ? 4096 : 8192) : kTileElems * 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[5 * kSlotBytes];   // K: 2 slots, V: 3
  auto kslot = [&](int i) __attribute__((always_inline)) { return reinterpret_cast<const uint16_t*>(lds_raw + i * kSlotBytes); };
  auto vslot = [&](int i) __attribute__((always_inline)) { return reinterpret_cast<const uint16_t*>(lds_raw + (2 + i) * kSlotBytes); };

  const int64_t total = (int64_t)p.n_tiles * p.hkv;
  const int64_t wid = xcd_remap(blockIdx.x, total);
  if (wid < 0) return;
  const int g = (int)(wid / p.n_tiles);
  const AttnTile tile = p.tiles[wid % p.n_tiles];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int head = PACK ? g * G + (lane & 31) / (kQRows / G) : g * G + (wave % G);
  const int qrow = PACK ? wave * (kQRows / G) + (lane & 31) % (kQRows / G) : (wave / G) * kQRows + (lane & 31);
  const bool row_ok = qrow < tile.nq;
  const int64_t tok = (int64_t)tile.q0 + qrow;

  const TileSeq<NKC, NKS, L2> ts(p, tile);
  if (ts.n_tiles == 0) {
    store_empty(p, tok, row_ok, head, lane >> 5);
    return;
  }
  const uint32_t lds_k0 = lds_addr_of(lds_raw);
  const uint32_t lds_v0 = lds_k0 + 2 * kSlotBytes;
  // K and V copies of tile j into K slot ks and V slot vs
  // (packed launches stream each anchor's K/V once per kv head: non-temporal)
  // full tiles of the first cross source (the anchor) take the copies with
  // offsets formed here; the rest (ragged, second-level and self tiles) the
  // general ones
  const FullTileCopy<NW, false, NKC, (PACK > 0), FC> kfull(ts.cs, wave, lane);
  const FullTileCopy<NW, true, NKC, (PACK > 0), FC> vfull(ts.cs, wave, lane);
  // (one-level launches: the two-level variants have no registers to spare)
  const int n_fast = L2 ? 0 : min(ts.n_full, ts.n_c1);
  auto issue = [&](int j, int ks, int vs) __attribute__((always_inline)) {
    if (j < n_fast) {
      kfull.issue(ts.cs, g, j * NKC, lds_k0 + ks * kSlotBytes, wave);
      vfull.issue(ts.cs, g, j * NKC, lds_v0 + vs * kSlotBytes, wave);
    } else if (NKC == NKS || j < ts.n_ct) {
      TileCopy<NW, false, NKC, (PACK > 0)>(ts.src(j), g, ts.kbase(j), lds_k0 + ks * kSlotBytes).issue_all(wave, lane);
      TileCopy<NW, true, NKC, (PACK > 0)>(ts.src(j), g, ts.kbase(j), lds_v0 + vs * kSlotBytes).issue_all(wave, lane);
    } else {
      TileCopy<NW, false, NKS, (PACK > 0)>(ts.src(j), g, ts.kbase(j), lds_k0 + ks * kSlotBytes).issue_all(wave, lane);
      TileCopy<NW, true, NKS, (PACK > 0)>(ts.src(j), g, ts.kbase(j), lds_v0 + vs * kSlotBytes).issue_all(wave, lane);
    }
  };
  issue(0, 0, 0);
  if (ts.n_tiles > 1) issue(1, 1, 1);

  WaveAttn w;
  w.init(p, tile, tok, row_ok, qrow, head, lane);

  // prologue: scores of tile 0
  f32x16_t s_cur[2];
  publish();
  if (ts.n_ct > 0) w.scores<FC, NKC>(kslot(0), s_cur);
  else w.scores<FS, NKS>(kslot(0), s_cur);
  if (ts.n_full == 0) w.mask<NKS>(s_cur, ts.kbase(0), 0 < ts.n_ct, ts.clen(0));
  w.rescale(w.row_max(s_cur));

  // step j: issue K(j+2), V(j+2); S(j+1) with P(j); PV(j) with mask/max of
  // j+1. PV_SELF / S_SELF: tiles j and j+1 are self tiles (format FS, else
  // FC). vs: V slot of tile j (j mod 3, kept as a rotating counter).
  int vs = 0;
  auto step = [&](int j, auto pv_tag, auto s_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool PV_SELF = decltype(pv_tag)::value;
    constexpr bool S_SELF = decltype(s_tag)::value;
    constexpr bool MASK_NEXT = decltype(mask_tag)::value;
    constexpr bool PV_FP8 = PV_SELF ? FS : FC, S_FP8 = S_SELF ? FS : FC;
    constexpr int PV_NK = PV_SELF ? NKS : NKC, S_NK = S_SELF ? NKS : NKC;
    // copies (1 KB each) per wave of one V tile of tile j+1's format and size
    constexpr int NV_NEXT = S_NK * (S_FP8 ? 128 : 256) / 1024 / NW;
    // waits for this wave's copies of K(j+1) and V(j) -- the copies of
    // V(j+1), issued last (by step j-1 or the prologue), may stay in flight;
    // the barrier then makes every wave's copies visible and guarantees that
    // step j-1 (which read K(j) and V(j-1)) is finished everywhere
    publish_keep<NV_NEXT>();
    if (j + 2 < ts.n_tiles) issue(j + 2, j & 1, vs == 0 ? 2 : vs - 1);   // V slot (j + 2) mod 3
    bf16x8_t pb[2][2];
    w.probs<PV_NK>(s_cur, pb);
    f32x16_t s_nxt[2];
    w.scores<S_FP8, S_NK>(kslot((j + 1) & 1), s_nxt);
    w.pv<PV_FP8, PV_NK>(vslot(vs), pb);
    vs = vs == 2 ? 0 : vs + 1;
    if constexpr (MASK_NEXT) w.mask<NKS>(s_nxt, ts.kbase(j + 1), j + 1 < ts.n_ct, ts.clen(j + 1));
    w.rescale(w.row_max(s_nxt));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
  };
  using Cross = MaskTag<false>;
  using Self = MaskTag<true>;
  int j = 0;
  for (; j + 1 < ts.n_full; ++j) step(j, Cross{}, Cross{}, MaskTag<false>{});
  for (; j + 1 < ts.n_ct; ++j) step(j, Cross{}, Cross{}, MaskTag<true>{});
  if (j + 1 < ts.n_tiles && j < ts.n_ct) {
    step(j, Cross{}, Self{}, MaskTag<true>{});
    ++j;
  }
  for (; j + 1 < ts.n_tiles; ++j) step(j, Self{}, Self{}, MaskTag<true>{});
  // epilogue: the last tile's PV (its V copy was issued by the last step, or
  // by the prologue)
  {
    publish();
    bf16x8_t pb[2][2];
    w.probs<(NKC > NKS ? NKC : NKS)>(s_cur, pb);   // a -inf half only adds zeros
    if (j < ts.n_ct) w.pv<FC, NKC>(vslot(vs), pb);
    else w.pv<FS, NKS>(vslot(vs), pb);
  }
  w.store(p, tok, row_ok, head);
}

// query tokens per tile: unpacked (pack 0; both the direct and the
// register-staged kernel), max(G, 4) waves of G heads x (waves / G) groups of
// 32 tokens; packed, `pack` waves of G heads x 32/G tokens
int attn_tile_tokens(int group, int pack) {
  return pack ? pack * (kQRows / group) : kQRows * (group >= 4 ? group : 4) / group;
}

// the packed width for launches whose runs of queries sharing an anchor have
// at most max_run tokens: the fewest waves (1, 2 or 4) whose rows hold them,
// or 0 (unpacked tiles) when more than four waves' worth, or when the
// unpacked tile has no more tokens than that packed one
int attn_pack_waves(int group, int max_run) {
  for (int w = 1; w <= 4; w *= 2)
    if (max_run <= w * (kQRows / group)) return w * (kQRows / group) < attn_tile_tokens(group, 0) ? w : 0;
  return 0;
}

bool attn_direct_ok(bool fp8_cross, bool fp8_self, float k_scale, float v_scale) {
  // E4M3 sources with unit scales are read by the direct kernel (decoded after
  // each LDS read); other scales take the register-staged kernel, which
  // applies them while staging
  return !(fp8_cross || fp8_self) || (k_scale == 1.0f && v_scale == 1.0f);
}

template <bool FC, bool FS, int PACK, bool L2>
static hipError_t launch_direct(const AttnParams& p, int group, dim3 gr, hipStream_t s) {
  const dim3 blk(PACK ? 64 * PACK : 256);
  switch (group) {
    case 1: attn_direct_kernel<1, FC, FS, PACK, L2><<<gr, blk, 0, s>>>(p); break;
    case 2: attn_direct_kernel<2, FC, FS, PACK, L2><<<gr, blk, 0, s>>>(p); break;
    case 4: attn_direct_kernel<4, FC, FS, PACK, L2><<<gr, blk, 0, s>>>(p); break;
    case 8: attn_direct_kernel<8, FC, FS, PACK, L2><<<gr, dim3(PACK ? 64 * PACK : 512), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int PACK, bool L2>
static hipError_t launch_direct_fmt(const AttnParams& p, int group, bool fp8_cross, bool fp8_self,
                                    dim3 gr, hipStream_t s) {
  if (fp8_cross && fp8_self) return launch_direct<true, true, PACK, L2>(p, group, gr, s);
  if (fp8_cross) return launch_direct<true, false, PACK, L2>(p, group, gr, s);
  if (fp8_self) return launch_direct<false, true, PACK, L2>(p, group, gr, s);
  return launch_direct<false, false, PACK, L2>(p, group, gr, s);
}

template <bool L2>
static hipError_t launch_direct_pack(const AttnParams& p, int group, bool fp8_cross, bool fp8_self, int pack,
                                     dim3 gr, hipStream_t s) {
  switch (pack) {
    case 0: return launch_direct_fmt<0, L2>(p, group, fp8_cross, fp8_self, gr, s);
    case 1: return launch_direct_fmt<1, L2>(p, group, fp8_cross, fp8_self, gr, s);
    case 2: return launch_direct_fmt<2, L2>(p, group, fp8_cross, fp8_self, gr, s);
    case 4: return launch_direct_fmt<4, L2>(p, group, fp8_cross, fp8_self, gr, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bf16(const AttnParams& p, int group, bool fp8_cross, bool fp8_self, int pack,
                            hipStream_t s) {
  if (p.n_tiles == 0) return hipSuccess;
  const int64_t total = (int64_t)p.n_tiles * p.hkv;
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 gr((unsigned)grid);
  const bool direct = attn_direct_ok(fp8_cross, fp8_self, p.k_scale, p.v_scale);
  if (pack && !direct) return hipErrorInvalidValue;      // packed tiles need the direct kernel
  if (direct) {
    if (p.two_level) return launch_direct_pack<true>(p, group, fp8_cross, fp8_self, pack, gr, s);
    return launch_direct_pack<false>(p, group, fp8_cross, fp8_self, pack, gr, s);
  }
  switch (group) {
    case 1: attn_bf16_kernel<1><<<gr, dim3(256), 0, s>>>(p); break;
    case 2: attn_bf16_kernel<2><<<gr, dim3(256), 0, s>>>(p); break;
    case 4: attn_bf16_kernel<4><<<gr, dim3(256), 0, s>>>(p); break;
    case 8: attn_bf16_kernel<8><<<gr, dim3(512), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// fp32 path: one wave per (token, head); explicit partials + LSE merge.
// ----------------------------------------------------------------------------
struct Partial {
  float m, l;
  float acc[2];
};

__device__ __forceinline__ void partial_scan(const float* kp, const float* vp, int64_t tstride,
                                             int k0, int k1, const float (&q)[2], int nd,
                                             float scale, int lane, Partial& st) {
  st.m = -INFINITY;
  st.l = 0.0f;
  st.acc[0] = st.acc[1] = 0.0f;
  for (int j = k0; j < k1; ++j) {
    const float* kr = kp + (int64_t)j * tstride;
    float part = 0.0f;
    for (int e = 0; e < nd; ++e) part += q[e] * kr[lane + 64 * e];
    const float sc = wave_sum(part) * scale;
    const float mn = fmaxf(st.m, sc);
    const float a = expf(st.m - mn);
    const float pj = expf(sc - mn);
    st.l = st.l * a + pj;
    const float* vr = vp + (int64_t)j * tstride;
    for (int e = 0; e < nd; ++e) st.acc[e] = st.acc[e] * a + pj * vr[lane + 64 * e];
    st.m = mn;
  }
}

__global__ void __launch_bounds__(256) attn_f32_kernel(AttnF32Params p) {
  const int wave = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (wave >= p.n_tok * p.hq) return;
  const int t = wave / p.hq;
  const int h = wave % p.hq;
  const int g = h / (p.hq / p.hkv);
  const int nd = p.d / 64;
  float q[2] = {0.0f, 0.0f};
  for (int e = 0; e < nd; ++e) q[e] = p.q[((int64_t)t * p.hq + h) * p.d + lane + 64 * e];
  const int64_t kvs = (int64_t)p.hkv * p.d;

  Partial cr, sf;
  const int a = p.tok_anchor[t];
  if (a >= 0) {
    partial_scan(p.ak + (int64_t)g * p.d, p.av + (int64_t)g * p.d, kvs, p.a_off[a],
                 p.a_off[a + 1], q, nd, p.scale, lane, cr);
  } else {
    cr.m = -INFINITY; cr.l = 0.0f; cr.acc[0] = cr.acc[1] = 0.0f;
  }
  partial_scan(p.k + (int64_t)g * p.d, p.v + (int64_t)g * p.d, kvs, p.tok_seg[t], t + 1, q, nd,
               p.scale, lane, sf);
  // partial results: O_i = acc_i / l_i, L_i = m_i + log l_i; merge by LSE
  const float Lc = cr.l > 0.0f ? cr.m + logf(cr.l) : -INFINITY;
  const float Ls = sf.l > 0.0f ? sf.m + logf(sf.l) : -INFINITY;
  const float mx = fmaxf(Lc, Ls);
  const float L = mx + logf(expf(Lc - mx) + expf(Ls - mx));
  const float wc = cr.l > 0.0f ? expf(Lc - L) : 0.0f;
  const float ws = sf.l > 0.0f ? expf(Ls - L) : 0.0f;
  for (int e = 0; e < nd; ++e) {
    const float oc = cr.l > 0.0f ? cr.acc[e] / cr.l : 0.0f;
    const float os = sf.l > 0.0f ? sf.acc[e] / sf.l : 0.0f;
    p.out[((int64_t)t * p.hq + h) * p.d + lane + 64 * e] = wc * oc + ws * os;
  }
  if (p.lse != nullptr && lane == 0) p.lse[(int64_t)t * p.hq + h] = L;
}

hipError_t launch_attn_f32(const AttnF32Params& p, hipStream_t s) {
  const int64_t waves = (int64_t)p.n_tok * p.hq;
  if (waves == 0) return hipSuccess;
  attn_f32_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace quail
