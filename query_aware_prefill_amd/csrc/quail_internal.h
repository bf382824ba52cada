// Internal declarations shared by the HIP kernels and the host runtime.
// Nothing here is part of the public C ABI (include/quail.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quail {

constexpr int kHeadDim = 128;   // head_dim of the MFMA attention and QKV epilogue
constexpr int kKeyTile = 64;    // keys per attention tile; slab rows are padded to this
constexpr int kQRows = 32;      // query tokens per wave in the attention kernel

// A key/value source for attention. Element (token t, kv head g, dim c) of K
// lives at k + t*tok_stride + g*head_stride + c; likewise V.
struct KVSrc {
  const void* k;
  const void* v;
  int64_t tok_stride;     // elements
  int64_t head_stride;    // elements
  int32_t len;            // valid tokens (rows >= len read as zero)
  int32_t fp8;            // 1: OCP E4M3 codes (decoded, times k_scale / v_scale)
};

// One attention work item: query tokens [q0, q0+nq) against
//   - every key of source `cross` (no mask), then
//   - every key of source `cross2` (no mask; the shared-prefix level of a
//     two-level cascade: anchor -> shared suffix prefix -> suffix), then
//   - keys [self_k0, self_qbase + row] of source `self` (causal), where row is
//     the query's offset from q0, and keys below seg_lo[q0 + row] are hidden.
// Any source may be -1 (absent); cross2 only together with cross.
struct AttnTile {
  int32_t q0, nq;
  int32_t cross;
  int32_t self;
  int32_t self_qbase;
  int32_t self_k0;
  int32_t cross2;
};

struct AttnParams {
  const AttnTile* tiles;
  int32_t n_tiles;
  const KVSrc* srcs;
  const int32_t* seg_lo;    // [tokens] first visible self key of each query token
  const uint16_t* q;        // bf16 [tokens][q_stride], head h at h*128
  int64_t q_stride;
  uint16_t* out;            // bf16 [tokens][o_stride]
  int64_t o_stride;
  float* lse;               // f32 [tokens][hq] or null
  int32_t hq, hkv;
  float scale_log2;         // softmax scale * log2(e)
  float k_scale, v_scale;   // fp8 dequantisation scales
  int32_t two_level;        // some tile has a cross2 source (selects that kernel variant)
};

// fp32 reference-precision cascade (small head dims, explicit two partials + merge)
struct AttnF32Params {
  const float* ak; const float* av;      // [sum La][hkv][d]
  const int32_t* a_off;                  // [n_anchors+1] (device)
  const float* q; const float* k; const float* v;   // [sum Ls][h][d]
  const int32_t* tok_anchor;             // [tokens] anchor index or -1
  const int32_t* tok_seg;                // [tokens] first token of the token's suffix
  float* out; float* lse;
  int32_t n_tok, hq, hkv, d;
  float scale;
};

enum GemmEpi : int32_t {
  EPI_STORE = 0,    // y = bf16(acc * scale)
  EPI_RESID = 1,    // y = y + acc * scale, y fp32         (residual add in place)
  EPI_SWIGLU = 2,   // y[n] = bf16(silu(g) * u), g from row n, u from row n + inter
  EPI_QKV = 3,      // RoPE on q/k heads, q -> q_out, k/v -> suffix buffers or slabs
};

struct GemmParams {
  const uint16_t* A; int64_t lda;        // bf16 [M][K]
  const uint8_t* A8;                     // W8A8 (instead of A): E4M3 codes [M][K], row stride lda bytes
  const float* a_scale;                  // W8A8: one scale per row of A8
  const int32_t* a_map;                  // optional: A row m is row a_map[m] of A
  const int32_t* y_map;                  // optional (RESID): output row m adds into Yf row y_map[m]
  const uint8_t* B;                      // fp8 [N_rows][K]
  const uint16_t* scale;                 // bf16 [N_rows]
  int32_t M, N, K;                       // N = output columns
  uint16_t* Y; int64_t ldy;              // STORE / SWIGLU output (bf16)
  float* Yf;                             // RESID: fp32 residual rows (stride ldy)
  int32_t inter;                         // SWIGLU: up rows start at `inter`
  // QKV epilogue
  int32_t hq, hkv;
  const float2* rope;                    // [max_pos][64] (cos, sin)
  const int32_t* pos;                    // [M] RoPE position of each row
  uint16_t* q_out;                       // [M][hq*128]
  int32_t kv_mode;                       // 0: suffix buffers, 1: anchor slabs
  uint16_t* k_out; uint16_t* v_out;      // kv_mode 0: [M][hkv][128]
  void* pool;                            // kv_mode 1: slab pool base
  const int64_t* kv_row;                 // kv_mode 1: [M] element offset of (slab, token)
  const int32_t* kv_lapad;               // kv_mode 1: [M] padded anchor length
  int32_t layer;
  int32_t kv_fp8;                        // slabs hold E4M3 codes
  float k_inv_scale, v_inv_scale;
};

struct NormParams {
  const float* x; int64_t ldx;           // fp32 residual rows
  const uint16_t* gamma;                 // bf16 [H] (null: gain 1)
  uint16_t* y; int64_t ldy;
  uint8_t* yq; float* ys;                // optional (instead of y): per-token E4M3 codes [rows][H] and scales
  const int32_t* row_map;                // optional: y row r reads x row row_map[r]
  int32_t rows, H;
  float eps;
};

struct Head8Params {
  const uint16_t* h; int64_t ldh;        // bf16 rows
  const int32_t* row_map;                // optional: row r reads h row row_map[r]
  const uint16_t* gamma;                 // final norm (bf16 [H]) or null
  const uint16_t* w8;                    // bf16 [H][8]
  const int32_t* out_map;                // optional: output slot of row r
  float* logits; uint8_t* token; uint8_t* decision;
  int32_t rows, H;
  float eps;
  uint32_t true_mask;
};

// ---- launchers (return the launch's hipError_t) ----
// fp8_cross / fp8_self: the cross (anchor) / self key sources of this launch
// hold E4M3 codes. With unit k/v scales every combination runs the direct
// HBM->LDS kernel; other scales take the register-staged kernel.
// pack > 0: packed tiles of attn_tile_tokens(group, pack) tokens, `pack`
// waves each of G heads x 32/G tokens in its 32 rows (attn_pack_waves picks
// it); requires the direct kernel. pack 0: unpacked tiles.
hipError_t launch_attn_bf16(const AttnParams& p, int group, bool fp8_cross, bool fp8_self, int pack,
                            hipStream_t s);
// whether a launch with these formats and scales runs the direct kernel
bool attn_direct_ok(bool fp8_cross, bool fp8_self, float k_scale, float v_scale);
// query tokens per attention tile (one workgroup) for GQA group size `group`
int attn_tile_tokens(int group, int pack);
// packed width (1, 2 or 4 waves; 0 = unpacked) for runs of at most max_run
// query tokens per anchor
int attn_pack_waves(int group, int max_run);
hipError_t launch_attn_f32(const AttnF32Params& p, hipStream_t s);
// A8 set: the W8A8 kernel (fp8 MFMA; N a multiple of 256, SWIGLU of 128, K of 128)
hipError_t launch_gemm(const GemmParams& p, GemmEpi epi, hipStream_t s);
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s);
// codes[m][k] = E4M3(x[m][k] * (448 / amax_m)), scale[m] = amax_m / 448 (x bf16
// [M][K], K a multiple of 8; a row of zeros: codes 0, scale 0)
hipError_t launch_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes, float* scale,
                                 hipStream_t s);
// h (fp32) = embedding rows; token ids outside [0, vocab) embed row 0 and are
// counted in *bad (nullable)
hipError_t launch_embed(const int32_t* tokens, const int32_t* tok_map, const uint16_t* embed,
                        float* h, int32_t rows, int32_t H, int32_t vocab, uint32_t* bad,
                        hipStream_t s);
// 256-byte guard regions at base + offs[i] (offs on the device): mode 1
// writes the guard pattern, mode 0 counts regions that differ from it in *bad
hipError_t launch_guard(uint8_t* base, const int64_t* offs, int32_t n, int32_t mode, uint32_t* bad,
                        hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, int32_t n, hipStream_t s);
// dst[dst_idx ? dst_idx[r] : r] = bf16(src[src_idx ? src_idx[r] : r]): fp32
// residual rows of H to bf16 rows
hipError_t launch_copy_rows(const float* src, int64_t lds, const int32_t* src_idx,
                            uint16_t* dst, int64_t ldd, const int32_t* dst_idx, int32_t rows,
                            int32_t H, hipStream_t s);
// rows 0..rows-1 of each of n_blocks slab blocks (src_block / dst_block bytes
// apart) into the same rows of another slab's blocks
hipError_t launch_copy_slab_rows(const uint8_t* src, int64_t src_block, uint8_t* dst, int64_t dst_block,
                                 int32_t rows, int32_t row_bytes, int32_t n_blocks, hipStream_t s);
hipError_t launch_head8(const Head8Params& p, hipStream_t s);
hipError_t launch_head8_f32(int32_t n, int32_t H, const float* x, const float* w8,
                            uint32_t true_mask, float* logits, uint8_t* token,
                            uint8_t* decision, hipStream_t s);
hipError_t launch_fp8_encode(int64_t n, const float* x, float inv_scale, uint8_t* out,
                             hipStream_t s);
hipError_t launch_fp8_decode(int64_t n, const uint8_t* codes, float scale, float* out,
                             hipStream_t s);

}  // namespace quail
